"""Pins for the CPU oracle: each test checks it against something other than itself
(library routines, brute force, closed forms, invariants, the pages' own figures).

CPU only.  Page citations name "Optimizing on-device inference for Apple Silicon"
and the section the fact comes from.
"""

import itertools
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers (test side)

def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack codes [N][K] (0..15) into words, low nibble = lowest k (the documented layout)."""
    N, K = codes.shape
    c = codes.astype(np.uint32).reshape(N, K // 8, 8)
    out = np.zeros((N, K // 8), np.uint32)
    for i in range(8):
        out |= c[:, :, i] << np.uint32(4 * i)
    return out


def unpack_codes_numpy(words: np.ndarray) -> np.ndarray:
    N, W = words.shape
    sh = np.arange(8, dtype=np.uint32) * 4
    return ((words[:, :, None] >> sh) & 0xF).reshape(N, W * 8).astype(np.float64)


def bf16(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def tiny_layer(E=4, H=64, I=64, k=1, seed=5, router_fp32=False):
    """A small random layer with the generator's distributions, built in the test."""
    rng = np.random.default_rng(seed)
    def qm(N, K):
        q = rng.integers(0, 1 << 32, size=(E + 1, N, K // 8), dtype=np.uint32)
        s = rng.uniform(0.005, 0.02, size=(E + 1, N, K // 64)).astype(np.float16)
        b = (s.astype(np.float32) * -8).astype(np.float16)
        return q, s, b
    w = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    rw = w if router_fp32 else bf16(w)
    g, u, d = qm(I, H), qm(I, H), qm(H, I)
    return synth.LayerWeights(rw, None, *g, *u, *d)


# ---------------------------------------------------------------- number decoding

def test_fp16_decoder_matches_numpy_on_every_pattern(oracle_lib):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_double(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decoder_matches_bit_shift():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=4000).astype(np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_double(b) for b in bits])
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


# ---------------------------------------------------------------- dequantisation
# Format: "Prefill > Dequantize weights during matmul" (4-bit code, scale and bias per 64).

def test_dequant_unpacks_documented_nibble_order():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 16, size=(5, 256))
    one = np.ones((5, 4), np.float16)
    zero = np.zeros((5, 4), np.float16)
    w = oracle.dequant(pack_codes(codes), one, zero)
    assert np.array_equal(w, codes.astype(np.float64))


def test_dequant_group_index_and_scale_bias():
    N, K = 3, 256
    s = (2.0 ** -np.arange(N * 4).reshape(N, 4)).astype(np.float16)
    b = np.full((N, 4), -0.25, np.float16)
    w = oracle.dequant(pack_codes(np.ones((N, K), int)), s, b)
    # code 1 everywhere: w[n][k] = s[n][k // 64] + b[n][k // 64]
    assert np.array_equal(w, np.repeat(s.astype(np.float64) - 0.25, 64, axis=1))


def test_dequant_symmetric_code8_is_zero():
    rng = np.random.default_rng(3)
    s = rng.uniform(0.005, 0.02, size=(4, 2)).astype(np.float16)
    b = (s.astype(np.float32) * -8).astype(np.float16)
    assert np.array_equal(b.astype(np.float64), -8 * s.astype(np.float64))  # exact in fp16
    w = oracle.dequant(pack_codes(np.full((4, 128), 8)), s, b)
    assert not np.any(w)


def test_dequant_random_against_numpy_unpack():
    L = synth.make_layer(0)
    q, s, b = L.down_q[3], L.down_s[3], L.down_b[3]
    w = oracle.dequant(q, s, b)
    ref = unpack_codes_numpy(q) * np.repeat(s.astype(np.float64), 64, 1) + np.repeat(b.astype(np.float64), 64, 1)
    assert np.array_equal(w, ref)


def test_dequant_bf16_scale_bias_closed_form():
    # the pages' checkpoint stores scale and bias as bf16 ("Prefill > Dequantize weights
    # during matmul"): with constant codes c, w = s c + b with s, b decoded by a bit shift
    rng = np.random.default_rng(21)
    N, K = 6, 192
    s = bf16(rng.uniform(0.005, 0.02, size=(N, K // 64)))
    b = bf16(rng.uniform(-0.2, 0.0, size=(N, K // 64)))
    sd = synth.bf16_bits_to_f32(s).astype(np.float64)
    bd = synth.bf16_bits_to_f32(b).astype(np.float64)
    for c in (0, 1, 7, 15):
        w = oracle.dequant(pack_codes(np.full((N, K), c)), s, b)
        assert np.array_equal(w, np.repeat(sd * c + bd, 64, axis=1)), c


def test_dequant_bf16_and_fp16_agree_where_both_formats_hold_the_values():
    # powers of two and small multiples are exact in both formats: the same weights
    rng = np.random.default_rng(22)
    N, K = 4, 128
    sv = 2.0 ** rng.integers(-9, -4, size=(N, K // 64)).astype(np.float64)
    bv = -8 * sv
    q = pack_codes(rng.integers(0, 16, size=(N, K)))
    w16 = oracle.dequant(q, sv.astype(np.float16), bv.astype(np.float16))
    wbf = oracle.dequant(q, bf16(sv), bf16(bv))
    assert np.array_equal(w16, wbf)


# ---------------------------------------------------------------- router

def test_logits_match_numpy_matmul_fp32_router():
    L = synth.make_layer(0)
    x = synth.make_x(0)
    r = oracle.route(x, L.router_w, None, 2)
    ref = synth.bf16_bits_to_f32(x).astype(np.float64) @ L.router_w.astype(np.float64).T
    assert np.allclose(r["logits"], ref, rtol=0, atol=1e-13)


def test_logits_match_numpy_matmul_bf16_router_with_bias():
    L = synth.make_layer(3)
    x = synth.make_x(3, rows=slice(0, 64))
    r = oracle.route(x, L.router_w, L.router_b, 8)
    ref = synth.bf16_bits_to_f32(x).astype(np.float64) @ synth.bf16_bits_to_f32(L.router_w).astype(np.float64).T
    ref = ref + L.router_b.astype(np.float64)
    assert np.allclose(r["logits"], ref, rtol=0, atol=1e-12)


def brute_force_topk(l, k):
    """Max-sum k-subset; among equal sums the lexicographically smallest index tuple."""
    best = None
    for sub in itertools.combinations(range(len(l)), k):
        key = (-sum(l[list(sub)]), sub)
        if best is None or key < best:
            best = key
    return np.array(best[1])


def test_topk_brute_force_all_subsets_tiny_config():
    L = synth.make_layer(0)
    x = synth.make_x(0)
    r = oracle.route(x, L.router_w, None, 2)
    for t in range(x.shape[0]):
        assert np.array_equal(r["ids"][t], brute_force_topk(r["logits"][t], 2))
        srt = sorted(range(16), key=lambda e: (-r["logits"][t][e], e))[:2]
        assert list(r["ranked"][t]) == srt


@pytest.mark.parametrize("k", [1, 3, 5])
def test_topk_brute_force_with_exact_ties(k):
    # duplicated router rows give bitwise-equal logits: the lower index must win
    L = tiny_layer(E=8, H=64)
    rw = L.router_w.copy()
    rw[5] = rw[2]
    rw[6] = rw[2]
    rw[7] = rw[1]
    x = bf16(np.random.default_rng(7).standard_normal((40, 64)))
    r = oracle.route(x, rw, None, k)
    ties = 0
    for t in range(40):
        l = r["logits"][t]
        assert l[5] == l[2] and l[6] == l[2] and l[7] == l[1]
        assert np.array_equal(r["ids"][t], brute_force_topk(l, k))
        ties += (2 in r["ids"][t]) != (5 in r["ids"][t])
    assert ties > 0  # the tie-break decided at least one boundary


def test_topk_bias_dominance():
    L = tiny_layer(E=12, H=64)
    b = np.zeros(12, np.float32)
    b[:4] = 100.0
    x = bf16(np.random.default_rng(8).standard_normal((10, 64)))
    r = oracle.route(x, L.router_w, b, 4)
    assert np.array_equal(r["ids"], np.tile(np.arange(4), (10, 1)))


def test_k_equals_E_gives_full_softmax():
    L = tiny_layer(E=6, H=128)
    x = bf16(np.random.default_rng(9).standard_normal((7, 128)))
    r = oracle.route(x, L.router_w, None, 6)
    assert np.array_equal(r["ids"], np.tile(np.arange(6), (7, 1)))
    assert np.allclose(r["gates"], scipy.special.softmax(r["logits"], axis=1), rtol=1e-14, atol=0)


def test_gates_closed_form_k2_and_invariants():
    L = synth.make_layer(0)
    x = synth.make_x(0)
    r = oracle.route(x, L.router_w, None, 2)
    for t in range(8):
        a, b = r["ids"][t]
        la, lb = r["logits"][t][a], r["logits"][t][b]
        assert abs(r["gates"][t][0] - scipy.special.expit(la - lb)) < 1e-15
    L2 = synth.make_layer(2)
    x2 = synth.make_x(2, rows=slice(0, 32))
    r2 = oracle.route(x2, L2.router_w, None, 8)
    g = r2["gates"]
    assert np.all(g > 0) and np.allclose(g.sum(1), 1.0, rtol=0, atol=1e-15)
    for t in range(32):
        l = r2["logits"][t][r2["ids"][t]]
        order = np.argsort(l)
        assert np.all(np.diff(g[t][order]) >= 0)  # gate monotone in logit
        assert np.all(np.diff(r2["ids"][t]) > 0)  # ascending, distinct


# ---------------------------------------------------------------- grouping
# "Prefill > Keep expert routing on the GPU": histogram, prefix scan, scatter.

def brute_force_group(ids, E):
    T, k = ids.shape
    groups = {e: [] for e in range(E + 1)}
    for t in range(T):
        for e in ids[t]:
            groups[int(e)].append(t)
        groups[E].append(t)
    counts = np.array([len(groups[e]) for e in range(E + 1)])
    row_token = np.array([t for e in range(E + 1) for t in groups[e]])
    return counts, row_token


def test_group_against_brute_force_and_invariants():
    L = synth.make_layer(2)
    x = synth.make_x(2, rows=slice(0, 300))
    r = oracle.route(x, L.router_w, None, 8)
    g = oracle.group(r["ids"], 256)
    counts, row_token = brute_force_group(r["ids"], 256)
    assert np.array_equal(g["counts"], counts)
    assert np.array_equal(g["row_token"], row_token)
    assert g["offsets"][0] == 0 and np.array_equal(np.diff(g["offsets"]), g["counts"])
    assert g["offsets"][-1] == 300 * 9 and g["counts"].sum() == 300 * 9 and g["counts"][256] == 300
    # slot map inverts the permutation; each token appears exactly k+1 times
    assert np.array_equal(np.sort(g["slot_row"].ravel()), np.arange(300 * 9))
    assert np.array_equal(g["row_token"][g["slot_row"]], np.repeat(np.arange(300)[:, None], 9, 1))
    assert np.array_equal(np.bincount(g["row_token"], minlength=300), np.full(300, 9))
    for e in range(257):
        seg = g["row_token"][g["offsets"][e]:g["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)  # ascending tokens, at most once per expert


def test_pages_routing_arithmetic_2k_tokens():
    fact = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))["routing_assignments"]
    L = synth.make_layer(2)
    x = synth.make_x(2, rows=slice(0, fact["tokens"]))
    r = oracle.route(x, L.router_w, None, fact["top_k"])
    g = oracle.group(r["ids"], fact["experts"])
    assert g["counts"][:fact["experts"]].sum() == fact["assignments"]
    assert g["counts"][:fact["experts"]].mean() == fact["mean_rows_per_expert"]
    assert g["counts"][:fact["experts"]].std() > 0  # uneven in practice


def test_pages_checkpoint_bits_per_weight():
    f = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))["checkpoint_size"]
    L = synth.make_layer(0)
    n_w = sum(getattr(L, m + "_q").size * 8 for m in ("gate", "up", "down"))
    n_b = sum(getattr(L, m + s).nbytes for m in ("gate", "up", "down") for s in ("_q", "_s", "_b"))
    bits = 8 * n_b / n_w
    assert bits == f["code_bits"] + (f["scale_bits"] + f["bias_bits"]) / f["group"]  # 4.5
    # 70 GB of bf16 is 35e9 weights; at 4.5 bits they take 19.7 GB, within 2% of the page's 19.4
    n_params = f["bf16_gb"] * 1e9 / 2
    assert abs(n_params * bits / 8 / 1e9 - f["q4_gb"]) / f["q4_gb"] < 0.02


# ---------------------------------------------------------------- experts and combine

def dense_reference(x_bits, L, ids, gates):
    """Dense-dequantised MoE: every expert on every token, masked by a dense gate matrix."""
    x = synth.bf16_bits_to_f32(x_bits).astype(np.float64)
    T = x.shape[0]
    E = L.gate_q.shape[0] - 1
    G = np.zeros((T, E + 1))
    for t in range(T):
        G[t, ids[t]] = gates[t]
    G[:, E] = 1.0

    def deq(q, s, b):
        return unpack_codes_numpy(q) * np.repeat(s.astype(np.float64), 64, 1) + np.repeat(b.astype(np.float64), 64, 1)

    out = np.zeros_like(x)
    for e in range(E + 1):
        Wg, Wu, Wd = deq(L.gate_q[e], L.gate_s[e], L.gate_b[e]), deq(L.up_q[e], L.up_s[e], L.up_b[e]), deq(L.down_q[e], L.down_s[e], L.down_b[e])
        a, u = x @ Wg.T, x @ Wu.T
        y = (a * scipy.special.expit(a) * u) @ Wd.T
        out += G[:, e:e + 1] * y
    return out


def test_experts_match_dense_reference_tiny_config():
    L = synth.make_layer(0)
    x = synth.make_x(0)
    r = oracle.forward(x, L, 2)
    ref = dense_reference(x, L, r["ids"], r["gates"])
    assert np.max(np.abs(r["out"] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_experts_match_dense_reference_all_experts_chosen():
    L = tiny_layer(E=3, H=64, I=128)
    x = bf16(np.random.default_rng(4).standard_normal((5, 64)))
    r = oracle.forward(x, L, 3)
    ref = dense_reference(x, L, r["ids"], r["gates"])
    assert np.max(np.abs(r["out"] - ref)) <= 1e-12 * np.max(np.abs(ref))


def _const_matrix(E1, N, K, code, s):
    q = np.tile(pack_codes(np.full((N, K), code)), (E1, 1, 1))
    sc = np.full((E1, N, K // 64), s, np.float16)
    return q, sc, np.zeros_like(sc)


def test_experts_closed_form_constant_weights():
    # every weight of every expert constant: gate alpha, up beta, down delta.  A one-hot
    # token x = v*e_h0 gives a = alpha*v, u = beta*v, h_i = silu(a)*u for all i, and every
    # output = I*delta*h per expert; the gates sum to 1 and the shared expert adds one more.
    E, H, I = 4, 128, 64
    gq, gs, gb = _const_matrix(E + 1, I, H, 3, 0.25)   # alpha = 0.75
    uq, us, ub = _const_matrix(E + 1, I, H, 5, 0.125)  # beta = 0.625
    dq, ds, db = _const_matrix(E + 1, H, I, 2, 0.5)    # delta = 1.0
    rw = bf16(np.random.default_rng(0).standard_normal((E, H)) * 0.02)
    L = synth.LayerWeights(rw, None, gq, gs, gb, uq, us, ub, dq, ds, db)
    x = np.zeros((3, H), np.uint16)
    vals = [1.5, -2.0, 0.375]
    for t, v in enumerate(vals):
        x[t, 7 + t] = bf16([v])[0]
    r = oracle.forward(x, L, 2)
    for t, v in enumerate(vals):
        a, u = 0.75 * v, 0.625 * v
        y = I * 1.0 * (a * scipy.special.expit(a) * u)
        assert np.allclose(r["out"][t], 2 * y, rtol=1e-14, atol=0)


def test_experts_zero_down_projection_gives_zero():
    L = synth.make_layer(0)
    s = L.down_s
    Lz = synth.LayerWeights(L.router_w, None, L.gate_q, L.gate_s, L.gate_b, L.up_q, L.up_s, L.up_b,
                            np.tile(pack_codes(np.full((256, 128), 8)), (17, 1, 1)), s,
                            (s.astype(np.float32) * -8).astype(np.float16))
    r = oracle.forward(synth.make_x(0), Lz, 2)
    assert not np.any(r["out"])


def test_experts_zero_gate_projection_gives_zero():
    L = synth.make_layer(0)
    s = L.gate_s
    Lz = synth.LayerWeights(L.router_w, None, np.tile(pack_codes(np.full((128, 256), 8)), (17, 1, 1)), s,
                            (s.astype(np.float32) * -8).astype(np.float16), L.up_q, L.up_s, L.up_b,
                            L.down_q, L.down_s, L.down_b)
    r = oracle.forward(synth.make_x(0), Lz, 2)
    assert not np.any(r["out"])


def test_down_scale_doubling_doubles_output_exactly():
    L = synth.make_layer(0)
    x = synth.make_x(0)
    r1 = oracle.forward(x, L, 2)
    L2 = synth.LayerWeights(L.router_w, None, L.gate_q, L.gate_s, L.gate_b, L.up_q, L.up_s, L.up_b,
                            L.down_q, (L.down_s * 2).astype(np.float16), (L.down_b * 2).astype(np.float16))
    r2 = oracle.forward(x, L2, 2)
    assert np.array_equal(r2["out"], 2 * r1["out"])


def test_single_expert_equals_twice_ffn_when_shared_is_the_same():
    L = tiny_layer(E=1, H=64, I=64)
    for nm in ("gate", "up", "down"):
        for sfx in ("_q", "_s", "_b"):
            a = getattr(L, nm + sfx)
            a[1] = a[0]
    x = bf16(np.random.default_rng(11).standard_normal((4, 64)))
    r = oracle.forward(x, L, 1)
    assert np.all(r["gates"] == 1.0)
    only_shared = oracle.experts(x, L, r["ids"], np.zeros_like(r["gates"]))
    assert np.array_equal(r["out"], 2 * only_shared)


def _zero_routed_down(L):
    """The layer with every routed expert's down projection zero (code 8, bias -8 s), the
    shared expert untouched."""
    E = L.down_q.shape[0] - 1
    dq, ds, db = L.down_q.copy(), L.down_s.copy(), L.down_b.copy()
    dq[:E] = 0x88888888
    if ds.dtype == np.uint16:  # bf16 bits
        db[:E] = bf16(synth.bf16_bits_to_f32(ds[:E]) * np.float32(-8))
    else:
        db[:E] = (ds[:E].astype(np.float32) * -8).astype(np.float16)
    return synth.LayerWeights(L.router_w, L.router_b, L.gate_q, L.gate_s, L.gate_b, L.up_q, L.up_s, L.up_b,
                              dq, ds, db, shared_gate=L.shared_gate)


def test_shared_gate_is_sigmoid_of_x_dot_w():
    # with the routed experts' outputs zero, out_t = sigmoid(x_t . w_sg) * FFN_shared(x_t):
    # the ratio to the ungated layer, per token, against numpy's dot and logistic
    sh = synth.shape_of(15)
    L = _zero_routed_down(synth.make_layer(15))
    x = synth.make_x(15)
    r = oracle.route(x, L.router_w, None, sh.k)
    gated = oracle.experts(x, L, r["ids"], r["gates"])
    L0 = synth.LayerWeights(*[getattr(L, f) for f in ("router_w", "router_b", "gate_q", "gate_s", "gate_b", "up_q",
                                                       "up_s", "up_b", "down_q", "down_s", "down_b")])
    plain = oracle.experts(x, L0, r["ids"], r["gates"])
    z = synth.bf16_bits_to_f32(x).astype(np.float64) @ synth.bf16_bits_to_f32(L.shared_gate).astype(np.float64)
    sig = scipy.special.expit(z)
    assert np.all((sig > 0.2) & (sig < 0.8))  # the gate is not saturated on these inputs
    np.testing.assert_allclose(gated, sig[:, None] * plain, rtol=1e-12, atol=1e-12 * np.max(np.abs(plain)))
    # a zero gate vector: sigmoid(0) = 1/2 exactly, so the output halves bitwise
    Lh = synth.LayerWeights(*[getattr(L0, f) for f in ("router_w", "router_b", "gate_q", "gate_s", "gate_b", "up_q",
                                                        "up_s", "up_b", "down_q", "down_s", "down_b")],
                            shared_gate=np.zeros(sh.H, np.uint16))
    assert np.array_equal(oracle.experts(x, Lh, r["ids"], r["gates"]), 0.5 * plain)


def test_bf16_qparam_layer_matches_dense_reference():
    # the whole layer with bf16 scale/bias and the shared gate against a dense numpy MoE
    L = synth.make_layer(15)
    x = synth.make_x(15)
    r = oracle.forward(x, L, 4)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    E = L.gate_q.shape[0] - 1

    def deq(q, s, b):
        sd = synth.bf16_bits_to_f32(s).astype(np.float64)
        bd = synth.bf16_bits_to_f32(b).astype(np.float64)
        return unpack_codes_numpy(q) * np.repeat(sd, 64, 1) + np.repeat(bd, 64, 1)

    G = np.zeros((x.shape[0], E + 1))
    for t in range(x.shape[0]):
        G[t, r["ids"][t]] = r["gates"][t]
    G[:, E] = scipy.special.expit(xf @ synth.bf16_bits_to_f32(L.shared_gate).astype(np.float64))
    ref = np.zeros_like(xf)
    for e in range(E + 1):
        a = xf @ deq(L.gate_q[e], L.gate_s[e], L.gate_b[e]).T
        u = xf @ deq(L.up_q[e], L.up_s[e], L.up_b[e]).T
        ref += G[:, e:e + 1] * ((a * scipy.special.expit(a) * u) @ deq(L.down_q[e], L.down_s[e], L.down_b[e]).T)
    assert np.max(np.abs(r["out"] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_token_permutation_equivariance_and_chunk_invariance():
    L = synth.make_layer(0)
    x = synth.make_x(0)
    r = oracle.forward(x, L, 2)
    perm = np.array([3, 0, 7, 1, 6, 2, 5, 4])
    rp = oracle.forward(x[perm], L, 2)
    assert np.array_equal(rp["out"], r["out"][perm])
    assert np.array_equal(rp["ids"], r["ids"][perm])
    a = oracle.forward(x[:5], L, 2)
    b = oracle.forward(x[5:], L, 2)
    assert np.array_equal(np.concatenate([a["out"], b["out"]]), r["out"])
