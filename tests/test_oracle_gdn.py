"""Pins for the Gated DeltaNet scan oracle (CPU only).

The scan follows "Optimizing on-device inference for Apple Silicon", section
"Prefill > Keep recurrent state on chip", read as the gated delta rule
S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t.  Each
test below checks the oracle against something that is not its own loop: closed
forms of special cases, the retrieval property that defines the delta rule, and a
second algorithm (the blockwise form that the same section names as the ablation),
written here with a triangular solve and matrix products.
"""

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth
from synth import bf16_bits_to_f32, f32_to_bf16_bits


def _bits(a):
    bits = f32_to_bf16_bits(np.asarray(a, np.float32))
    assert np.array_equal(bf16_bits_to_f32(bits), np.asarray(a, np.float32)), "value must be exact in bf16"
    return bits


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def test_pure_decay_closed_form():
    """beta = 0 writes nothing: the state only decays, S_t = (prod alpha) S_0, and
    o_t = (prod_{tau<=t} alpha_tau) S_0 q_t."""
    g = synth.gdn_inputs(0, seed=3, nonzero_state=True)
    beta = np.zeros_like(g.beta)
    out, S = oracle.gdn_scan(g.q, g.k, g.v, g.alpha, beta, g.state)
    T, hv = g.alpha.shape
    group = hv // g.q.shape[1]
    cum = np.cumprod(g.alpha.astype(np.float64), axis=0)  # [T][hv]
    S0 = g.state.astype(np.float64)
    q = _f64(g.q)
    for h in range(hv):
        want_o = cum[:, h, None] * (q[:, h // group] @ S0[h].T)  # [T][dv]
        np.testing.assert_allclose(out[:, h], want_o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(S[h], cum[-1, h] * S0[h], rtol=1e-12, atol=1e-300)


def test_unit_key_retrieval():
    """With beta = 1 and a unit key, the update stores v_t at k_t exactly:
    S_t k_t = v_t whatever the decay and the earlier state, so q_t = k_t reads v_t back."""
    rng = np.random.default_rng(5)
    T, hk, hv, d = 24, 1, 2, 128
    k = np.zeros((T, hk, d), np.float32)
    for t in range(T):
        # unit keys exact in bf16: +-1 on one axis, or four entries of +-1/2
        if t % 2 == 0:
            k[t, 0, rng.integers(d)] = rng.choice([-1.0, 1.0])
        else:
            idx = rng.choice(d, 4, replace=False)
            k[t, 0, idx] = rng.choice([-0.5, 0.5], 4)
    kb = _bits(k)
    v = f32_to_bf16_bits(rng.standard_normal((T, hv, d)).astype(np.float32))
    alpha = rng.uniform(0.3, 1.0, (T, hv)).astype(np.float32)
    beta = np.ones((T, hv), np.float32)
    S0 = rng.standard_normal((hv, d, d)).astype(np.float32)
    out, _ = oracle.gdn_scan(kb, kb, v, alpha, beta, S0)
    np.testing.assert_allclose(out, _f64(v), rtol=0, atol=1e-12)


def test_decay_applies_before_the_write():
    """Two orthogonal unit keys e_a, e_b with beta = 1: writing v1 at e_a, then v2 at
    e_b with decay a2, leaves S e_a = a2 * v1 (old content decays) and S e_b = v2 (the
    new write does not)."""
    d, hv = 128, 1
    ea, eb = 3, 77
    k = np.zeros((2, 1, d), np.float32)
    k[0, 0, ea] = 1.0
    k[1, 0, eb] = 1.0
    q = np.zeros((2, 1, d), np.float32)
    q[0, 0, ea] = 1.0
    q[1, 0, ea] = 1.0
    rng = np.random.default_rng(9)
    v = f32_to_bf16_bits(rng.standard_normal((2, hv, d)).astype(np.float32))
    alpha = np.array([[0.75], [0.375]], np.float32)
    beta = np.ones((2, hv), np.float32)
    out, S = oracle.gdn_scan(_bits(q), _bits(k), v, alpha, beta)
    v64 = _f64(v)
    np.testing.assert_allclose(out[0, 0], v64[0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[1, 0], 0.375 * v64[0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(S[0][:, eb], v64[1, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(S[0][:, ea], 0.375 * v64[0, 0], rtol=0, atol=1e-15)
    others = np.delete(np.arange(d), [ea, eb])
    assert not S[0][:, others].any()


def test_constant_key_geometric_closed_form():
    """alpha = 1, one unit key u, constant beta = b and value v: along u the state moves
    geometrically towards v, S_t u = (1-b)^t S_0 u + (1 - (1-b)^t) v, and directions
    orthogonal to u keep S_0's content."""
    d, T, b = 128, 40, 0.25
    u = np.zeros(d, np.float32)
    u[[5, 9, 60, 100]] = [0.5, -0.5, 0.5, 0.5]
    w = np.zeros(d, np.float32)
    w[[5, 9]] = [0.5, 0.5]  # w . u = 0
    k = np.broadcast_to(u, (T, 1, d)).copy()
    q = k.copy()
    q[T - 1, 0] = w
    rng = np.random.default_rng(2)
    v1 = f32_to_bf16_bits(rng.standard_normal(d).astype(np.float32))
    v = np.broadcast_to(v1, (T, 1, d)).copy()
    S0 = rng.standard_normal((1, d, d)).astype(np.float32)
    out, S = oracle.gdn_scan(_bits(q), _bits(k), v, np.ones((T, 1), np.float32), np.full((T, 1), b, np.float32), S0)
    S0u = S0[0].astype(np.float64) @ u.astype(np.float64)
    vv = _f64(v1)
    for t in range(T - 1):
        r = (1 - b) ** (t + 1)
        np.testing.assert_allclose(out[t, 0], r * S0u + (1 - r) * vv, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out[T - 1, 0], S0[0].astype(np.float64) @ w.astype(np.float64), rtol=1e-12, atol=1e-12)


def blockwise_scan(q_bits, k_bits, v_bits, alpha, beta, S0, chunk):
    """The blockwise form of the same recurrence: within a chunk with start state S and
    cumulative decays g_r, the written vectors D solve the unit lower-triangular system
    (I + L) D = diag(beta) (V - diag(g) K S^T), L[r][s] = beta_r (g_r/g_s) k_r.k_s (s<r);
    then O = diag(g) Q S^T + (M o Q K^T) D with M[r][s] = g_r/g_s (s<=r), and the end
    state is g_last S + D^T diag(g_last/g) K."""
    q, k, v = _f64(q_bits), _f64(k_bits), _f64(v_bits)
    T, hk, d = k.shape
    hv = v.shape[1]
    grp = hv // hk
    out = np.zeros((T, hv, v.shape[2]))
    S = S0.astype(np.float64).copy()
    for h in range(hv):
        Sh = S[h]
        for c0 in range(0, T, chunk):
            c1 = min(T, c0 + chunk)
            K = k[c0:c1, h // grp]
            Q = q[c0:c1, h // grp]
            V = v[c0:c1, h]
            bt = beta[c0:c1, h].astype(np.float64)
            g = np.cumprod(alpha[c0:c1, h].astype(np.float64))
            ratio = g[:, None] / g[None, :]
            n = c1 - c0
            L = np.tril(bt[:, None] * ratio * (K @ K.T), -1)
            rhs = bt[:, None] * (V - g[:, None] * (K @ Sh.T))
            D = scipy.linalg.solve_triangular(np.eye(n) + L, rhs, lower=True, unit_diagonal=True)
            M = np.tril(ratio)
            out[c0:c1, h] = g[:, None] * (Q @ Sh.T) + (M * (Q @ K.T)) @ D
            Sh = g[-1] * Sh + D.T @ ((g[-1] / g)[:, None] * K)
        S[h] = Sh
    return out, S


@pytest.mark.parametrize("cfg,chunk", [(0, 8), (3, 16)])
def test_matches_blockwise_form(cfg, chunk):
    g = synth.gdn_inputs(cfg, seed=11, nonzero_state=True)
    out, S = oracle.gdn_scan(g.q, g.k, g.v, g.alpha, g.beta, g.state)
    want_o, want_S = blockwise_scan(g.q, g.k, g.v, g.alpha, g.beta, g.state, chunk)
    np.testing.assert_allclose(out, want_o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S, want_S, rtol=1e-10, atol=1e-12)


def test_key_head_sharing():
    """Consecutive value heads share a key head: with 2 key heads and 4 value heads,
    value heads 0 and 1 read key head 0.  Checked against runs with one key head per
    value head, the key head copied."""
    g = synth.gdn_inputs(0, seed=4, nonzero_state=True)
    out, S = oracle.gdn_scan(g.q, g.k, g.v, g.alpha, g.beta, g.state)
    hk = g.q.shape[1]
    grp = g.v.shape[1] // hk
    q_rep = np.repeat(g.q, grp, axis=1)
    k_rep = np.repeat(g.k, grp, axis=1)
    out2, S2 = oracle.gdn_scan(q_rep, k_rep, g.v, g.alpha, g.beta, g.state)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(S, S2)
    # a different key head gives a different result (the mapping matters)
    k_swapped = g.k[:, ::-1].copy()
    out3, _ = oracle.gdn_scan(g.q, k_swapped, g.v, g.alpha, g.beta, g.state)
    assert not np.allclose(out3, out)


def test_state_carries_across_chunks():
    """A prompt scanned in two chunks, the state handed from one to the next, gives the
    same outputs and end state as one scan (section "Prefill > Bound temporary memory
    with prompt chunking": the recurrent state carries context between chunks)."""
    g = synth.gdn_inputs(0, seed=6, nonzero_state=True)
    out, S = oracle.gdn_scan(g.q, g.k, g.v, g.alpha, g.beta, g.state)
    c = 15
    o1, S1 = oracle.gdn_scan(g.q[:c], g.k[:c], g.v[:c], g.alpha[:c], g.beta[:c], g.state)
    o2, S2 = oracle.gdn_scan(g.q[c:], g.k[c:], g.v[c:], g.alpha[c:], g.beta[c:], S1)
    np.testing.assert_array_equal(np.concatenate([o1, o2]), out)
    np.testing.assert_array_equal(S2, S)


def test_empty_prompt_keeps_state():
    g = synth.gdn_inputs(0, seed=1, nonzero_state=True)
    out, S = oracle.gdn_scan(g.q[:0], g.k[:0], g.v[:0], g.alpha[:0], g.beta[:0], g.state)
    assert out.shape == (0,) + g.v.shape[1:]
    np.testing.assert_array_equal(S, g.state.astype(np.float64))
