"""Shared helpers of the GPU parity tests: run the HIP library through its C ABI and
compare with the oracle (bit-exact routing, max-abs-rel outputs)."""

from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

TOL = 2e-2  # max|gpu - oracle| / max|oracle| over the output tensor
# Gates: softmax of the chosen fp32 logits (binary64 for re-ranked tokens).  A logit error
# d moves a gate by at most about g*(|d_e| + max_j |d_j|) plus a few ulp of exp and the
# division; the fp32 logits measure |d| <= 1.1e-6 against the exact ones (the worst of
# the 4K and 128K workloads), so gates stay within ~2.2e-6 + 1e-7.
GATE_TOL = 2e-6


def say(msg: str) -> None:
    print(msg, flush=True)


def ensure_lib():
    from sparse_moe_02_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return binding


def to_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


def token_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.max(np.abs(got - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    return float(np.max(num / den))


def run_prefill(layer_w, x_bits, k, chunk, device="cuda:0", flags=0, logits=False):
    import torch

    from sparse_moe_02_amd.layer import MoeLayer, bf16_bits, bf16_tensor

    layer = MoeLayer(layer_w, top_k=k, max_chunk_tokens=chunk, device=device, flags=flags)
    x = bf16_tensor(x_bits, device)
    out, d = layer.prefill(x, debug=True, logits=logits)
    torch.cuda.synchronize()
    res = {key: v.cpu().numpy() for key, v in d.items()}
    res["out"] = to_f64(bf16_bits(out))
    layer.close()
    return res


def check_routing_prefill(res, ref_ids, ref_gates, x_len, E, k, chunk, group_of_chunk):
    """ids bit-exact, gates close; per chunk counts/offsets/row_token bit-exact."""
    assert np.array_equal(res["topk_ids"], ref_ids), "top-k ids differ from the oracle"
    gerr = float(np.max(np.abs(res["gates"] - ref_gates)))
    assert gerr <= GATE_TOL, f"gates differ by {gerr}"
    nch = (x_len + chunk - 1) // chunk
    for c in range(nch):
        lo, hi = c * chunk, min(x_len, (c + 1) * chunk)
        g = group_of_chunk(lo, hi)
        n = (hi - lo) * (k + 1)
        assert np.array_equal(res["counts"][c], g["counts"]), f"counts differ in chunk {c}"
        assert np.array_equal(res["offsets"][c], g["offsets"]), f"offsets differ in chunk {c}"
        rt = res["row_token"][c * chunk * (k + 1): c * chunk * (k + 1) + n]
        assert np.array_equal(rt, g["row_token"]), f"row_token differs in chunk {c}"
    return gerr


def gateup_split(counts, T, H, I, E, k, chunk, n_cu):
    """The grouped GEMM's rule for splitting its last round of gate/up items along K, run
    on the host from one chunk's expert counts: returns (pieces per split item, split
    items).  An expert with n rows makes ceil(n / 160) M-blocks; items = M-blocks x
    ceil(I / 256); the last round is split when it fills at most half of the n_cu
    workgroups, into S = min(4, n_cu // items_in_round, K-steps, slots // items) pieces."""
    nmb = sum(-(-int(n) // 160) for n in counts if n)
    nb = -(-I // 256)
    nss = H // 128
    r = (nb * nmb) % n_cu
    if r == 0 or 2 * r > n_cu:
        return 1, 0
    ti = -(-r // nb) * nb
    mt_max = (min(160, chunk) + 31) // 32
    slot = mt_max * 32 * 2 * 256 // 2
    rows = chunk * (k + 1)
    part = min(4 * nb * (rows // 160 + E + 2), 256) * slot * 8
    max_pieces = max(rows * H * 2, part) // (slot * 8)
    s = min(4, n_cu // ti, nss, max_pieces // ti, 1024 // ti)
    return (s, ti) if s >= 2 else (1, 0)


def certificate_margin(l32, r32, l64):
    """max over (t, e) of |l32 - l64| / r32: the fp32 logits' error as a fraction of the
    radius the selection certifies them with (must stay <= 0.1, a 10x margin)."""
    err = np.abs(l32.astype(np.float64) - l64)
    return float(np.max(err / r32.astype(np.float64))), float(np.max(err)), float(np.min(r32))
