"""The seeded input generator: determinism, layout, and the distributions the
configurations promise (CPU only)."""

import numpy as np

import oracle
import synth


def test_deterministic_and_random_access():
    a = synth.make_layer(0)
    b = synth.make_layer(0)
    for f in ("router_w", "gate_q", "gate_s", "down_q", "down_b"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    full = synth.make_x(4, rows=slice(4090, 4102))
    assert np.array_equal(full[:6], synth.make_x(4, rows=slice(4090, 4096)))
    assert np.array_equal(full[6:], synth.make_x(4, rows=slice(4096, 4102)))
    assert not np.array_equal(synth.make_x(1, layer=0), synth.make_x(1, layer=1))


def test_shapes_and_symmetric_bias():
    L = synth.make_layer(0)
    E, H, I = 16, 256, 128
    assert L.router_w.shape == (E, H) and L.router_w.dtype == np.float32
    assert L.gate_q.shape == (E + 1, I, H // 8) and L.gate_s.shape == (E + 1, I, H // 64)
    assert L.down_q.shape == (E + 1, H, I // 8) and L.down_s.shape == (E + 1, H, I // 64)
    for m in ("gate", "up", "down"):
        s = getattr(L, m + "_s").astype(np.float64)
        assert np.array_equal(getattr(L, m + "_b").astype(np.float64), -8 * s)
        assert s.min() >= 0.005 - 1e-5 and s.max() <= 0.02 + 1e-5
    L2 = synth.make_layer(2)
    assert L2.router_w.dtype == np.uint16 and L2.router_b is None
    assert L2.nbytes() == 455_802_880


def test_codes_uniform():
    L = synth.make_layer(0)
    sh = np.arange(8, dtype=np.uint32) * 4
    codes = ((L.gate_q[..., None] >> sh) & 0xF).ravel()
    hist = np.bincount(codes, minlength=16)
    assert hist.size == 16 and np.all(np.abs(hist / hist.mean() - 1) < 0.05)


def test_bf16_rounding_ties_to_even():
    vals = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(vals))
    assert list(got) == [1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7]


def test_uniform_and_zipf_expert_loads():
    L2 = synth.make_layer(2)
    x = synth.make_x(2)
    c2 = oracle.group(oracle.route(x, L2.router_w, None, 8)["ids"], 256)["counts"][:256]
    assert 60 <= c2.min() and c2.max() <= 220 and c2.mean() == 128
    L3 = synth.make_layer(3)
    assert np.array_equal(L3.gate_q, L2.gate_q) and L3.router_b is not None
    c3 = oracle.group(oracle.route(x, L3.router_w, L3.router_b, 8)["ids"], 256)["counts"][:256]
    assert c3.max() > 1000 and (c3 > 1000).sum() >= 5
    assert ((c3 >= 0) & (c3 <= 4)).sum() >= 100 and (c3 == 0).sum() >= 50
