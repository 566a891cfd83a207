"""The C-ABI library on the CPU: it loads without a GPU, exports every function that
include/moe.h declares, and its host validation returns the documented statuses
before touching a device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    from sparse_moe_02_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return binding


def declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported(B):
    names = declared_functions()
    assert {"moe_plan_create", "moe_forward_prefill", "moe_forward_decode"} <= set(names)
    for n in names:
        assert hasattr(B.lib(), n), n
    assert set(B.EXPORTED) == set(names)


def test_status_strings(B):
    for code, name in B.STATUS_NAMES.items():
        s = B.moe_status_string(code)
        assert isinstance(s, str) and s
    assert B.moe_status_string(0) == "ok"
    assert "gfx950" in B.moe_version()


def _cfg(B, **kw):
    c = dict(hidden=2048, inter=512, n_experts=256, top_k=8, group_size=64, router_dtype=B.MOE_BF16,
             qparam_dtype=B.MOE_FP16, max_chunk_tokens=4096, flags=0)
    c.update(kw)
    return B.moe_config(**c)


def _weights(B, base=0x10000):
    w = B.moe_weights()
    w.router_w = base
    for i, m in enumerate(("gate", "up", "down", "s_gate", "s_up", "s_down")):
        p = base + 0x1000 * (i + 1)
        setattr(w, m, B.moe_qmat(p, p + 0x100, p + 0x200))
    return w


@pytest.mark.parametrize("kw,status", [
    (dict(group_size=32), 2), (dict(hidden=2000), 2), (dict(hidden=128), 2), (dict(inter=320), 2),
    (dict(inter=64), 2), (dict(n_experts=257), 2), (dict(n_experts=0), 2), (dict(top_k=0), 2),
    (dict(top_k=17, n_experts=32), 2), (dict(top_k=9, n_experts=8), 2), (dict(max_chunk_tokens=0), 2),
    (dict(flags=6), 2), (dict(flags=7), 2), (dict(flags=1 << 7), 2), (dict(flags=1 << 31), 2),
    (dict(router_dtype=1), 3), (dict(qparam_dtype=2), 3), (dict(qparam_dtype=7), 3),
])
def test_plan_rejects_bad_config(B, kw, status):
    with pytest.raises(B.MoeError) as ei:
        B.moe_plan_create(_cfg(B, **kw), _weights(B))
    assert ei.value.status == status


@pytest.mark.parametrize("kw", [
    dict(flags=1), dict(flags=5), dict(flags=16), dict(flags=64), dict(flags=5 | 16 | 64),
    dict(qparam_dtype=0),  # bf16 scale/bias (the pages' checkpoint format)
    # the largest accepted chunk with the largest intermediate size and top-k: a down GEMM
    # M-block's h rows lie up to 65536 x 17 x 4096 x 2 bytes (> 2^32) into the workspace
    dict(max_chunk_tokens=65536, top_k=16, inter=4096, n_experts=32),
    dict(max_chunk_tokens=65536, hidden=16384),
])
def test_plan_accepts_valid_flags_and_sizes(B, kw):
    # host validation passes; on a machine without a gfx950 the device query then fails
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(B.MoeError) as ei:
        B.moe_plan_create(_cfg(B, **kw), _weights(B))
    assert ei.value.status == 7


def test_flag_values_match_header(B):
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    for name in ("MOE_F_NO_FALLBACK", "MOE_F_SEPARATE_DEQUANT", "MOE_F_HOST_ROUTING"):
        m = re.search(r"#define " + name + r" \(1u << (\d+)\)", hdr)
        assert m and getattr(B, name) == 1 << int(m.group(1)), name
    assert re.search(r"#define MOE_F_FORCE_BM\(rows\) \(\(uint32_t\)\(\(rows\) / 32\) & 0xfu\)", hdr)
    assert [B.MOE_F_FORCE_BM(r) for r in (32, 64, 96, 128, 160)] == [1, 2, 3, 4, 5]
    assert re.search(r"MOE_ERR_WAIT = 11", hdr) and B.MOE_ERR_WAIT == 11


def test_plan_rejects_null_and_misaligned_weights(B):
    w = _weights(B)
    w.gate = B.moe_qmat(None, 0x2000, 0x3000)
    with pytest.raises(B.MoeError) as ei:
        B.moe_plan_create(_cfg(B), w)
    assert ei.value.status == 1
    w = _weights(B)
    w.router_w = None
    with pytest.raises(B.MoeError) as ei:
        B.moe_plan_create(_cfg(B), w)
    assert ei.value.status == 1
    w = _weights(B)
    w.down = B.moe_qmat(0x2004, 0x3000, 0x4000)
    with pytest.raises(B.MoeError) as ei:
        B.moe_plan_create(_cfg(B), w)
    assert ei.value.status == 4
    w = _weights(B)
    w.shared_gate = 0x9008  # the optional shared-expert gate vector must be 16-byte aligned
    with pytest.raises(B.MoeError) as ei:
        B.moe_plan_create(_cfg(B), w)
    assert ei.value.status == 4


def test_plan_needs_gfx950_device(B):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the device check passes there")
    with pytest.raises(B.MoeError) as ei:
        B.moe_plan_create(_cfg(B), _weights(B))
    assert ei.value.status == 7


def test_forwards_reject_null_plan(B):
    L = B.lib()
    assert L.moe_forward_prefill(None, 0x1000, 1, 0x2000, 0x3000, 1 << 20, None, None) == 1
    assert L.moe_forward_decode(None, 0x1000, 0x2000, 0x3000, 1 << 20, None, None) == 1
    assert L.moe_workspace_init(None, 0x3000, 1 << 20, None) == 1
    assert L.moe_workspace_check(None, 0x3000, 1 << 20, None) == 1


def test_pack_qparams_host_validation(B):
    # every case is rejected on the host, before anything is enqueued
    L = B.lib()
    assert L.moe_pack_qparams(None, 0x200000, 16, 64, None) == 1
    assert L.moe_pack_qparams(0x100000, None, 16, 64, None) == 1
    for rows, k in ((0, 64), (8, 64), (24, 64), (16, 0), (16, 32), (16, 96), (-16, 64)):
        assert L.moe_pack_qparams(0x100000, 0x200000, rows, k, None) == 2, (rows, k)
    assert L.moe_pack_qparams(0x100002, 0x200000, 16, 64, None) == 4
    assert L.moe_pack_qparams(0x100000, 0x200006, 16, 64, None) == 4
    # 32 rows x 2 groups = 128 bytes: destinations starting inside the source overlap it
    assert L.moe_pack_qparams(0x100000, 0x100040, 32, 128, None) == 9
    assert L.moe_pack_qparams(0x100040, 0x100000, 32, 128, None) == 9
    assert L.moe_pack_qparams(0x100000, 0x100000, 32, 128, None) == 9


def test_pack_codes_host_validation(B):
    L = B.lib()
    assert L.moe_pack_codes(None, 0x200000, 16, 128, None) == 1
    assert L.moe_pack_codes(0x100000, None, 16, 128, None) == 1
    for rows, k in ((0, 128), (8, 128), (24, 128), (16, 0), (16, 64), (16, 192), (-16, 128)):
        assert L.moe_pack_codes(0x100000, 0x200000, rows, k, None) == 2, (rows, k)
    assert L.moe_pack_codes(0x100008, 0x200000, 16, 128, None) == 4
    assert L.moe_pack_codes(0x100000, 0x200004, 16, 128, None) == 4
    # 16 rows x 16 words = 1 KiB
    assert L.moe_pack_codes(0x100000, 0x100200, 16, 128, None) == 9
    assert L.moe_pack_codes(0x100200, 0x100000, 16, 128, None) == 9


def test_product_path_fails_loudly_without_library(B, monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def test_product_package_does_not_import_oracle():
    pkg = os.path.join(ROOT, "sparse_moe_02_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", src), f"{f} mentions the oracle"
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c")):
            src = open(os.path.join(ROOT, "oracle", f)).read()
            assert "import sparse_moe_02_amd" not in src and "csrc" not in src


def test_gdn_scan_validation(B):
    """moe_gdn_scan's host checks return their statuses before touching a device; valid
    arguments reach the device check (no GPU here: MOE_ERR_DEVICE)."""
    L = B.lib()
    base = 0x100000
    q, k, v, al, be, st, out = (base + i * 0x10000000 for i in range(7))

    def call(T=8, hk=2, hv=4, dk=128, dv=128, **kw):
        a = dict(q=q, k=k, v=v, al=al, be=be, st=st, out=out)
        a.update(kw)
        return L.moe_gdn_scan(T, hk, hv, dk, dv, a["q"], a["k"], a["v"], a["al"], a["be"], a["st"], a["out"], None)

    assert call(T=-1) == B.MOE_ERR_TOKENS
    assert call(dk=64) == B.MOE_ERR_SHAPE
    assert call(dv=256) == B.MOE_ERR_SHAPE
    assert call(hk=3, hv=4) == B.MOE_ERR_SHAPE
    assert call(hk=0) == B.MOE_ERR_SHAPE
    assert call(hv=8192, hk=1) == B.MOE_ERR_SHAPE
    assert call(st=None) == B.MOE_ERR_NULL
    assert call(q=None) == B.MOE_ERR_NULL
    assert call(T=0, q=None, k=None, v=None, al=None, be=None, out=None) == B.MOE_ERR_DEVICE
    assert call(k=k + 8) == B.MOE_ERR_ALIGN
    assert call(st=st + 4) == B.MOE_ERR_ALIGN
    assert call(al=al + 2) == B.MOE_ERR_ALIGN
    assert call(out=out + 1) == B.MOE_ERR_ALIGN
    assert call(out=v) == B.MOE_ERR_ALIAS
    assert call(st=q) == B.MOE_ERR_ALIAS
    assert call(out=st) == B.MOE_ERR_ALIAS
    assert call() == B.MOE_ERR_DEVICE
