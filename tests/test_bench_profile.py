"""Host logic of the benchmark's HBM-traffic figure: the committed FETCH_SIZE/WRITE_SIZE
summary is used only while the kernel sources it was taken from are unchanged."""
import hashlib
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write_profile(path, root, srcs, sha, kernel, value):
    with open(path, "w") as f:
        f.write("# traffic\n\n    sources: " + " ".join(srcs) + "\n")
        f.write("    sources_sha256: " + sha + "\n")
        f.write(f"    traffic_bytes {kernel} {value}\n")


@pytest.fixture()
def tree(tmp_path):
    (tmp_path / "src").mkdir()
    (tmp_path / "src" / "a.hip").write_bytes(b"kernel a\n")
    (tmp_path / "src" / "b.hpp").write_bytes(b"header b\n")
    srcs = ["src/a.hip", "src/b.hpp"]
    h = hashlib.sha256()
    for s in srcs:
        h.update((tmp_path / s).read_bytes())
    return tmp_path, srcs, h.hexdigest()


def test_traffic_used_while_sources_unchanged(tree, monkeypatch):
    root, srcs, sha = tree
    b = _bench()
    prof = root / "prof.md"
    _write_profile(prof, root, srcs, sha, "k_gemm_gateup", 603785441)
    monkeypatch.setattr(b, "ROOT", str(root))
    monkeypatch.setattr(b, "TRAFFIC_PROFILE", str(prof))
    assert b.profiled_traffic("k_gemm_gateup") == 603785441.0
    assert b.profiled_traffic("k_decode1") is None  # not in the summary


def test_traffic_dropped_once_a_source_changes(tree, monkeypatch):
    root, srcs, sha = tree
    b = _bench()
    prof = root / "prof.md"
    _write_profile(prof, root, srcs, sha, "k_gemm_gateup", 603785441)
    (root / "src" / "b.hpp").write_bytes(b"header b, edited\n")
    monkeypatch.setattr(b, "ROOT", str(root))
    monkeypatch.setattr(b, "TRAFFIC_PROFILE", str(prof))
    assert b.profiled_traffic("k_gemm_gateup") is None


def test_missing_profile_gives_none(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "TRAFFIC_PROFILE", str(tmp_path / "absent.md"))
    assert b.profiled_traffic("k_gemm_gateup") is None


def test_committed_profile_names_existing_sources():
    b = _bench()
    text = open(b.TRAFFIC_PROFILE).read().split("\n")
    srcs = [l.split()[1:] for l in text if l.split()[:1] == ["sources:"]]
    assert srcs and srcs[0], "the summary lists the sources it was taken from"
    for s in srcs[0]:
        assert os.path.exists(os.path.join(ROOT, s)), s
