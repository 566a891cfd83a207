"""Build of the HIP library (libmoe_mi355x.so) with hipcc for gfx950.

Compiles every source under ``csrc/`` in parallel into ``_build/`` and links the
shared library next to this file.  Always recompiles.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
ROOT_INCLUDE = os.path.join(os.path.dirname(HERE), "include")
PROBES_SRC = os.path.join(HERE, "probes", "probes.hip")
PROBES_LIB = os.path.join(HERE, "probes", "libmoe_probes.so")

ARCH = "gfx950"
# packed-fp32 instructions are disabled: plain fp32 code only
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", ROOT_INCLUDE,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
               "-Wno-pass-failed"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-x", "hip", *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build(jobs: int = 8) -> str:
    """The layer's library, then the benchmark's probe library (a separate .so)."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources() + [PROBES_SRC]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PROBES_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
