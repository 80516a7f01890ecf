"""Build libring_kv.so (the C interface in include/ring_kv.h) in-tree for gfx950.

    python -m ring_kv_amd.build            # or: python ring_kv_amd/build.py
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libring_kv.so")
# measurement-only streaming read probe, used by bench.py (not part of the C interface)
PROBE_LIB = os.path.join(HERE, "libring_kv_probe.so")
PROBE_SRC = "probe.hip"
SOURCES = ["abi.hip", "attn_chunked.hip", "attn_prefill.hip", "attn_merge.hip",
           "attn_contig.hip", "accept.hip", "layout.hip", "paging.hip", "pager.cpp"]
ARCH = "gfx950"

# Packed-fp32 VALU forms stay off: hipcc would otherwise form v_pk_* f32 ops from plain float
# code (the host pass warns that it does not know the feature; that is harmless).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{os.path.join(ROOT, 'include')}"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libring_kv)")


def _compile(hipcc: str, src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    pobj = _compile(hipcc, PROBE_SRC)
    r = subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", pobj, "-o",
                        PROBE_LIB + ".tmp"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (probe)\n{r.stdout}\n{r.stderr}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
