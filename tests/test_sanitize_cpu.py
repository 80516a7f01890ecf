"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU): the library's host side
(argument checks, split choice, pager, paging batches) built with both sanitizers on the host
pass only, and driven by tests/sanitize_driver.cpp (random pager sequences with invariants, every
entry point's rejection paths, which return before any HIP call)."""
import os
import subprocess

import pytest

from ring_kv_amd.build import SOURCES   # the library's own source list

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="ROCm's hipcc is needed")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "driver")
    host_sanitizers = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", *host_sanitizers, f"-I{os.path.join(ROOT, 'include')}",
           *[os.path.join(ROOT, "ring_kv_amd", "csrc", s) for s in SOURCES],
           os.path.join(ROOT, "tests", "sanitize_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, cwd=str(tmp_path))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "sanitized host checks passed" in r.stdout
