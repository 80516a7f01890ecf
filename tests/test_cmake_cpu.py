"""The CMake build (CMakeLists.txt) of the C library, on the CPU: hipcc cross-compiles for gfx950;
the library it links exports every function include/ring_kv.h declares, and loads."""
import ctypes
import os
import shutil
import subprocess

import pytest

from ring_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("cmake") is None or shutil.which("ninja") is None
                    or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="cmake, ninja and ROCm are needed for the CMake build")
def test_cmake_build_exports_the_interface(tmp_path):
    build = tmp_path / "build"
    for cmd in (["cmake", "-S", ROOT, "-B", str(build), "-G", "Ninja"],
                ["cmake", "--build", str(build), "-j", "8"]):
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=1200)
        assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    flags = (build / "build.ninja").read_text()
    assert "--offload-arch=gfx950" in flags
    assert "-Xclang -target-feature -Xclang -packed-fp32-ops" in flags
    lib = ctypes.CDLL(str(build / "libring_kv.so"))
    for name in _lib.declared_functions():
        assert hasattr(lib, name), name
    lib.rkv_abi_version.restype = ctypes.c_int32
    assert lib.rkv_abi_version() == 1
