"""The host side of the library under AddressSanitizer.

api.cpp (argument validation, numpy.matmul broadcast resolution, batch
folding, the quantisation-parameter axes, workspace sizing, the dispatch
plans) is rebuilt with host-side ASan (device code unchanged), linked with the
normal kernel objects into a separate libomm, and the whole CPU ABI suite runs
against it in a child process with the ASan runtime preloaded.  Any invalid
host memory access there aborts the child with an ASan report.  CPU only."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "onnx_matmul_family_amd")
HIPCC = "/opt/rocm/bin/hipcc"


def asan_runtime():
    c = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return c[-1] if c else None


@pytest.mark.skipif(not os.path.exists(HIPCC) or asan_runtime() is None, reason="hipcc / ASan runtime not available")
def test_abi_suite_under_asan(tmp_path):
    from onnx_matmul_family_amd import build as b
    objs = [os.path.join(b.BUILD, s + ".o") for s in b.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        b.build()
    api_o = str(tmp_path / "api_asan.o")
    lib = str(tmp_path / "libomm_asan.so")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include")]
    subprocess.run([HIPCC] + flags + ["-x", "hip", "-c", os.path.join(PKG, "csrc", "api.cpp"), "-o", api_o],
                   check=True, capture_output=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", "-o", lib,
                    api_o] + objs, check=True, capture_output=True)
    env = dict(os.environ, OMM_LIB=lib, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert "AddressSanitizer" not in r.stderr + r.stdout, (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " passed" in r.stdout
