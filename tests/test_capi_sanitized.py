"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): csrc/api.hip is compiled with the sanitizers on its host pass
only (device code is built as usual), linked with the library's other objects
and tests/capi_host_check.cpp, and run.  The check program drives every entry
point's argument validation, including extreme sizes, and the workspace-size
queries; a memory error, a signed overflow or a failed expectation fails the
test.  Needs the objects of a normal build (block_scaled_fp4_permute_amd/_build)."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_scaled_fp4_permute_amd")
BUILD = os.path.join(PKG, "_build")
ROCM = "/opt/rocm"

try:
    import torch
    _HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    _HAVE_GPU = False

pytestmark = pytest.mark.skipif(_HAVE_GPU, reason="fake device addresses: host-only checks, run without a GPU")

SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]


def test_capi_validation_under_asan_ubsan(tmp_path):
    from block_scaled_fp4_permute_amd import build as B
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("ROCm toolchain not found")
    others = [o for o in glob.glob(os.path.join(BUILD, "*.o")) if os.path.basename(o) != "api.o"]
    srcs = [os.path.basename(s).replace(".hip", ".o") for s in B.sources()]
    if sorted(os.path.basename(o) for o in others) != sorted(s for s in srcs if s != "api.o"):
        pytest.skip("library objects missing: build first (python -m block_scaled_fp4_permute_amd.build)")
    api_o = str(tmp_path / "api_san.o")
    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    subprocess.run([hipcc, *B.HIPCC_FLAGS, *host_san, "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o],
                   check=True, capture_output=True)
    drv_o = str(tmp_path / "check.o")
    subprocess.run([clangxx, "-std=c++17", "-O1", "-g", "-I", os.path.join(ROOT, "include"), *SAN, "-c",
                    os.path.join(ROOT, "tests", "capi_host_check.cpp"), "-o", drv_o], check=True, capture_output=True)
    exe = str(tmp_path / "check")
    subprocess.run([clangxx, *SAN, drv_o, api_o, *others, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "ok: 0 failed" in r.stdout
