"""Host code under AddressSanitizer (CPU only, no HIP call is made).

tests/asan/abi_oracle_checks.cpp drives every C-ABI entry point through the
argument checks the host makes before any HIP call, and the fp64 C oracle's
forward and backward through small ragged batches with every mask rule.  It is
linked with the C-ABI source (hstu_attn.hip: descriptor, pointer, stride,
workspace and shape validation, error messages) compiled with the sanitizer on
its host code, the oracle compiled with the sanitizer, and the built library
for the launch wrappers, which these paths never reach.  An invalid access or
a leak aborts the program; the test also requires its "ok" line.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "jagged_hstu_attention_attn_amd", "csrc")
LIB = os.path.join(ROOT, "jagged_hstu_attention_attn_amd", "libhstu_attn.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer"]


def _run(cmd, cwd):
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout[-3000:]}{res.stderr[-3000:]}"
    return res


@pytest.mark.skipif(not all(os.path.exists(p) for p in (HIPCC, CLANG, CLANGXX)),
                    reason="ROCm clang / hipcc not installed")
def test_host_code_under_address_sanitizer(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("library not built (run __graft_entry__.build())")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    # the C-ABI source: sanitizer on its host code only
    _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-fPIC", *SAN,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", *inc,
          "-c", os.path.join(CSRC, "hstu_attn.hip"), "-o", "abi.o"], tmp_path)
    _run([CLANG, "-std=c11", *SAN, "-fsanitize=address", "-Wno-unknown-pragmas",
          "-c", os.path.join(ROOT, "oracle", "hstu_oracle.c"), "-o", "oracle.o"], tmp_path)
    _run([CLANGXX, "-std=c++17", *SAN, "-fsanitize=address", *inc,
          "-c", os.path.join(ROOT, "tests", "asan", "abi_oracle_checks.cpp"), "-o", "drv.o"],
         tmp_path)
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
          "drv.o", "oracle.o", "abi.o", LIB, f"-Wl,-rpath,{ROCM}/lib", "-lm", "-o", "checks"],
         tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23")
    res = subprocess.run([str(tmp_path / "checks")], cwd=tmp_path, capture_output=True,
                         text=True, timeout=300, env=env)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ok:" in res.stdout and "AddressSanitizer" not in out, out[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
