"""The library's host logic (validation, tile scheduler, decode planner, status
strings) built with AddressSanitizer and UBSan and driven by tests/native/host_checks.c
through the C ABI.  Every call there returns before any device work, so this runs
on the CPU; the kernels come from the regular build's objects."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
BUILD = os.path.join(ROOT, "attention_fa_fwd_amd", "_build")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}"
    return r.stdout


def test_host_logic_is_clean_under_asan_and_ubsan(tmp_path):
    objs = [o for o in glob.glob(os.path.join(BUILD, "*.o")) if not o.endswith("fa_api.o")]
    if not os.path.exists(HIPCC) or not os.path.exists(CLANG) or len(objs) < 5:
        pytest.skip("needs hipcc, clang and the regular build's objects")
    api = str(tmp_path / "fa_api_san.o")
    lib = str(tmp_path / "libfa_san.so")
    exe = str(tmp_path / "host_checks")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + SAN +
         ["-c", os.path.join(ROOT, "attention_fa_fwd_amd", "csrc", "fa_api.hip"), "-o", api])
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + SAN + ["-o", lib, api] + objs)
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "native", "host_checks.c"),
          "-o", exe, lib, "-Wl,-rpath," + str(tmp_path)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    out = _run([exe], env=env, timeout=600)
    assert "host checks passed" in out
