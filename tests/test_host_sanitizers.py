"""The C-ABI layer's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

pe_api.hip (argument checks, configuration validation, error reporting, the static-scratch lookup) is
compiled with host-side sanitizers and linked with the other objects of the regular build; the ABI tests
then run in a child process against that library with the sanitizer runtime preloaded. Any sanitizer
report fails the test. Device code is not instrumented (the sanitizers apply to the host pass only).
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_RT = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"


def test_abi_tests_pass_under_host_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists(ASAN_RT):
        pytest.skip("hipcc or the sanitizer runtime is not available")
    from eagle_drafting_amd import build
    objs = [os.path.join(build.OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in build.sources()
            if not s.endswith("pe_api.hip")]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "eagle_drafting_amd", "csrc")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    obj = str(tmp_path / "pe_api_san.o")
    lib = str(tmp_path / "libpe_san.so")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *build.NO_PACKED_FP32,
                        *san, *inc, "-c", os.path.join(ROOT, "eagle_drafting_amd", "csrc", "pe_api.hip"), "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", obj, *objs,
                        "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, PE_LIBRARY=lib, LD_PRELOAD=ASAN_RT,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
