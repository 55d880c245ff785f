"""Build libpe.so (the gfx950 HIP kernels and the C ABI of include/pe.h) in-tree with hipcc.

Every .hip source is compiled to its own object in parallel (each kernel is launched from the source that
defines it, so no relocatable device code is needed), then the objects are linked into one shared library.

The device pass is compiled with the target feature that stops the backend from forming packed fp32
instructions (v_pk_fma_f32 and its add / mul forms); hipcc hands the same -Xclang option to the host pass,
which does not know the feature and says so once per source. Only that host-pass message is dropped from
the output. tests/test_build_guard.py checks the device code of the built library for those instructions,
and that the option is what removes them.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libpe.so")
OBJ_DIR = os.path.join(PKG, "_build")

NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_PASS_NOTE = "packed-fp32-ops' is not a recognized feature"

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    *NO_PACKED_FP32,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpe.so)")


def sources() -> list:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _filtered(text: str) -> str:
    return "\n".join(line for line in text.splitlines() if HOST_PASS_NOTE not in line)


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, _filtered(r.stdout + r.stderr)


def build(verbose: bool = False, jobs: int = None) -> str:
    """Compile every HIP source and link eagle_drafting_amd/libpe.so (always recompiles)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[hipcc(), *HIPCC_FLAGS, *inc, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, out), s in zip(results, srcs):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(s)} ({rc}):\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    rc, out = _run(link)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
