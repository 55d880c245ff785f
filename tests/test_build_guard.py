"""The gfx950 device code of libpe.so holds no packed fp32 arithmetic (no GPU needed).

Packed fp32 instructions (v_pk_fma_f32, v_pk_mul_f32, v_pk_add_f32) are kept out of every kernel by a
backend target feature given to the device pass (eagle_drafting_amd/build.py). These tests read the
built library's gfx950 code objects (one offload bundle per source) and disassemble them with the ROCm
LLVM tools, and they check on a two-line kernel that the option is what keeps the instructions out:
the same source compiled without it does contain one.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "eagle_drafting_amd", "libpe.so")
LLVM = "/opt/rocm/llvm/bin"
PACKED = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tool(name):
    p = os.path.join(LLVM, name)
    if not os.path.exists(p):
        pytest.skip(f"{name} not available")
    return p


def _device_asm(so_path, tmp_path):
    """Disassembly of every gfx950 code object bundled in the .hip_fatbin section of so_path."""
    fat = tmp_path / "fat.bin"
    subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", so_path, str(tmp_path / "x.so")],
                   check=True, capture_output=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), data)]
    assert starts, "no offload bundle in .hip_fatbin"
    asm = []
    for i, s in enumerate(starts):
        part = tmp_path / f"b{i}.bin"
        part.write_bytes(data[s: starts[i + 1] if i + 1 < len(starts) else len(data)])
        co = tmp_path / f"b{i}.co"
        subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--input={part}",
                        f"--targets={TARGET}", f"--output={co}"], check=True, capture_output=True)
        r = subprocess.run([_tool("llvm-objdump"), "-d", str(co)], check=True, capture_output=True, text=True)
        asm.append(r.stdout)
    return asm


def test_library_device_code_has_no_packed_fp32(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libpe.so not built")
    asm = _device_asm(LIB, tmp_path)
    text = "\n".join(asm)
    # the disassembly is the real device code: every source's kernels are in it
    for kernel in ("attn_bf16_kernel", "gemm_tiled_kernel", "gemm_stream_kernel", "gemm_kernel",
                   "accept_compact_kernel", "sample_decide_kernel", "rope_table_kernel"):
        assert kernel in text, kernel
    assert "v_mfma" in text
    hits = sorted(set(m.group(0) for m in PACKED.finditer(text)))
    assert not hits, f"packed fp32 instructions in libpe.so: {hits}"


def test_the_build_option_is_what_removes_packed_fp32(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    from eagle_drafting_amd import build
    src = tmp_path / "pk.hip"
    src.write_text("#include <hip/hip_runtime.h>\n"
                   "__global__ void k(float2* a, const float2* b, float s) {\n"
                   "  int i = threadIdx.x; float2 x = a[i], y = b[i];\n"
                   "  x.x = x.x * s + y.x; x.y = x.y * s + y.y; a[i] = x; }\n")
    counts = []
    for extra in ([], build.NO_PACKED_FP32):
        so = tmp_path / f"pk{len(extra)}.so"
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", *extra, str(src), "-o", str(so)],
                       check=True, capture_output=True)
        counts.append(sum(len(PACKED.findall(a)) for a in _device_asm(str(so), tmp_path)))
    assert counts[0] > 0 and counts[1] == 0, counts
