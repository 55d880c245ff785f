"""The C-ABI library: it loads, exports every function include/pe.h declares, and rejects bad arguments
on the host before touching a GPU (no GPU needed)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from eagle_drafting_amd import binding
    return binding.load_library()


def test_library_exports_every_declared_function(lib):
    names = _declared_functions()
    assert "pe_init" in names and "pe_draft_step" in names and "pe_verify" in names
    from eagle_drafting_amd import binding
    raw = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert sorted(binding.EXPORTED) == names


def _good(**kw):
    from eagle_drafting_amd import binding
    args = dict(n_layers=4, d_model=2048, n_q_heads=32, n_kv_heads=4, head_dim=128, ffn_dim=6144, vocab=151936,
                dtype="bf16", max_batch=8, max_k=11, max_ctx=4224, n_slots=10)
    args.update(kw)
    return binding.make_config(**args)


def test_config_validation_host_only(lib):
    from eagle_drafting_amd import binding as b
    assert b.pe_config_validate(_good()) == b.PE_OK
    assert b.pe_config_validate(_good(dtype="f32", d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
                                      ffn_dim=512, vocab=4096, max_ctx=128)) == b.PE_OK
    bad = {
        "n_layers": (0, b.PE_ERR_INVALID), "n_kv_heads": (5, b.PE_ERR_INVALID), "max_batch": (0, b.PE_ERR_INVALID),
        "max_k": (17, b.PE_ERR_INVALID), "head_dim": (96, b.PE_ERR_UNSUPPORTED), "d_model": (2040, b.PE_ERR_UNSUPPORTED),
        "vocab": (151937, b.PE_ERR_UNSUPPORTED), "n_slots": (0, b.PE_ERR_INVALID),
    }
    for field, (val, want) in bad.items():
        assert b.pe_config_validate(_good(**{field: val})) == want, field
        assert b.pe_last_error(None)
    # G * max_k beyond one workgroup's query rows
    assert b.pe_config_validate(_good(n_kv_heads=1, max_k=8)) == b.PE_ERR_UNSUPPORTED
    # the two variants: flags are 0 / 1, bf16 drafters only, and FP8 weights go with summed rows
    f32 = dict(dtype="f32", d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn_dim=512, vocab=4096, max_ctx=128)
    assert b.pe_config_validate(_good(row_concat=1)) == b.PE_OK
    assert b.pe_config_validate(_good(weight_fp8=1)) == b.PE_OK
    assert b.pe_config_validate(_good(row_concat=2)) == b.PE_ERR_INVALID
    assert b.pe_config_validate(_good(weight_fp8=-1)) == b.PE_ERR_INVALID
    assert b.pe_config_validate(_good(row_concat=1, **f32)) == b.PE_ERR_UNSUPPORTED
    assert b.pe_config_validate(_good(weight_fp8=1, **f32)) == b.PE_ERR_UNSUPPORTED
    assert b.pe_config_validate(_good(weight_fp8=1, row_concat=1)) == b.PE_ERR_UNSUPPORTED


def test_status_strings(lib):
    from eagle_drafting_amd import binding as b
    assert b.pe_status_string(b.PE_OK) == "ok"
    assert "invalid" in b.pe_status_string(b.PE_ERR_INVALID)


def test_init_rejects_null_pointers_before_any_gpu_call(lib):
    from eagle_drafting_amd import binding as b
    cfg = _good()
    with pytest.raises(b.PeError) as e:
        b.pe_init(cfg, b.pe_weights(), b.pe_kv(), 0)
    assert e.value.status == b.PE_ERR_INVALID


def test_calls_on_null_ctx_are_rejected(lib):
    from eagle_drafting_amd import binding as b
    assert lib.pe_draft_step(None, 1, 1, None, None, None, None, None, None) == b.PE_ERR_INVALID
    assert lib.pe_verify(None, 1, 1, *([None] * 13)) == b.PE_ERR_INVALID
    assert lib.pe_destroy(None) == b.PE_OK


def test_python_binding_fails_loudly_without_library(tmp_path):
    from eagle_drafting_amd import binding as b
    saved = b._lib
    try:
        b._lib = None
        with pytest.raises(ImportError):
            b.load_library(str(tmp_path / "missing.so"))
    finally:
        b._lib = saved


def test_static_verify_rejects_bad_arguments_on_the_host(lib):
    from eagle_drafting_amd import binding as b
    good = dict(B=4, K=3, vocab=4096, dtype=b.PE_BF16)
    ptrs = [16] * 13  # non-null, 16-byte aligned stand-ins: never dereferenced, the checks fail first
    for kw in ({"B": 0}, {"B": 1025}, {"K": 0}, {"K": 17}, {"vocab": 4100}, {"vocab": 0}, {"dtype": 7}):
        a = {**good, **kw}
        assert lib.pe_verify_static(a["B"], a["K"], a["vocab"], a["dtype"], *ptrs, None) == b.PE_ERR_INVALID, kw
        assert b.pe_last_error(None)
    assert lib.pe_verify_static(4, 3, 4096, b.PE_BF16, None, *ptrs[1:], None) == b.PE_ERR_INVALID
    assert lib.pe_verify_static(4, 3, 4096, b.PE_BF16, 8, *ptrs[1:], None) == b.PE_ERR_INVALID  # misaligned


def test_gpu_calls_without_a_device_return_hip_errors(lib):
    # on a host without a usable GPU the first HIP call fails; the library reports PE_ERR_HIP instead of
    # aborting (valid arguments, so the host checks pass)
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    from eagle_drafting_amd import binding as b
    assert lib.pe_verify_static(4, 3, 4096, b.PE_BF16, *([16] * 13), None) == b.PE_ERR_HIP
    assert "hip" in b.pe_last_error(None).lower()
    w = b.pe_weights()
    for f in ("fc", "embed", "emb_mask", "h_shared", "final_norm", "lm_head"):
        setattr(w, f, 16)
    kv = b.pe_kv()
    for l in range(4):
        for arr in (w.attn_norm, w.wqkv, w.wo, w.mlp_norm, w.wgate, w.wup, w.wdown, kv.k, kv.v):
            arr[l] = 16
    with pytest.raises(b.PeError) as e:
        b.pe_init(_good(), w, kv, 0)
    assert e.value.status == b.PE_ERR_HIP
