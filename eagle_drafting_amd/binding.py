"""ctypes binding of libpe.so (include/pe.h). Argument marshalling only: every step of the draft and
verify path runs in the library's HIP kernels. Tensors are passed as device pointers (torch tensors,
or raw integer addresses); the library never takes ownership.

The library must be built (eagle_drafting_amd.build); importing this module without it raises.
"""

from __future__ import annotations

import ctypes
import os
import sys
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_void_p

PE_MAX_LAYERS = 8
PE_MAX_BATCH = 1024
PE_MAX_K = 16

PE_OK, PE_ERR_INVALID, PE_ERR_UNSUPPORTED, PE_ERR_OOM, PE_ERR_HIP = 0, 1, 2, 3, 4
PE_F32, PE_BF16 = 0, 1
PE_PROF_LM_HEAD, PE_PROF_ATTENTION, PE_PROF_GATE_UP, PE_PROF_VERIFY_SCAN = 0, 1, 2, 3
PE_PROF_QKV, PE_PROF_O_PROJ, PE_PROF_DOWN, PE_PROF_ROWS = 4, 5, 6, 7
PE_PROF_COUNT = 8

# the in-tree build; PE_LIBRARY names another build of the same library (e.g. one with host sanitizers)
LIB_PATH = os.environ.get("PE_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpe.so")

EXPORTED = ["pe_config_validate", "pe_init", "pe_draft_step", "pe_draft_rows", "pe_draft_ar", "pe_draft_catchup",
            "pe_verify", "pe_verify_sampled", "pe_verify_static",
            "pe_destroy",
            "pe_device_flags", "pe_profile_enable", "pe_profile_read", "pe_status_string", "pe_last_error"]


class pe_config(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("d_model", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("ffn_dim", c_int32), ("vocab", c_int32), ("rms_eps", c_float),
                ("rope_base", c_float), ("dtype", c_int32), ("max_batch", c_int32), ("max_k", c_int32),
                ("max_ctx", c_int32), ("n_slots", c_int32), ("row_concat", c_int32), ("weight_fp8", c_int32)]


_L = c_void_p * PE_MAX_LAYERS


class pe_weights(ctypes.Structure):
    _fields_ = [("fc", c_void_p), ("embed", c_void_p), ("emb_mask", c_void_p), ("h_shared", c_void_p),
                ("final_norm", c_void_p), ("lm_head", c_void_p), ("attn_norm", _L), ("wqkv", _L), ("wo", _L),
                ("mlp_norm", _L), ("wgate", _L), ("wup", _L), ("wdown", _L), ("embed_norm", c_void_p)]


class pe_kv(ctypes.Structure):
    _fields_ = [("k", _L), ("v", _L)]


class PeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


def _status_name(s: int) -> str:
    return {0: "PE_OK", 1: "PE_ERR_INVALID", 2: "PE_ERR_UNSUPPORTED", 3: "PE_ERR_OOM", 4: "PE_ERR_HIP"}.get(s, str(s))


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libpe.so (once). Raises if it is missing: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m eagle_drafting_amd.build` "
                          "(hipcc, gfx950); the draft/verify path has no other implementation")
    # libpe.so needs the HIP runtime by soname; when PyTorch (which ships its own copy of that runtime) is
    # present, load it first so that the process holds one runtime and torch's device buffers and
    # streams are valid for the library.
    if "torch" not in sys.modules:
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
    lib = ctypes.CDLL(path)
    vp, i32 = c_void_p, c_int32
    sig = {
        "pe_config_validate": ([POINTER(pe_config)], i32),
        "pe_init": ([POINTER(pe_config), POINTER(pe_weights), POINTER(pe_kv), vp, POINTER(vp)], i32),
        "pe_draft_step": ([vp, i32, i32, vp, vp, vp, vp, vp, vp], i32),
        "pe_draft_rows": ([vp, i32, i32, vp, vp, vp, vp, vp], i32),
        "pe_draft_ar": ([vp, i32, i32, vp, vp, vp, vp, vp, vp], i32),
        "pe_draft_catchup": ([vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp], i32),
        "pe_verify": ([vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp], i32),
        "pe_verify_sampled": ([vp, i32, i32, vp, vp, c_float, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
                              i32),
        "pe_verify_static": ([i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp], i32),
        "pe_destroy": ([vp], i32),
        "pe_device_flags": ([vp, i32, POINTER(i32)], i32),
        "pe_profile_enable": ([vp, i32], i32),
        "pe_profile_read": ([vp, i32, POINTER(c_double), POINTER(c_int64)], i32),
        "pe_status_string": ([i32], c_char_p),
        "pe_last_error": ([vp], c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _check(status: int, ctx=None):
    if status != PE_OK:
        msg = load_library().pe_last_error(ctx).decode(errors="replace")
        raise PeError(status, msg)


def pe_status_string(status: int) -> str:
    return load_library().pe_status_string(status).decode()


def pe_last_error(ctx=None) -> str:
    return load_library().pe_last_error(ctx).decode(errors="replace")


def pe_config_validate(cfg: pe_config) -> int:
    """Host-only check; returns the pe_status (0 = valid)."""
    return load_library().pe_config_validate(ctypes.byref(cfg))


def pe_init(cfg: pe_config, weights: pe_weights, kv: pe_kv, stream: int = 0):
    """Returns an opaque ctx handle (int). stream: a hipStream_t address (0 = default stream)."""
    out = c_void_p()
    _check(load_library().pe_init(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(kv), stream or None,
                                  ctypes.byref(out)))
    return out.value


def pe_draft_step(ctx, B, K, req_slot, seq_len, last_token, target_hidden, draft_tokens, logits=None):
    _check(load_library().pe_draft_step(ctx, B, K, _ptr(req_slot), _ptr(seq_len), _ptr(last_token),
                                        _ptr(target_hidden), _ptr(draft_tokens), _ptr(logits)), ctx)


def pe_draft_ar(ctx, B, K, req_slot, seq_len, last_token, target_hidden, draft_tokens, logits=None):
    _check(load_library().pe_draft_ar(ctx, B, K, _ptr(req_slot), _ptr(seq_len), _ptr(last_token),
                                      _ptr(target_hidden), _ptr(draft_tokens), _ptr(logits)), ctx)


def pe_draft_catchup(ctx, B, K, R, req_slot, seq_len, n_real, tokens, target_hidden, draft_tokens, logits=None):
    _check(load_library().pe_draft_catchup(ctx, B, K, R, _ptr(req_slot), _ptr(seq_len), _ptr(n_real), _ptr(tokens),
                                           _ptr(target_hidden), _ptr(draft_tokens), _ptr(logits)), ctx)


def pe_draft_rows(ctx, B, K, req_slot, seq_len, rows, draft_tokens, logits=None):
    _check(load_library().pe_draft_rows(ctx, B, K, _ptr(req_slot), _ptr(seq_len), _ptr(rows), _ptr(draft_tokens),
                                        _ptr(logits)), ctx)


def pe_verify(ctx, B, K, target_logits, draft_tokens, finished, req_slot, seq_len, accept_len, cu_accept,
              out_tokens, keep_index, n_keep, req_slot_next, seq_len_next, last_token_next):
    _check(load_library().pe_verify(ctx, B, K, _ptr(target_logits), _ptr(draft_tokens), _ptr(finished),
                                    _ptr(req_slot), _ptr(seq_len), _ptr(accept_len), _ptr(cu_accept),
                                    _ptr(out_tokens), _ptr(keep_index), _ptr(n_keep), _ptr(req_slot_next),
                                    _ptr(seq_len_next), _ptr(last_token_next)), ctx)


def pe_verify_sampled(ctx, B, K, target_logits, draft_tokens, temperature, u, v, finished, req_slot, seq_len,
                      accept_len, cu_accept, out_tokens, keep_index, n_keep, req_slot_next, seq_len_next,
                      last_token_next):
    _check(load_library().pe_verify_sampled(
        ctx, B, K, _ptr(target_logits), _ptr(draft_tokens), float(temperature), _ptr(u), _ptr(v), _ptr(finished),
        _ptr(req_slot), _ptr(seq_len), _ptr(accept_len), _ptr(cu_accept), _ptr(out_tokens), _ptr(keep_index),
        _ptr(n_keep), _ptr(req_slot_next), _ptr(seq_len_next), _ptr(last_token_next)), ctx)


def pe_verify_static(B, K, vocab, dtype, target_logits, draft_tokens, finished, req_slot, seq_len, accept_len,
                     cu_accept, out_tokens, keep_index, n_keep, req_slot_next, seq_len_next, last_token_next,
                     stream=0):
    """pe_verify without a ctx and without allocating (static scratch inside the library).
    dtype: "f32" / "bf16" or PE_F32 / PE_BF16."""
    dt = {"f32": PE_F32, "bf16": PE_BF16}.get(dtype, dtype)
    _check(load_library().pe_verify_static(
        B, K, vocab, int(dt), _ptr(target_logits), _ptr(draft_tokens), _ptr(finished), _ptr(req_slot),
        _ptr(seq_len), _ptr(accept_len), _ptr(cu_accept), _ptr(out_tokens), _ptr(keep_index), _ptr(n_keep),
        _ptr(req_slot_next), _ptr(seq_len_next), _ptr(last_token_next), stream or None))


def pe_destroy(ctx):
    _check(load_library().pe_destroy(ctx))


def pe_device_flags(ctx, clear: bool = False) -> int:
    out = c_int32()
    _check(load_library().pe_device_flags(ctx, 1 if clear else 0, ctypes.byref(out)), ctx)
    return out.value


def pe_profile_enable(ctx, mask: int = (1 << PE_PROF_COUNT) - 1):
    """Record per-launch events for the kernels whose bit (1 << PE_PROF_*) is set; 0 stops."""
    _check(load_library().pe_profile_enable(ctx, int(mask)), ctx)


def pe_profile_read(ctx, which: int):
    """(summed milliseconds, launches) of one profiled kernel since pe_profile_enable."""
    ms, n = c_double(), c_int64()
    _check(load_library().pe_profile_read(ctx, which, ctypes.byref(ms), ctypes.byref(n)), ctx)
    return ms.value, n.value


# ---- struct builders (marshalling helpers) ----------------------------------------------------------

def make_config(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, dtype, max_batch, max_k,
                max_ctx, n_slots, rms_eps=1e-6, rope_base=10000.0, row_concat=0, weight_fp8=0) -> pe_config:
    return pe_config(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, rms_eps, rope_base,
                     PE_BF16 if dtype in ("bf16", PE_BF16) else PE_F32, max_batch, max_k, max_ctx, n_slots,
                     int(row_concat), int(weight_fp8))


def make_weights(t: dict, n_layers: int) -> pe_weights:
    """t: name -> device tensor, names as in include/pe.h ('fc', ..., 'l{i}.wqkv', ...)."""
    w = pe_weights()
    for name in ("fc", "embed", "emb_mask", "h_shared", "final_norm", "lm_head"):
        setattr(w, name, _ptr(t[name]))
    for l in range(n_layers):
        for name in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgate", "wup", "wdown"):
            getattr(w, name)[l] = _ptr(t[f"l{l}.{name}"])
    if "embed_norm" in t:
        w.embed_norm = _ptr(t["embed_norm"])
    return w


def make_kv(k_layers, v_layers) -> pe_kv:
    kv = pe_kv()
    for l, (k, v) in enumerate(zip(k_layers, v_layers)):
        kv.k[l] = _ptr(k)
        kv.v[l] = _ptr(v)
    return kv
