"""Copies of the synthetic inputs in GPU memory (torch tensors), for the GPU tests and the benchmark.

Only moves data: bf16 inputs keep their exact bit patterns; nothing here computes.
"""

from __future__ import annotations

import numpy as np

from .inputs import make_kv_cache, make_weight, weight_shapes
from .workloads import Workload


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16" and a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def upload_weights(s, device="cuda", keep_host=False):
    """Generate and upload every tensor of drafter shape s; returns (device dict, host dict or None)."""
    dev, host = {}, ({} if keep_host else None)
    for name in weight_shapes(s):
        raw = make_weight(s, name)
        dev[name] = to_device(raw, s.dtype, device)
        if keep_host:
            host[name] = raw
    return dev, host


def upload_kv(w: Workload, state: dict, device="cuda", request_keys=None):
    """Per-layer K and V caches [n_slots, Hkv, max_ctx, hd] holding each request's context."""
    ks, vs = [], []
    for l in range(w.shape.n_layers):
        ks.append(to_device(make_kv_cache(w, l, 0, state, request_keys), w.shape.dtype, device))
        vs.append(to_device(make_kv_cache(w, l, 1, state, request_keys), w.shape.dtype, device))
    return ks, vs


def upload_state(state: dict, dtype: str, device="cuda") -> dict:
    return {"req_slot": to_device(state["req_slot"], "i32", device),
            "seq_len": to_device(state["seq_len"], "i32", device),
            "last_token": to_device(state["last_token"], "i32", device),
            "target_hidden": to_device(state["target_hidden"], dtype, device)}


def config_args(w: Workload, max_batch=None, max_k=None, max_ctx=None, n_slots=None) -> dict:
    s = w.shape
    return dict(n_layers=s.n_layers, d_model=s.d_model, n_q_heads=s.n_q_heads, n_kv_heads=s.n_kv_heads,
                head_dim=s.head_dim, ffn_dim=s.ffn_dim, vocab=s.vocab, dtype=s.dtype,
                max_batch=max_batch or w.B, max_k=max_k or w.K, max_ctx=max_ctx or w.max_ctx,
                n_slots=n_slots or w.n_slots, rms_eps=s.rms_eps, rope_base=s.rope_base, row_concat=int(s.row_concat))
