"""Seeded generators for drafter weights, request state, KV caches and target logits.

Every tensor has its own child generators (numpy PCG64 seeded with [seed, tensor code, ..., chunk]), so
any tensor or any request's KV block can be regenerated alone, in any order and with any thread count.

bf16 tensors are produced by round-to-nearest-even of float32 draws and returned as raw uint16 bits;
`bf16_bits_to_f32` gives the exact float32 values those bits encode.
"""

from __future__ import annotations

import os

import numpy as np

from .workloads import DrafterShape, Workload

_CHUNK = 1 << 22


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)

    def conv(s):
        u = flat[s:s + _CHUNK].view(np.uint32)
        r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
        out[s:s + _CHUNK] = r.astype(np.uint16)

    starts = range(0, flat.size, _CHUNK)
    if flat.size > _CHUNK:
        list(_pool().map(conv, starts))
    else:
        for s in starts:
            conv(s)
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bf16_bits(x))


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def _normal(key: tuple, shape, scale=1.0, loc=0.0) -> np.ndarray:
    """N(loc, scale^2) float32 draws; chunk c of 2^22 values comes from child generator [*key, c], so
    the values do not depend on how many threads fill them."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)

    def fill(c):
        s0, s1 = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        part = out[s0:s1]
        _rng(*key, c).standard_normal(s1 - s0, dtype=np.float32, out=part)
        if scale != 1.0:
            part *= np.float32(scale)
        if loc != 0.0:
            part += np.float32(loc)

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        list(_pool().map(fill, range(nchunks)))
    return out.reshape(shape)


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return x if dtype == "f32" else bf16_bits(x)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a generated tensor (float32 array, or uint16 bf16 bits)."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float64)
    return bf16_bits_to_f32(arr).astype(np.float64)


# tensor codes for the per-tensor child generators
_CODES = {"fc": 1, "embed": 2, "emb_mask": 3, "h_shared": 4, "final_norm": 5, "lm_head": 6, "embed_norm": 7,
          "attn_norm": 10, "wqkv": 11, "wo": 12, "mlp_norm": 13, "wgate": 14, "wup": 15, "wdown": 16}


def weight_shapes(s: DrafterShape) -> dict:
    d, V, F = s.d_model, s.vocab, s.ffn_dim
    shapes = {"fc": (d, 3 * d), "embed": (V, d), "emb_mask": (d,), "h_shared": (d,),
              "final_norm": (d,), "lm_head": (V, d)}
    for l in range(s.n_layers):
        shapes[f"l{l}.attn_norm"] = (d,)
        shapes[f"l{l}.wqkv"] = (s.qkv_dim, d)
        shapes[f"l{l}.wo"] = (d, s.q_dim)
        shapes[f"l{l}.mlp_norm"] = (d,)
        shapes[f"l{l}.wgate"] = (F, d)
        shapes[f"l{l}.wup"] = (F, d)
        shapes[f"l{l}.wdown"] = (d, F)
    if s.row_concat:
        shapes["l0.wqkv"] = (s.qkv_dim, 2 * d)
        shapes["embed_norm"] = (d,)
    return shapes


def make_weight(s: DrafterShape, name: str, seed: int = None) -> np.ndarray:
    """One drafter tensor. Matrices are [out, in] (y = x . W^T), drawn N(0, 0.02); norm gains are
    1 + N(0, 0.02). Returned as float32 (f32 shapes) or bf16 bits (bf16 shapes)."""
    shape = weight_shapes(s)[name]
    if "." in name:
        layer, base = name.split(".")
        layer = int(layer[1:])
    else:
        layer, base = 0, name
    key = (s.weight_seed if seed is None else seed, _CODES[base], layer)
    if base.endswith("norm"):
        x = _normal(key, shape, 0.02, 1.0)
    else:
        x = _normal(key, shape, 0.02)
    return _encode(x, s.dtype)


def make_weights(s: DrafterShape, seed: int = None) -> dict:
    return {name: make_weight(s, name, seed) for name in weight_shapes(s)}


def make_state(w: Workload, step: int = 0) -> dict:
    """Per-request state for one drafting step.

    req_slot [B] int32: distinct KV slots (a random subset of n_slots)
    seq_len [B] int32: drafter context length L_b
    last_token [B] int32: token the target just produced, uniform in [0, V)
    target_hidden [B, 3d]: the three captured target hidden states (low, middle, high layer) as
        contiguous d-blocks, N(0, 1)
    alpha [B] float64: per-position planting probability for the target logits
    """
    s = w.shape
    rng = _rng(w.seed, 100, step)
    lo, hi = w.ctx
    seq_len = rng.integers(lo, hi + 1, size=w.B).astype(np.int32)
    req_slot = rng.permutation(w.n_slots)[: w.B].astype(np.int32)
    last_token = rng.integers(0, s.vocab, size=w.B).astype(np.int32)
    hid = _normal((w.seed, 101, step), (w.B, 3 * s.d_model))
    if isinstance(w.alpha, tuple):
        alpha = rng.uniform(w.alpha[0], w.alpha[1], size=w.B)
    else:
        alpha = np.full(w.B, float(w.alpha))
    return {"req_slot": req_slot, "seq_len": seq_len, "last_token": last_token,
            "target_hidden": _encode(hid, s.dtype), "alpha": alpha}


def kv_block(w: Workload, layer: int, kind: int, request_key: int, L: int) -> np.ndarray:
    """Context keys (kind 0) or values (kind 1) of one request: [Hkv, L, hd] N(0, 1), encoded.
    Cached keys count as already rotated by RoPE."""
    s = w.shape
    return _encode(_normal((w.seed, 200 + kind, layer, request_key), (s.n_kv_heads, L, s.head_dim)), s.dtype)


def make_kv_cache(w: Workload, layer: int, kind: int, state: dict, request_keys=None) -> np.ndarray:
    """Full cache tensor of one layer, [n_slots, Hkv, max_ctx, hd]; slot req_slot[b] holds request b's
    context in positions [0, L_b); everything else is zero."""
    s = w.shape
    dt = np.float32 if s.dtype == "f32" else np.uint16
    cache = np.zeros((w.n_slots, s.n_kv_heads, w.max_ctx, s.head_dim), dtype=dt)
    keys = list(range(w.B) if request_keys is None else request_keys)

    def fill(b):
        L = int(state["seq_len"][b])
        cache[state["req_slot"][b], :, :L, :] = kv_block(w, layer, kind, keys[b], L)

    global _KV_POOL
    if _KV_POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _KV_POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    list(_KV_POOL.map(fill, range(w.B)))
    return cache


_KV_POOL = None


def random_draft(w: Workload, step: int = 0) -> np.ndarray:
    """Harness draft tokens [B, K] int32, uniform in [0, V): verify inputs independent of any drafter."""
    rng = _rng(w.seed, 300, step)
    return rng.integers(0, w.shape.vocab, size=(w.B, w.K)).astype(np.int32)


def plant_target_logits(w: Workload, draft: np.ndarray, alpha: np.ndarray, step: int = 0) -> np.ndarray:
    """Target logits [B, K+1, V] N(0, 1), encoded in the shape's dtype.

    For position i < K of request b: with probability alpha[b] the draft token draft[b, i] receives
    the value (row maximum + 1); otherwise a different token, uniform over the other V - 1, does.
    Position K (the bonus position) keeps its plain draw.
    """
    s = w.shape
    V = s.vocab
    rng = _rng(w.seed, 400, step)
    B, K = draft.shape
    T = _normal((w.seed, 401, step), (B, K + 1, V))
    if s.dtype == "bf16":
        T = round_bf16(T)
    hit = rng.random((B, K)) < alpha[:, None]
    other = rng.integers(0, V - 1, size=(B, K))
    for b in range(B):
        for i in range(K):
            tok = int(draft[b, i])
            if not hit[b, i]:
                u = int(other[b, i])
                tok = u if u < tok else u + 1
            top = np.float32(T[b, i].max()) + np.float32(1.0)
            T[b, i, tok] = top
    if s.dtype == "bf16":
        return bf16_bits(T)
    return T


def churn_finished(w: Workload, step: int) -> np.ndarray:
    """finished [B] uint8: round(churn * B) requests, chosen without replacement."""
    rng = _rng(w.seed, 500, step)
    n_fin = int(np.floor(w.churn * w.B + 0.5))
    fin = np.zeros(w.B, dtype=np.uint8)
    if n_fin:
        fin[rng.choice(w.B, size=n_fin, replace=False)] = 1
    return fin


def new_request(w: Workload, step: int, index: int) -> dict:
    """A request that joins after churn: context length from new_ctx, fresh last token and hiddens."""
    s = w.shape
    rng = _rng(w.seed, 600, step, index)
    L = int(rng.integers(w.new_ctx[0], w.new_ctx[1] + 1))
    tok = int(rng.integers(0, s.vocab))
    hid = _encode(_normal((w.seed, 601, step, index), (3 * s.d_model,)), s.dtype)
    return {"seq_len": L, "last_token": tok, "target_hidden": hid, "request_key": 10_000 * (step + 1) + index}


def step_hiddens(w: Workload, step: int) -> np.ndarray:
    """Fresh target hidden states [B, 3d] for every request slot of a later step (N(0, 1), encoded):
    each step's hiddens come from a new target pass."""
    s = w.shape
    return _encode(_normal((w.seed, 700, step), (w.B, 3 * s.d_model)), s.dtype)


def catchup_inputs(w: Workload, R: int, step: int = 0) -> dict:
    """Inputs of a catch-up step: per request R token / hidden pairs and a real-row count.

    tokens [B, R] int32 uniform in [0, V); target_hidden [B, R, 3d] N(0, 1), encoded; n_real [B] uniform
    in 1..R with request 0 at R and (B > 1) request B - 1 at 1, so both ends are always present.
    """
    s = w.shape
    rng = _rng(w.seed, 800, step)
    tokens = rng.integers(0, s.vocab, size=(w.B, R)).astype(np.int32)
    n_real = rng.integers(1, R + 1, size=w.B).astype(np.int32)
    n_real[0] = R
    if w.B > 1:
        n_real[-1] = 1
    hid = _encode(_normal((w.seed, 801, step), (w.B, R, 3 * s.d_model)), s.dtype)
    return {"tokens": tokens, "target_hidden": hid, "n_real": n_real}
