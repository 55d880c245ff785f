"""Helpers of the GPU parity tests: run the HIP path through the C ABI and compare with the oracle.

Tolerances: per-row relative logit error max_v |gpu - oracle| / max_v |oracle| <= 1e-4 for the fp32
drafter and 2e-2 for bf16 (fixed by the target of this path); draft tokens identical except where the
oracle's top-2 logit gap is below tol * max_v |oracle|, in which case the GPU's token must be within that
margin of the oracle's maximum. Verify and compaction outputs are integers: bit-exact.

K/V rows appended to the cache are checked per (position, kv head), the same row-relative measure over
hd values. Their tolerance is not fixed by the target (it names logits); KV_TOL derives it from the bf16
drafter's arithmetic: oracle.bf16_rounding_budget runs the oracle with bf16 rounding at exactly the points
where the kernels round (normalised operands, queries, cache keys and values, softmax weights, attention and
SwiGLU outputs; float64 elsewhere) and finds per-head K/V differences from the plain oracle of up to
1.76e-2 at the last layer of a 15-row catch-up step (1.3e-2 at layer 2), against 1.16e-2 for its logits.
The kernels add their own float32 accumulation orders and rounding realisations to that, so K/V rows get
2.5e-2 (bf16) and logits keep 2e-2; the fp32 drafter keeps 1e-4 for both.
"""

from __future__ import annotations

import sys
import time

import numpy as np

from oracle import pe_oracle as O
from synth import make_state
from synth.device import config_args, to_device, upload_kv, upload_state, upload_weights
from synth.inputs import kv_block, to_f64

TOL = {"f32": 1e-4, "bf16": 2e-2}
KV_TOL = {"f32": 1e-4, "bf16": 2.5e-2}


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


_WEIGHTS = {}
_W64 = {}


def shape_weights(s):
    """Device (and host) tensors of drafter s; one drafter stays resident at a time."""
    if s.name not in _WEIGHTS:
        _WEIGHTS.clear()
        log(f"upload weights of {s.name}")
        _WEIGHTS[s.name] = upload_weights(s, keep_host=True)
    return _WEIGHTS[s.name]


def shape_weights64(s):
    if s.name not in _W64:
        _W64.clear()
        _W64[s.name] = {k: to_f64(v, s.dtype) for k, v in shape_weights(s)[1].items()}
    return _W64[s.name]


class GpuDrafter:
    """One workload's synthetic inputs on the GPU plus an initialised pe ctx."""

    def __init__(self, w, state=None, max_batch=None, max_k=None, cfg_extra=None):
        import torch
        import eagle_drafting_amd as pe
        self.torch, self.pe, self.w = torch, pe, w
        s = w.shape
        self.dev, self.host = shape_weights(s)
        self.state = state if state is not None else make_state(w)
        log("upload kv")
        self.kc, self.vc = upload_kv(w, self.state)
        self.d = upload_state(self.state, s.dtype)
        self.cfg = pe.make_config(**{**config_args(w, max_batch, max_k), **(cfg_extra or {})})
        self.stream = torch.cuda.current_stream().cuda_stream
        self.ctx = pe.pe_init(self.cfg, pe.make_weights(self.dev, s.n_layers), pe.make_kv(self.kc, self.vc),
                              self.stream)
        log("ctx ready")

    def draft(self, K=None, B=None, logits=True, rows=None, dstate=None):
        torch = self.torch
        K = K or self.w.K
        d = dstate or self.d
        B = B or int(d["req_slot"].shape[0])
        draft = torch.empty((B, K), dtype=torch.int32, device="cuda")
        z = torch.empty((B, K, self.w.shape.vocab), dtype=torch.float32, device="cuda") if logits else None
        if rows is None:
            self.pe.pe_draft_step(self.ctx, B, K, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"],
                                  draft, z)
        else:
            self.pe.pe_draft_rows(self.ctx, B, K, d["req_slot"], d["seq_len"], rows, draft, z)
        torch.cuda.synchronize()
        return draft, z

    def kv_rows(self, layer, b, K):
        """This step's K and V rows of request b in layer `layer` as float64 [K, Hkv, hd]."""
        L = int(self.state["seq_len"][b])
        slot = int(self.state["req_slot"][b])
        k = self.kc[layer][slot, :, L:L + K, :].float().cpu().numpy().transpose(1, 0, 2)
        v = self.vc[layer][slot, :, L:L + K, :].float().cpu().numpy().transpose(1, 0, 2)
        return k.astype(np.float64), v.astype(np.float64)

    def close(self):
        if self.ctx is not None:
            ctx, self.ctx = self.ctx, None
            self.pe.pe_destroy(ctx)


def oracle_draft(w, W64, state, K, requests, rows=None):
    """The oracle's draft step for a subset of requests (requests are independent)."""
    req = list(requests)
    seq = state["seq_len"][req]

    def ctx(l, i):
        b = req[i]
        L = int(seq[i])
        return (to_f64(kv_block(w, l, 0, b, L), w.shape.dtype), to_f64(kv_block(w, l, 1, b, L), w.shape.dtype))

    if rows is not None:
        return O.draft_rows(w.shape, W64, rows, seq, ctx)
    st = {"last_token": state["last_token"][req],
          "target_hidden": to_f64(state["target_hidden"][req], w.shape.dtype), "seq_len": seq}
    return O.draft_step(w.shape, W64, st, ctx, K)


def check_logits(gpu, ref, tol, what=""):
    gpu = np.asarray(gpu, dtype=np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    scale = np.abs(ref).max(-1)
    rel = np.abs(gpu - ref).max(-1) / scale
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU logits"
    assert rel.max() <= tol, f"{what}: max row-relative logit error {rel.max():.3e} > {tol} (row {rel.argmax()})"
    return float(rel.max())


def check_rows(gpu, ref, tol, what=""):
    """Row-relative check for activations / KV rows [..., n]."""
    return check_logits(gpu, ref, tol, what)


def check_tokens(gpu_tok, ref_logits, tol, what=""):
    """Draft tokens: identical, except where the oracle's top-2 gap is under tol * max|logit|; there the
    GPU token must score within that margin of the oracle maximum. Returns (strict matches, exempt rows)."""
    ref = np.asarray(ref_logits, dtype=np.float64).reshape(-1, ref_logits.shape[-1])
    tok = np.asarray(gpu_tok).reshape(-1)
    scale = np.abs(ref).max(-1)
    ref_tok = O.argmax_first(ref)
    srt = np.sort(ref, axis=-1)
    gap = srt[:, -1] - srt[:, -2]
    exempt = gap < tol * scale
    strict_bad = (~exempt) & (tok != ref_tok)
    assert not strict_bad.any(), f"{what}: draft token differs at rows {np.nonzero(strict_bad)[0][:8]}"
    margin_ok = ref[np.arange(ref.shape[0]), tok] >= srt[:, -1] - tol * scale
    assert margin_ok.all(), f"{what}: exempt-row token outside the margin at rows {np.nonzero(~margin_ok)[0][:8]}"
    return int((tok == ref_tok).sum()), int(exempt.sum())


def run_verify(pe, ctx, B, K, T_dev, draft_dev, finished_dev, slot_dev, seq_dev):
    import torch
    i32 = dict(dtype=torch.int32, device="cuda")
    out = {"accept_len": torch.full((B,), -7, **i32), "cu_accept": torch.full((B + 1,), -7, **i32),
           "out_tokens": torch.full((B * (K + 1),), -7, **i32), "keep_index": torch.full((B,), -7, **i32),
           "n_keep": torch.full((1,), -7, **i32), "req_slot_next": torch.full((B,), -7, **i32),
           "seq_len_next": torch.full((B,), -7, **i32), "last_token_next": torch.full((B,), -7, **i32)}
    pe.pe_verify(ctx, B, K, T_dev, draft_dev, finished_dev, slot_dev, seq_dev, out["accept_len"], out["cu_accept"],
                 out["out_tokens"], out["keep_index"], out["n_keep"], out["req_slot_next"], out["seq_len_next"],
                 out["last_token_next"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def check_verify(got, T_host_exact, draft, finished, req_slot, seq_len):
    """Bit-exact comparison of pe_verify's outputs with the oracle's verify + compact."""
    v = O.verify(T_host_exact, draft)
    c = O.compact(v, req_slot, seq_len, finished)
    B = draft.shape[0]
    n_keep = c["n_keep"]
    tot = int(c["cu_accept"][B])
    assert np.array_equal(got["accept_len"], v["accept_len"])
    assert np.array_equal(got["cu_accept"], c["cu_accept"])
    assert np.array_equal(got["out_tokens"][:tot], c["out_tokens"])
    assert int(got["n_keep"][0]) == n_keep
    assert np.array_equal(got["keep_index"][:n_keep], c["keep_index"])
    assert np.array_equal(got["req_slot_next"][:n_keep], c["req_slot_next"])
    assert np.array_equal(got["seq_len_next"][:n_keep], c["seq_len_next"])
    assert np.array_equal(got["last_token_next"][:n_keep], c["last_token_next"])
    return v, c


__all__ = ["TOL", "KV_TOL", "log", "GpuDrafter", "shape_weights", "shape_weights64", "oracle_draft", "check_logits", "check_rows",
           "check_tokens", "run_verify", "check_verify", "to_device"]
