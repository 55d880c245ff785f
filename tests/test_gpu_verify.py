"""GPU parity of pe_verify (greedy accept + batch-metadata rebuild) against the oracle: bit-exact.

Inputs are the harness's draft tokens and planted target logits, so these cases do not depend on the
drafter's numerics. Every named workload plus edge cases (K = 1, all-match, first-position mismatch,
ties, every request finished, the largest batch).
"""

import numpy as np
import pytest

from synth import WORKLOADS, Workload, DrafterShape, make_state, plant_target_logits, random_draft, churn_finished
from synth.inputs import bf16_bits, bf16_bits_to_f32
from tests.gpu_util import check_verify, log, run_verify, to_device

pytestmark = pytest.mark.gpu


class VerifyCtx:
    """A pe ctx whose drafter is minimal (1 layer, d = 32): only its vocab, dtype and capacity matter here."""

    def __init__(self, V, dtype, max_batch, max_k):
        import torch
        import eagle_drafting_amd as pe
        self.pe = pe
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        d, F, hd = 32, 32, 64
        z = lambda *shape: torch.zeros(shape, dtype=tdt, device="cuda")
        self.t = {"fc": z(d, 3 * d), "embed": z(V, d), "emb_mask": z(d), "h_shared": z(d), "final_norm": z(d),
                  "lm_head": z(V, d), "l0.attn_norm": z(d), "l0.wqkv": z(3 * hd, d), "l0.wo": z(d, hd),
                  "l0.mlp_norm": z(d), "l0.wgate": z(F, d), "l0.wup": z(F, d), "l0.wdown": z(d, F)}
        self.k, self.v = z(1, 1, max_k + 1, hd), z(1, 1, max_k + 1, hd)
        cfg = pe.make_config(1, d, 1, 1, hd, F, V, dtype, max_batch, max_k, max_k + 1, 1)
        self.ctx = pe.pe_init(cfg, pe.make_weights(self.t, 1), pe.make_kv([self.k], [self.v]),
                              torch.cuda.current_stream().cuda_stream)

    def close(self):
        self.pe.pe_destroy(self.ctx)


def _exact(T, dtype):
    return T if dtype == "f32" else bf16_bits_to_f32(T)


def _run_case(dtype, T, draft, finished, req_slot, seq_len, ctx=None):
    B, K1, V = T.shape
    K = K1 - 1
    own = ctx is None
    if own:
        ctx = VerifyCtx(V, dtype, B, K)
    try:
        got = run_verify(ctx.pe, ctx.ctx, B, K, to_device(T, dtype), to_device(draft, "i32"),
                         None if finished is None else to_device(finished, "u8"), to_device(req_slot, "i32"),
                         to_device(seq_len, "i32"))
        return check_verify(got, _exact(T, dtype), draft, finished, req_slot, seq_len)
    finally:
        if own:
            ctx.close()


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_verify_parity_workloads(name):
    w = WORKLOADS[name]
    log(f"verify parity {name}")
    st = make_state(w)
    draft = random_draft(w)
    T = plant_target_logits(w, draft, st["alpha"])
    fin = churn_finished(w, 0) if w.churn else None
    v, c = _run_case(w.shape.dtype, T, draft, fin, st["req_slot"], st["seq_len"])
    log(f"  mean accept_len {v['accept_len'].mean():.3f}, n_keep {c['n_keep']}")


def _small(B, K, V, dtype, seed):
    rng = np.random.default_rng(seed)
    T = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    if dtype == "bf16":
        T = bf16_bits_to_f32(bf16_bits(T))
    draft = rng.integers(0, V, size=(B, K)).astype(np.int32)
    slot = rng.permutation(B + 5)[:B].astype(np.int32)
    seq = rng.integers(0, 1000, size=B).astype(np.int32)
    return rng, T, draft, slot, seq


def _enc(T, dtype):
    return T if dtype == "f32" else bf16_bits(T)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_verify_edge_cases(dtype):
    V = 1000
    # K = 1, B = 1
    rng, T, draft, slot, seq = _small(1, 1, V, dtype, 1)
    _run_case(dtype, _enc(T, dtype), draft, None, slot, seq)
    # all match -> K + 1 accepted; first-position mismatch -> 1
    for K in (1, 4, 16):
        rng, T, draft, slot, seq = _small(6, K, V, dtype, 10 + K)
        draft[:3] = T[:3, :K].argmax(-1)
        draft[3:] = T[3:, :K].argmax(-1)
        draft[3:, 0] = (draft[3:, 0] + 1) % V
        v, _ = _run_case(dtype, _enc(T, dtype), draft, None, slot, seq)
        assert list(v["accept_len"]) == [K + 1] * 3 + [1] * 3
    # ties: the row maximum appears at several indices; the lowest wins on both sides
    rng, T, draft, slot, seq = _small(5, 3, V, dtype, 3)
    for b in range(5):
        for i in range(4):
            idx = np.sort(rng.choice(V, size=3, replace=False))
            T[b, i, idx] = 7.0
            if i < 3 and b % 2 == 0:
                draft[b, i] = idx[0]
    v, _ = _run_case(dtype, _enc(T, dtype), draft, None, slot, seq)
    assert all(v["accept_len"][b] == 4 for b in (0, 2, 4))
    # every request finished / none finished / alternating
    rng, T, draft, slot, seq = _small(9, 5, V, dtype, 4)
    for fin in (np.ones(9, np.uint8), np.zeros(9, np.uint8), (np.arange(9) % 2).astype(np.uint8)):
        _run_case(dtype, _enc(T, dtype), draft, fin, slot, seq)


def test_verify_largest_batch_and_depth():
    # B = 1024 (one thread per request in the scan), K = 16
    rng, T, draft, slot, seq = _small(1024, 16, 64, "bf16", 5)
    m = rng.random((1024, 16)) < 0.8
    t = T[:, :16].argmax(-1)
    draft[m] = t[m]
    fin = (rng.random(1024) < 0.1).astype(np.uint8)
    _run_case("bf16", bf16_bits(T), draft, fin, slot, seq)


def test_verify_reuses_ctx_and_sizes_vary():
    ctx = VerifyCtx(2048, "bf16", 64, 11)
    try:
        for i, (B, K) in enumerate(((64, 11), (1, 1), (17, 5), (64, 3))):
            rng, T, draft, slot, seq = _small(B, K, 2048, "bf16", 40 + i)
            m = rng.random((B, K)) < 0.7
            draft[m] = T[:, :K].argmax(-1)[m]
            _run_case("bf16", bf16_bits(T), draft, (rng.random(B) < 0.2).astype(np.uint8), slot, seq, ctx=ctx)
    finally:
        ctx.close()
