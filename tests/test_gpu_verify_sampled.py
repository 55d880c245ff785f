"""GPU parity of pe_verify_sampled (temperature > 0) against the oracle's verify_sampled.

Inputs: the harness's draft tokens, planted target logits, and seeded uniforms. The oracle decides in
float64 and the kernels in float32, so acceptance uniforms closer than 1e-3 to their decision boundary
p_i(draft) are redrawn (then every acceptance decision is fixed). The accepted drafts, accept_len and all
integer metadata must then match exactly. The draw after the accepted drafts must be a token that an exact
inverse-CDF draw picks for a threshold within 1e-4 of the total weight of the given one (the float32 sums
over up to 201088 weights differ from the float64 ones by far less), and must carry weight (never the
rejected draft).
"""

import numpy as np
import pytest

from oracle import pe_oracle as O
from synth import WORKLOADS, make_state, plant_target_logits, random_draft, churn_finished
from synth.inputs import bf16_bits_to_f32
from tests.gpu_util import log, to_device
from tests.test_gpu_verify import VerifyCtx

pytestmark = pytest.mark.gpu

TOL_DRAW = 1e-4


def _exact(T, dtype):
    return T if dtype == "f32" else bf16_bits_to_f32(T)


def _uniforms(T, draft, tau, seed):
    """u [B, K] away from every p_i(draft) by at least 1e-3, v [B, K+1]."""
    rng = np.random.default_rng(seed)
    B, K = draft.shape
    u = rng.random((B, K))
    for b in range(B):
        for i in range(K):
            p = O.softmax_temperature(T[b, i], tau)[draft[b, i]]
            while abs(u[b, i] - p) < 1e-3:
                u[b, i] = rng.random()
    v = rng.random((B, K + 1))
    return u.astype(np.float32), v.astype(np.float32)


def _run(pe, ctx, T_dev, draft, tau, u, v, finished, slot, seq):
    import torch
    B, K = draft.shape
    i32 = dict(dtype=torch.int32, device="cuda")
    out = {k: torch.full((n,), -7, **i32) for k, n in (("accept_len", B), ("cu_accept", B + 1),
                                                        ("out_tokens", B * (K + 1)), ("keep_index", B),
                                                        ("n_keep", 1), ("req_slot_next", B),
                                                        ("seq_len_next", B), ("last_token_next", B))}
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    pe.pe_verify_sampled(ctx, B, K, T_dev, to_device(draft, "i32"), tau, f32(u), f32(v),
                         None if finished is None else to_device(finished, "u8"), to_device(slot, "i32"),
                         to_device(seq, "i32"), out["accept_len"], out["cu_accept"], out["out_tokens"],
                         out["keep_index"], out["n_keep"], out["req_slot_next"], out["seq_len_next"],
                         out["last_token_next"])
    torch.cuda.synchronize()
    return {k: t.cpu().numpy() for k, t in out.items()}


def _check(got, T, draft, tau, u, v, finished, slot, seq):
    B, K = draft.shape
    ref = O.verify_sampled(T, draft, tau, u.astype(np.float64), v.astype(np.float64))
    assert np.array_equal(got["accept_len"], ref["accept_len"]), "accept_len differs"
    cu = got["cu_accept"]
    assert cu[0] == 0 and np.array_equal(np.diff(cu), ref["accept_len"]), "cu_accept differs"
    t_gpu = np.full((B, K + 1), -1, dtype=np.int64)
    for b in range(B):
        n = int(ref["n"][b])
        toks = got["out_tokens"][cu[b]:cu[b + 1]]
        assert np.array_equal(toks[:n], draft[b, :n]), f"request {b}: accepted drafts differ"
        x = int(toks[n])
        p = O.softmax_temperature(T[b, n], tau)
        w = p.copy()
        if n < K:
            w[draft[b, n]] = 0.0
        c = np.cumsum(w)
        theta = float(v[b, n]) * c[-1]
        lo = c[x - 1] if x > 0 else 0.0
        assert 0 <= x < w.shape[0] and w[x] > 0.0, f"request {b}: drew a token without weight ({x})"
        assert lo <= theta + TOL_DRAW * c[-1] and c[x] > theta - TOL_DRAW * c[-1], \
            f"request {b}: draw {x} inconsistent with the threshold (oracle {ref['t'][b, n]})"
        t_gpu[b, : n + 1] = toks
    mine = {"t": t_gpu, "accept_len": got["accept_len"], "bonus": t_gpu[np.arange(B), ref["n"]]}
    c = O.compact(mine, slot, seq, finished)
    nk = c["n_keep"]
    assert int(got["n_keep"][0]) == nk
    assert np.array_equal(got["keep_index"][:nk], c["keep_index"])
    assert np.array_equal(got["req_slot_next"][:nk], c["req_slot_next"])
    assert np.array_equal(got["seq_len_next"][:nk], c["seq_len_next"])
    assert np.array_equal(got["last_token_next"][:nk], c["last_token_next"])
    return ref


# at temperature 0.3 and above a planted token (row maximum + 1) holds little of the mass of a 150 k
# vocabulary, so most verifies stop at position 0; at 0.1 planted positions are almost always accepted,
# which exercises long accepted prefixes and the bonus draw
@pytest.mark.parametrize("name,tau", [("tiny-fp32-B1-K4-L64", 0.3), ("tiny-fp32-B1-K4-L64", 0.1),
                                      ("qwen3coder-bf16-B1-K3-L2048", 0.3), ("qwen3coder-bf16-B1-K3-L2048", 0.1),
                                      ("qwen3coder-bf16-B8-K7-L1024to4096", 0.7),
                                      ("qwen3coder-bf16-B8-K11-L1024to4096", 0.1),
                                      ("qwen3coder-bf16-B128-K7-L512to4096-churn", 0.3),
                                      ("gptoss20b-bf16-B64-K10-L2048to8192", 1.0)])
def test_sampled_verify_parity(name, tau):
    w = WORKLOADS[name]
    log(f"sampled verify parity {name} temperature {tau}")
    st = make_state(w)
    draft = random_draft(w)
    T = plant_target_logits(w, draft, st["alpha"])
    T_exact = _exact(T, w.shape.dtype)
    fin = churn_finished(w, 0) if w.churn else None
    u, v = _uniforms(T_exact, draft, tau, w.seed + 17)
    ctx = VerifyCtx(w.shape.vocab, w.shape.dtype, w.B, w.K)
    try:
        got = _run(ctx.pe, ctx.ctx, to_device(T, w.shape.dtype), draft, tau, u, v, fin, st["req_slot"], st["seq_len"])
    finally:
        ctx.close()
    ref = _check(got, T_exact, draft, tau, u, v, fin, st["req_slot"], st["seq_len"])
    log(f"  mean accept_len {ref['accept_len'].mean():.3f}")


def test_sampled_verify_rejects_bad_temperature():
    import eagle_drafting_amd as pe
    ctx = VerifyCtx(4096, "f32", 2, 2)
    try:
        rng = np.random.default_rng(5)
        T = rng.standard_normal((2, 3, 4096)).astype(np.float32)
        draft = rng.integers(0, 4096, size=(2, 2)).astype(np.int32)
        u, v = rng.random((2, 2)), rng.random((2, 3))
        for tau in (0.0, -1.0, float("nan")):
            with pytest.raises(pe.PeError) as e:
                _run(ctx.pe, ctx.ctx, to_device(T, "f32"), draft, tau, u, v, None, np.arange(2, dtype=np.int32),
                     np.zeros(2, dtype=np.int32))
            assert e.value.status == pe.PE_ERR_INVALID
    finally:
        ctx.close()
