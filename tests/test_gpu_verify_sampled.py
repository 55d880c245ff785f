"""GPU parity of pe_verify_sampled (temperature > 0) against the oracle's verify_sampled.

Inputs: the harness's draft tokens, planted target logits, and seeded uniforms. The oracle decides in
float64 and the kernels in float32, so a decision whose float64 margin is below the float32 error bound
of the kernels' arithmetic is not fixed by the definition alone. That bound, relative to the quantity it
bounds, is derived from how the kernels compute (unit roundoff 2^-24):

  * each weight exp(x / tau - m): the product x * (1 / tau) rounds once, an error of at most A ulp in the
    exponent with A = max |x| / tau over the row; the subtraction and the exponential's own scaling give
    at most |x / tau - m| ulp more and the hardware exp2 two more. Summed over a row, the |x / tau - m|
    parts weigh sum_t w_t |log w_t| <= 2 S ln V (w_t <= 1, S = sum w_t), so a total S or a weight carries
    at most (A + 4 ln V + 2) ulp from the exponentials;
  * each lane's running sum over its ~32 elements of a 2048-token chunk (an add per element and, per
    batch of 32 elements, a rescale by one multiply: at most three roundings per element), then at most
    20 pairwise merges (shuffles, waves, chunks; three roundings each): 3 (32 + 20) ulp;
  * the acceptance test u < ed / S divides two such quantities: p carries at most twice the above;
  * a draw compares its threshold v (S - ed) with a running total over up to nchunks chunk totals (one
    rounding each) and a 256-thread block scan inside the chunk (~40 roundings).

The tests take twice that bound: an acceptance uniform within w_acc * p of p_i(draft) is redrawn (about
3e-5 * p to 5e-5 * p here, against the former 1e-3 absolute), and a draw passes if it is the token an exact
inverse-CDF draw picks for a threshold within w_draw * total of the given one (about 5e-5 of the row's
mass). The accepted drafts, accept_len and all integer metadata must then match exactly, and a drawn token
must carry weight (never the rejected draft). test_sampled_verify_near_boundaries places uniforms at 1.5
times these windows on either side of a decision, so decisions next to their boundary are exercised.
"""

import numpy as np
import pytest

from oracle import pe_oracle as O
from synth import WORKLOADS, make_state, plant_target_logits, random_draft, churn_finished
from synth.inputs import bf16_bits_to_f32
from tests.gpu_util import log, to_device
from tests.test_gpu_verify import VerifyCtx

pytestmark = pytest.mark.gpu

ULP = 2.0 ** -24


def _window_acc(row, tau):
    """Twice the float32 bound on the relative error of p(x) for one target row (docstring)."""
    A = float(np.abs(row).max()) / tau
    return 2.0 * (2 * A + 8 * np.log(row.shape[-1]) + 3 * (32 + 20) + 10) * ULP


def _window_draw(row, tau):
    """Twice the float32 bound on a draw's threshold and running totals, relative to the row's mass."""
    V = row.shape[-1]
    nchunks = -(-V // 2048)  # the kernels' ~2048-token chunks
    A = float(np.abs(row).max()) / tau
    return 2.0 * (2 * A + 8 * np.log(V) + 3 * (32 + 20) + nchunks + 40) * ULP


def _exact(T, dtype):
    return T if dtype == "f32" else bf16_bits_to_f32(T)


def _uniforms(T, draft, tau, seed):
    """u [B, K] outside the float32 window around every p_i(draft), v [B, K+1]."""
    rng = np.random.default_rng(seed)
    B, K = draft.shape
    u = rng.random((B, K))
    for b in range(B):
        for i in range(K):
            p = O.softmax_temperature(T[b, i], tau)[draft[b, i]]
            w = _window_acc(T[b, i], tau) * p
            while abs(float(np.float32(u[b, i])) - p) <= w:
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
        tol = _window_draw(T[b, n], tau) * c[-1]
        assert 0 <= x < w.shape[0] and w[x] > 0.0, f"request {b}: drew a token without weight ({x})"
        lo = c[x - 1] if x > 0 else 0.0
        assert lo <= theta + tol and c[x] > theta - tol, \
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
    return ref, c


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
    ref, _ = _check(got, T_exact, draft, tau, u, v, fin, st["req_slot"], st["seq_len"])
    log(f"  mean accept_len {ref['accept_len'].mean():.3f}")


@pytest.mark.parametrize("V,dtype", [(4096, "f32"), (151936, "bf16")])
def test_sampled_verify_near_boundaries(V, dtype):
    """Decisions placed just outside the float32 window (1.5 times the doubled bound) on either side of
    their boundary. Request b accepts its drafts before position b % (K + 1) with u just below p_i(draft),
    rejects there with u just above it (or, at K, makes the bonus draw); the draw's threshold sits just
    past the start of a chosen token's bin (even b) or just short of its end (odd b). Every decision is
    then fixed by the definition, and the GPU must take it: accept_len, the accepted drafts and the drawn
    token exactly."""
    rng = np.random.default_rng(91 + V)
    B, K, tau = 8, 3, 0.3
    T = rng.standard_normal((B, K + 1, V)).astype(np.float32) * 2.0
    if dtype == "bf16":
        from synth.inputs import bf16_bits
        T_dev_host = bf16_bits(T)
        T = bf16_bits_to_f32(T_dev_host)
    else:
        T_dev_host = T
    draft = np.empty((B, K), dtype=np.int32)
    u = np.empty((B, K), dtype=np.float64)
    v = rng.random((B, K + 1))
    want_tok = np.empty(B, dtype=np.int64)
    for b in range(B):
        n = b % (K + 1)
        for i in range(K):
            p = O.softmax_temperature(T[b, i], tau)
            # a draft with enough mass that u = p (1 +- 1.5 w) stays inside (0, 1)
            draft[b, i] = int(np.argsort(p)[-2 - (b + i) % 3])
            w = 1.5 * _window_acc(T[b, i], tau)
            u[b, i] = p[draft[b, i]] * (1.0 - w) if i < n else p[draft[b, i]] * (1.0 + w)
            assert 0.0 < u[b, i] < 1.0
        # the draw at position n: weights without the rejected draft (n < K) or p_K itself
        wts = O.softmax_temperature(T[b, n], tau)
        if n < K:
            wts[draft[b, n]] = 0.0
        c = np.cumsum(wts)
        tot = c[-1]
        tol = 1.5 * _window_draw(T[b, n], tau) * tot
        heavy = [int(o) for o in np.argsort(wts)[::-1][:6] if wts[o] > 4 * tol]
        x = heavy[b % len(heavy)]  # a heavy token, not always the heaviest
        lo = c[x - 1] if x > 0 else 0.0
        theta = lo + tol if b % 2 == 0 else c[x] - tol
        v[b, n] = theta / tot
        want_tok[b] = x
    u32, v32 = u.astype(np.float32), v.astype(np.float32)
    # the float32 uniforms keep every decision on its side (their rounding is far inside the windows)
    ref = O.verify_sampled(T, draft, tau, u32.astype(np.float64), v32.astype(np.float64))
    assert np.array_equal(ref["n"], np.arange(B) % (K + 1))
    assert np.array_equal(ref["bonus"], want_tok)
    slot = np.arange(B, dtype=np.int32)
    seq = np.full(B, 100, dtype=np.int32)
    ctx = VerifyCtx(V, dtype, B, K)
    try:
        got = _run(ctx.pe, ctx.ctx, to_device(T_dev_host, dtype), draft, tau, u32, v32, None, slot, seq)
    finally:
        ctx.close()
    assert np.array_equal(got["accept_len"], ref["accept_len"])
    cu = got["cu_accept"]
    for b in range(B):
        n = int(ref["n"][b])
        toks = got["out_tokens"][cu[b]:cu[b + 1]]
        assert np.array_equal(toks[:n], draft[b, :n])
        assert int(toks[n]) == want_tok[b], (b, int(toks[n]), want_tok[b])
    _check(got, T, draft, tau, u32, v32, None, slot, seq)


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


def test_sampled_verify_gpu_emits_the_target_distribution():
    # the defining property on the GPU itself: 1024 requests share one target row and one draft (not the
    # argmax), each with its own uniforms; over 20 calls the first emitted token follows
    # p_0 = softmax(T_0 / temperature) and the draft is accepted at rate p_0(draft) (5 sigma)
    from scipy.special import softmax
    B, K, V, tau = 1024, 1, 16, 0.8
    rng = np.random.default_rng(77)
    row = rng.standard_normal((K + 1, V)).astype(np.float32) * 1.5
    T = np.broadcast_to(row, (B, K + 1, V)).copy()
    d0 = int(np.argsort(row[0])[-2])
    draft = np.full((B, K), d0, dtype=np.int32)
    ctx = VerifyCtx(V, "f32", B, K)
    counts, acc, N = np.zeros(V), 0, 0
    try:
        for it in range(20):
            u = rng.random((B, K)).astype(np.float32)
            v = rng.random((B, K + 1)).astype(np.float32)
            got = _run(ctx.pe, ctx.ctx, to_device(T, "f32"), draft, tau, u, v, None, np.arange(B, dtype=np.int32),
                       np.zeros(B, dtype=np.int32))
            first = got["out_tokens"][got["cu_accept"][:B]]
            np.add.at(counts, first, 1)
            acc += int((got["accept_len"] == 2).sum())
            N += B
    finally:
        ctx.close()
    p0 = softmax(row[0].astype(np.float64) / tau)
    sig = np.sqrt(p0 * (1 - p0) / N)
    assert np.all(np.abs(counts / N - p0) < 5 * sig + 1e-12), (counts / N, p0)
    assert abs(acc / N - p0[d0]) < 5 * np.sqrt(p0[d0] * (1 - p0[d0]) / N)


@pytest.mark.parametrize("case", ["k1", "all_finished", "largest_batch"])
def test_sampled_verify_edge_cases(case):
    rng = np.random.default_rng({"k1": 1, "all_finished": 2, "largest_batch": 3}[case])
    B, K, V, dtype = {"k1": (5, 1, 4096, "bf16"), "all_finished": (7, 3, 4096, "f32"),
                      "largest_batch": (1024, 2, 1024, "bf16")}[case]
    T = rng.standard_normal((B, K + 1, V)).astype(np.float32) * 3.0
    if dtype == "bf16":
        from synth.inputs import bf16_bits
        T_dev_host = bf16_bits(T)
        T = bf16_bits_to_f32(T_dev_host)
    else:
        T_dev_host = T
    draft = np.where(rng.random((B, K)) < 0.5, T[:, :K].argmax(-1), rng.integers(0, V, (B, K))).astype(np.int32)
    tau = 0.5
    u, v = _uniforms(T, draft, tau, 9)
    fin = np.ones(B, dtype=np.uint8) if case == "all_finished" else (rng.random(B) < 0.3).astype(np.uint8)
    slot = rng.permutation(B + 3)[:B].astype(np.int32)
    seq = rng.integers(0, 500, B).astype(np.int32)
    ctx = VerifyCtx(V, dtype, B, K)
    try:
        got = _run(ctx.pe, ctx.ctx, to_device(T_dev_host, dtype), draft, tau, u, v, fin, slot, seq)
    finally:
        ctx.close()
    _check(got, T, draft, tau, u, v, fin, slot, seq)
    if case == "all_finished":
        assert int(got["n_keep"][0]) == 0
