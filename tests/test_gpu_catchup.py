"""GPU parity of the multi-row catch-up step (pe_draft_catchup) against the oracle's draft_step_catchup.

Request b runs n_real[b] real rows (an emitted token with the target hidden states that produced it) and
then placeholder rows, R + K rows in all, from position seq_len[b]; its K drafts come from rows
n_real[b] - 1 .. n_real[b] + K - 2. Per request: draft logits within the row-relative tolerance, draft
tokens identical up to the top-2-gap exemption, and the K/V of all R + K rows per (position, kv head), as
in every other draft test, within the K/V tolerance of tests/gpu_util.py (derived there from the bf16
drafter's rounding points; the 15-row case here is the one that sets it: the rounding-point oracle alone
reaches 1.76e-2 per head at its last layer).
Row counts cover the small-batch kernels, the weight-stream kernel (the row build too) and the 128 x 128
tiled kernel; n_real mixes 1 (a plain step) and R (a fully accepted previous step).
"""

import numpy as np
import pytest

from oracle import pe_oracle as O
from synth import QWEN3_CODER, TINY_FP32, Workload
from synth.device import to_device
from synth.inputs import catchup_inputs, kv_block, to_f64
from tests.gpu_util import KV_TOL, TOL, GpuDrafter, check_logits, check_rows, check_tokens, log, shape_weights64

pytestmark = pytest.mark.gpu


def _gpu_catchup(g, K, R, inp):
    torch = g.torch
    s = g.w.shape
    B = g.w.B
    draft = torch.full((B, K), -1, dtype=torch.int32, device="cuda")
    z = torch.empty((B, K, s.vocab), dtype=torch.float32, device="cuda")
    g.pe.pe_draft_catchup(g.ctx, B, K, R, g.d["req_slot"], g.d["seq_len"], to_device(inp["n_real"], "i32"),
                          to_device(inp["tokens"], "i32"), to_device(inp["target_hidden"], s.dtype), draft, z)
    torch.cuda.synchronize()
    return draft.cpu().numpy(), z.cpu().numpy()


def _oracle_catchup(w, W64, state, K, inp, req):
    seq = state["seq_len"][req]

    def ctx(l, i):
        b, L = req[i], int(seq[i])
        return (to_f64(kv_block(w, l, 0, b, L), w.shape.dtype), to_f64(kv_block(w, l, 1, b, L), w.shape.dtype))

    st = {"tokens": inp["tokens"][req], "target_hidden": to_f64(inp["target_hidden"][req], w.shape.dtype),
          "n_real": inp["n_real"][req], "seq_len": seq}
    return O.draft_step_catchup(w.shape, W64, st, ctx, K)


def _check_kv(g, ref, req, rows, tol):
    """Every layer's K and V rows of the sampled requests, row-relative per (position, kv head)."""
    err = 0.0
    for l in range(g.w.shape.n_layers):
        for i, b in enumerate(req):
            k, v = g.kv_rows(l, b, rows)  # [rows, Hkv, hd]
            err = max(err, check_rows(k, ref["k_new"][l][i], tol, f"{g.w.name} K rows l{l} b{b}"),
                      check_rows(v, ref["v_new"][l][i], tol, f"{g.w.name} V rows l{l} b{b}"))
    return err


CASES = [  # B, K, R: layer rows B (R + K), LM-head rows B K
    (1, 3, 4),    # 7 / 3: small-batch kernels, a fully accepted previous step
    (4, 3, 4),    # 28 / 12: layers on the weight-stream kernel, LM head on the stream kernel
    (3, 2, 1),    # 9 / 6: R = 1, the plain step's shape
    (8, 7, 8),    # 120 / 56: the row build itself (64 rows) on the stream kernel
    (20, 3, 4),   # 140 / 60: layers on the 128 x 128 tiled kernel
]


@pytest.mark.parametrize("B,K,R", CASES, ids=lambda v: str(v))
def test_catchup_parity(B, K, R):
    w = Workload(f"qwen3coder-bf16-B{B}-K{K}-R{R}-catchup", QWEN3_CODER, B, K, (60, 400), 0.7, 7800 + 40 * B + K + R)
    log(f"catch-up parity B {B} K {K} R {R}")
    tol = TOL[w.shape.dtype]
    g = GpuDrafter(w, max_k=R + K - 1)
    try:
        inp = catchup_inputs(w, R)
        log(f"  n_real {inp['n_real'].tolist()[:12]}")
        draft, z = _gpu_catchup(g, K, R, inp)
        req = list(range(B)) if B <= 4 else sorted({0, 1, B // 2, B - 1})
        ref = _oracle_catchup(w, shape_weights64(w.shape), g.state, K, inp, req)
        err = check_logits(z[req], ref["logits"], tol, w.name)
        strict, exempt = check_tokens(draft[req], ref["logits"], tol, w.name)
        kv_err = _check_kv(g, ref, req, R + K, KV_TOL[w.shape.dtype])
        log(f"  logit err {err:.2e}, kv err {kv_err:.2e}, tokens strict {strict}/{len(req) * K}, exempt {exempt}")
    finally:
        g.close()


@pytest.mark.parametrize("name,R", [("qwen3coder-bf16-B1-K3-L2048", 4), ("qwen3coder-bf16-B32-K7-L512to4096-churn", 8)])
def test_catchup_parity_bench_workloads(name, R):
    """The bench's catch-up configurations at full size: the headline request (context 2048, R = K + 1)
    and the 32-request batch (contexts up to 4096, 15 rows per request) on sampled requests."""
    from synth import WORKLOADS
    w = WORKLOADS[name]
    K = w.K
    log(f"catch-up parity at full size {name} R {R}")
    tol = TOL[w.shape.dtype]
    g = GpuDrafter(w, max_k=R + K - 1)
    try:
        inp = catchup_inputs(w, R)
        draft, z = _gpu_catchup(g, K, R, inp)
        req = [0] if w.B == 1 else [0, 13, w.B - 1]
        ref = _oracle_catchup(w, shape_weights64(w.shape), g.state, K, inp, req)
        err = check_logits(z[req], ref["logits"], tol, w.name)
        strict, exempt = check_tokens(draft[req], ref["logits"], tol, w.name)
        kv_err = _check_kv(g, ref, req, R + K, KV_TOL[w.shape.dtype])
        log(f"  n_real {inp['n_real'][req].tolist()}, logit err {err:.2e}, kv err {kv_err:.2e}, "
            f"tokens strict {strict}/{len(req) * K}, exempt {exempt}")
    finally:
        g.close()


def test_catchup_with_one_real_row_is_the_plain_step():
    # R = 1: the same rows, plans and kernels as pe_draft_step, so the results are bit-identical
    w = Workload("qwen3coder-bf16-B5-K3-catchup-plain", QWEN3_CODER, 5, 3, (60, 400), 0.7, 7900)
    g = GpuDrafter(w)
    try:
        inp = {"tokens": g.state["last_token"][:, None].astype(np.int32),
               "target_hidden": g.state["target_hidden"][:, None, :], "n_real": np.ones(w.B, dtype=np.int32)}
        d_c, z_c = _gpu_catchup(g, w.K, 1, inp)
        k_c = g.kc[0].clone()
        d_p, z_p = g.draft()
        assert np.array_equal(d_c, d_p.cpu().numpy())
        assert np.array_equal(z_c, z_p.cpu().numpy())
        assert g.torch.equal(k_c, g.kc[0])
    finally:
        g.close()


def test_catchup_rejects_bad_sizes_and_fp32():
    w = Workload("qwen3coder-bf16-B2-K3-catchup-args", QWEN3_CODER, 2, 3, (60, 100), 0.7, 7901)
    g = GpuDrafter(w, max_k=5)
    try:
        inp = catchup_inputs(w, 3)
        with pytest.raises(g.pe.PeError) as e:
            _gpu_catchup(g, 3, 4, catchup_inputs(w, 4))  # R + K = 7 > max_k + 1
        assert e.value.status == g.pe.PE_ERR_INVALID
        with pytest.raises(g.pe.PeError) as e:
            _gpu_catchup(g, 3, 0, inp)
        assert e.value.status == g.pe.PE_ERR_INVALID
    finally:
        g.close()
    wf = Workload("tiny-fp32-B1-K2-catchup", TINY_FP32, 1, 2, (10, 20), 0.7, 7902)
    gf = GpuDrafter(wf, max_k=3)
    try:
        with pytest.raises(gf.pe.PeError) as e:
            _gpu_catchup(gf, 2, 2, catchup_inputs(wf, 2))
        assert e.value.status == gf.pe.PE_ERR_UNSUPPORTED
    finally:
        gf.close()
