"""GPU parity of the draft step with FP8 drafter weights (weight_fp8 = 1) against the oracle's draft step on
the same weights quantized per output row (oracle.weights_fp8: E4M3 codes of w / s_n, s_n = max |w| / 448,
both sides deciding the codes in float32).

Per request: logits within the row-relative tolerance, draft tokens identical up to the top-2-gap
exemption, and the K/V of the K draft rows within the same tolerance. FP8 weights run on the small-batch
kernel (up to 16 rows: the headline request, 4 requests at K = 3, one request at K = 11), on the
weight-stream kernel (17-128 rows: B 4 K 7, B 8 K 11) and on the 128 x 128 tiled kernel (B 32 K 7).
"""

import numpy as np
import pytest

from oracle import pe_oracle as O
from synth import QWEN3_CODER, WORKLOADS, Workload
from tests.gpu_util import KV_TOL, TOL, GpuDrafter, check_logits, check_rows, check_tokens, log, oracle_draft, shape_weights64

pytestmark = pytest.mark.gpu

_W8 = {}


def _weights_fp8(shape):
    if shape.name not in _W8:
        _W8.clear()
        _W8[shape.name] = O.weights_fp8(shape, shape_weights64(shape))
    return _W8[shape.name]


@pytest.mark.parametrize("name", ["qwen3coder-bf16-B1-K3-L2048", "qwen3coder-bf16-B4-K3-L1024to4096",
                                  "qwen3coder-bf16-B1-K11-L1024to4096"])
def test_fp8_weights_parity(name):
    w = WORKLOADS[name]
    log(f"FP8 weights parity {name}")
    tol = TOL[w.shape.dtype]
    g = GpuDrafter(w, cfg_extra={"weight_fp8": 1})
    try:
        draft, z = g.draft()
        draft, z = draft.cpu().numpy(), z.cpu().numpy()
        req = list(range(w.B))
        W8 = _weights_fp8(w.shape)
        st = dict(g.state)
        ref = oracle_draft(w, W8, st, w.K, req)
        err = check_logits(z[req], ref["logits"], tol, w.name)
        strict, exempt = check_tokens(draft[req], ref["logits"], tol, w.name)
        kv_err = 0.0
        for l in range(w.shape.n_layers):
            for i, b in enumerate(req):
                k, v = g.kv_rows(l, b, w.K)
                kv_err = max(kv_err, check_rows(k, ref["k_new"][l][i], KV_TOL[w.shape.dtype], f"{w.name} K rows l{l} b{b}"),
                             check_rows(v, ref["v_new"][l][i], KV_TOL[w.shape.dtype], f"{w.name} V rows l{l} b{b}"))
        # the quantization is visible: the bf16 oracle differs from the FP8 one by more than rounding
        d_bf16 = oracle_draft(w, shape_weights64(w.shape), st, w.K, req[:1])["logits"][0]
        rel_q = np.abs(d_bf16 - ref["logits"][0]).max() / np.abs(ref["logits"][0]).max()
        log(f"  logit err {err:.2e}, kv err {kv_err:.2e}, tokens strict {strict}/{len(req) * w.K}, exempt {exempt}; "
            f"bf16 vs fp8 oracle {rel_q:.2e}")
    finally:
        g.close()


@pytest.mark.parametrize("name", ["qwen3coder-bf16-B4-K7-L1024to4096", "qwen3coder-bf16-B8-K11-L1024to4096"])
def test_fp8_weights_parity_stream_kernel(name):
    """17-128 rows per projection: FP8 codes through the weight-stream kernel (K-split partials scaled
    before the reduce); sampled requests."""
    w = WORKLOADS[name]
    log(f"FP8 weights parity (weight-stream kernel) {name}")
    tol = TOL[w.shape.dtype]
    g = GpuDrafter(w, cfg_extra={"weight_fp8": 1})
    try:
        draft, z = g.draft()
        draft, z = draft.cpu().numpy(), z.cpu().numpy()
        req = [0, w.B - 1]
        ref = oracle_draft(w, _weights_fp8(w.shape), dict(g.state), w.K, req)
        err = check_logits(z[req], ref["logits"], tol, w.name)
        strict, exempt = check_tokens(draft[req], ref["logits"], tol, w.name)
        kv_err = 0.0
        for l in range(w.shape.n_layers):
            for i, b in enumerate(req):
                k, v = g.kv_rows(l, b, w.K)
                kv_err = max(kv_err, check_rows(k, ref["k_new"][l][i], KV_TOL[w.shape.dtype], f"{w.name} K rows l{l} b{b}"),
                             check_rows(v, ref["v_new"][l][i], KV_TOL[w.shape.dtype], f"{w.name} V rows l{l} b{b}"))
        log(f"  logit err {err:.2e}, kv err {kv_err:.2e}, tokens strict {strict}/{len(req) * w.K}, exempt {exempt}")
    finally:
        g.close()


def test_fp8_weights_parity_tiled_kernel():
    """More than 128 rows per projection: FP8 codes through the 128 x 128 tiled kernel (32 requests at
    K = 7: 256 layer rows, a 224-row vocabulary projection; K-split partials scaled before the reduce);
    sampled requests."""
    w = WORKLOADS["qwen3coder-bf16-B32-K7-L512to4096-churn"]
    log(f"FP8 weights parity (tiled kernel) {w.name}")
    tol = TOL[w.shape.dtype]
    g = GpuDrafter(w, cfg_extra={"weight_fp8": 1})
    try:
        draft, z = g.draft()
        draft, z = draft.cpu().numpy(), z.cpu().numpy()
        req = [0, 17, w.B - 1]
        ref = oracle_draft(w, _weights_fp8(w.shape), dict(g.state), w.K, req)
        err = check_logits(z[req], ref["logits"], tol, w.name)
        strict, exempt = check_tokens(draft[req], ref["logits"], tol, w.name)
        kv_err = 0.0
        for l in range(w.shape.n_layers):
            for i, b in enumerate(req):
                k, v = g.kv_rows(l, b, w.K)
                kv_err = max(kv_err, check_rows(k, ref["k_new"][l][i], KV_TOL[w.shape.dtype], f"{w.name} K rows l{l} b{b}"),
                             check_rows(v, ref["v_new"][l][i], KV_TOL[w.shape.dtype], f"{w.name} V rows l{l} b{b}"))
        log(f"  logit err {err:.2e}, kv err {kv_err:.2e}, tokens strict {strict}/{len(req) * w.K}, exempt {exempt}")
    finally:
        g.close()


def test_fp8_weights_catchup_and_autoregressive():
    """The other entry points on an FP8 ctx: a catch-up step (R = 4 real-row slots, 7 rows per request)
    and autoregressive drafting (one row per pass), against the oracle on the quantized weights."""
    from synth.device import to_device
    from synth.inputs import catchup_inputs, kv_block, to_f64
    w = Workload("qwen3coder-bf16-B2-K3-fp8-entry", QWEN3_CODER, 2, 3, (200, 900), 0.7, 8310)
    tol = TOL[w.shape.dtype]
    K, R = 3, 4
    g = GpuDrafter(w, max_k=R + K - 1, cfg_extra={"weight_fp8": 1})
    torch = g.torch
    W8 = _weights_fp8(w.shape)
    st = g.state
    req = [0, 1]

    def ctx(l, i):
        L = int(st["seq_len"][i])
        return (to_f64(kv_block(w, l, 0, i, L), w.shape.dtype), to_f64(kv_block(w, l, 1, i, L), w.shape.dtype))

    try:
        inp = catchup_inputs(w, R)
        draft = torch.full((w.B, K), -1, dtype=torch.int32, device="cuda")
        z = torch.empty((w.B, K, w.shape.vocab), dtype=torch.float32, device="cuda")
        g.pe.pe_draft_catchup(g.ctx, w.B, K, R, g.d["req_slot"], g.d["seq_len"], to_device(inp["n_real"], "i32"),
                              to_device(inp["tokens"], "i32"), to_device(inp["target_hidden"], w.shape.dtype), draft, z)
        torch.cuda.synchronize()
        ref = O.draft_step_catchup(w.shape, W8, {"tokens": inp["tokens"], "n_real": inp["n_real"],
                                                 "target_hidden": to_f64(inp["target_hidden"], w.shape.dtype),
                                                 "seq_len": st["seq_len"]}, ctx, K)
        err = check_logits(z.cpu().numpy(), ref["logits"], tol, "fp8 catch-up")
        check_tokens(draft.cpu().numpy(), ref["logits"], tol, "fp8 catch-up")
        log(f"  fp8 catch-up: logit err {err:.2e}")

        draft.fill_(-1)
        g.pe.pe_draft_ar(g.ctx, w.B, K, g.d["req_slot"], g.d["seq_len"], g.d["last_token"], g.d["target_hidden"],
                         draft, z)
        torch.cuda.synchronize()
        d_ar = draft.cpu().numpy()
        ref = O.draft_autoregressive(w.shape, W8, {"last_token": st["last_token"], "seq_len": st["seq_len"],
                                                   "target_hidden": to_f64(st["target_hidden"], w.shape.dtype)},
                                     ctx, K, feed=d_ar)
        for i in range(K):
            err = check_logits(z.cpu().numpy()[:, i], ref["logits"][:, i], tol, f"fp8 autoregressive pass {i}")
            check_tokens(d_ar[:, i], ref["logits"][:, i], tol, f"fp8 autoregressive pass {i}")
        log(f"  fp8 autoregressive: last pass logit err {err:.2e}")
    finally:
        g.close()
