"""GPU parity of autoregressive drafting (pe_draft_ar) against the oracle's draft_autoregressive.

Autoregressive drafting is the sequential chain parallel drafting replaces: K passes of one row per
request, each feeding back the previous pass's hidden state and drafted token. The oracle follows the
GPU's token choices (feed), so every pass is compared on the same input even where a near-tie let the
GPU pick another token within the tolerance. Per pass: logits within the row-relative tolerance, the
drafted token identical up to the top-2-gap exemption; the K/V of all K + 1 positions (the K passes and
the trailing layers-only pass) within the same tolerance.
"""

import numpy as np
import pytest

from oracle import pe_oracle as O
from synth import QWEN3_CODER, WORKLOADS, Workload
from synth.inputs import kv_block, to_f64
from tests.gpu_util import KV_TOL, TOL, GpuDrafter, check_logits, check_rows, check_tokens, log, shape_weights64

pytestmark = pytest.mark.gpu


def _gpu_ar(g, K):
    torch = g.torch
    d = g.d
    B = int(d["req_slot"].shape[0])
    draft = torch.full((B, K), -1, dtype=torch.int32, device="cuda")
    z = torch.empty((B, K, g.w.shape.vocab), dtype=torch.float32, device="cuda")
    g.pe.pe_draft_ar(g.ctx, B, K, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"], draft, z)
    torch.cuda.synchronize()
    return draft.cpu().numpy(), z.cpu().numpy()


def _oracle_ar(w, W64, state, K, req, feed):
    seq = state["seq_len"][req]

    def ctx(l, i):
        b, L = req[i], int(seq[i])
        return (to_f64(kv_block(w, l, 0, b, L), w.shape.dtype), to_f64(kv_block(w, l, 1, b, L), w.shape.dtype))

    st = {"last_token": state["last_token"][req],
          "target_hidden": to_f64(state["target_hidden"][req], w.shape.dtype), "seq_len": seq}
    return O.draft_autoregressive(w.shape, W64, st, ctx, K, tail=True, feed=feed)


_SMALL = {"B9-K2": Workload("qwen3coder-bf16-B9-K2-ar", QWEN3_CODER, 9, 2, (60, 400), 0.7, 7700),
          "B17-K2": Workload("qwen3coder-bf16-B17-K2-ar", QWEN3_CODER, 17, 2, (60, 400), 0.7, 7701)}


@pytest.mark.parametrize("name", ["qwen3coder-bf16-B1-K3-L2048", "qwen3coder-bf16-B4-K3-L1024to4096", "B9-K2",
                                  "B17-K2"])
def test_autoregressive_parity(name):
    """One-row passes of 1 and 4 requests (small-batch kernels), 9 (the LM head on the weight-stream
    kernel) and 17 (every projection on it); the larger batches on sampled requests."""
    w = _SMALL.get(name) or WORKLOADS[name]
    log(f"autoregressive draft parity {name}")
    tol = TOL[w.shape.dtype]
    g = GpuDrafter(w)
    try:
        K = w.K
        draft, z = _gpu_ar(g, K)
        req = list(range(w.B)) if w.B <= 4 else [0, w.B // 2, w.B - 1]
        ref = _oracle_ar(w, shape_weights64(w.shape), g.state, K, req, feed=draft[req])
        strict = exempt = 0
        for i in range(K):
            check_logits(z[req, i], ref["logits"][:, i], tol, f"{name} pass {i}")
            s_, e_ = check_tokens(draft[req, i], ref["logits"][:, i], tol, f"{name} pass {i}")
            strict, exempt = strict + s_, exempt + e_
        kv_err = 0.0
        for l in range(w.shape.n_layers):
            for i, b in enumerate(req):
                k, v = g.kv_rows(l, b, K + 1)
                kv_err = max(kv_err, check_rows(k, ref["k_new"][l][i], KV_TOL[w.shape.dtype], f"{name} K rows l{l} b{b}"),
                             check_rows(v, ref["v_new"][l][i], KV_TOL[w.shape.dtype], f"{name} V rows l{l} b{b}"))
        log(f"  {w.name}: tokens strict {strict}/{len(req) * K}, exempt {exempt}, kv err {kv_err:.2e}")
    finally:
        g.close()


def test_autoregressive_pass0_matches_parallel_row0():
    # pass 0 of the chain and row 0 of the parallel step see the same context and the same input row
    w = WORKLOADS["qwen3coder-bf16-B4-K3-L1024to4096"]
    tol = TOL[w.shape.dtype]
    g = GpuDrafter(w)
    try:
        _, z_ar = _gpu_ar(g, w.K)
        draft_pe, z_pe = g.draft()
        z_pe = z_pe.cpu().numpy()
        check_logits(z_ar[:, 0], z_pe[:, 0], tol, "pass 0 vs parallel row 0")
    finally:
        g.close()


def test_autoregressive_rejects_fp32_drafter():
    w = WORKLOADS["tiny-fp32-B1-K4-L64"]
    g = GpuDrafter(w)
    try:
        with pytest.raises(g.pe.PeError) as e:
            _gpu_ar(g, w.K)
        assert e.value.status == g.pe.PE_ERR_UNSUPPORTED
    finally:
        g.close()
