"""GPU parity of the parallel draft step with concatenated input rows (row_concat = 1) against the oracle's
draft_step_concat: each row is [embedding || hidden], 2d wide into layer 0's attention with each half
RMS-normalised under its own gain, and the hidden half is the residual stream.

Per request: logits within the row-relative tolerance, draft tokens identical up to the top-2-gap
exemption, and the K/V of all K + 1 rows (with the trailing placeholder row) within the same tolerance.
Row counts cover the small-batch kernels (4 rows, the row build on the 4-column tiles), the weight-stream
kernel (32 layer rows) and the 128 x 128 tiled kernel (160 rows), where layer 0's QKV reads the bf16
concatenated operand.
"""

import numpy as np
import pytest

from oracle import pe_oracle as O
from synth import Workload
from synth.inputs import kv_block, to_f64
from synth.workloads import QWEN3_CODER_CONCAT
from tests.gpu_util import KV_TOL, TOL, GpuDrafter, check_logits, check_rows, check_tokens, log, shape_weights64

pytestmark = pytest.mark.gpu


def _oracle(w, W64, state, K, req):
    seq = state["seq_len"][req]

    def ctx(l, i):
        b, L = req[i], int(seq[i])
        return (to_f64(kv_block(w, l, 0, b, L), w.shape.dtype), to_f64(kv_block(w, l, 1, b, L), w.shape.dtype))

    st = {"last_token": state["last_token"][req], "target_hidden": to_f64(state["target_hidden"][req], w.shape.dtype),
          "seq_len": seq}
    return O.draft_step_concat(w.shape, W64, st, ctx, K, tail=True)


@pytest.mark.parametrize("B,K", [(1, 3), (4, 7), (20, 7)], ids=lambda v: str(v))
def test_concat_rows_parity(B, K):
    w = Workload(f"qwen3coder-concat-bf16-B{B}-K{K}", QWEN3_CODER_CONCAT, B, K, (60, 400), 0.7, 8100 + 10 * B + K)
    log(f"concatenated rows parity B {B} K {K} (layer rows {B * (K + 1)})")
    tol = TOL[w.shape.dtype]
    g = GpuDrafter(w)
    try:
        draft, z = g.draft()
        draft, z = draft.cpu().numpy(), z.cpu().numpy()
        req = list(range(B)) if B <= 4 else [0, 7, B - 1]
        ref = _oracle(w, shape_weights64(w.shape), g.state, K, req)
        err = check_logits(z[req], ref["logits"], tol, w.name)
        strict, exempt = check_tokens(draft[req], ref["logits"], tol, w.name)
        kv_err = 0.0
        for l in range(w.shape.n_layers):
            for i, b in enumerate(req):
                k, v = g.kv_rows(l, b, K + 1)
                kv_err = max(kv_err, check_rows(k, ref["k_new"][l][i], KV_TOL[w.shape.dtype], f"{w.name} K rows l{l} b{b}"),
                             check_rows(v, ref["v_new"][l][i], KV_TOL[w.shape.dtype], f"{w.name} V rows l{l} b{b}"))
        log(f"  logit err {err:.2e}, kv err {kv_err:.2e}, tokens strict {strict}/{len(req) * K}, exempt {exempt}")
    finally:
        g.close()


def test_concat_rows_parity_headline_size():
    """One request at context 2048, K 3: the headline configuration with concatenated rows (the bench's
    concat_rows_step times this shape)."""
    w = Workload("qwen3coder-concat-bf16-B1-K3-L2048", QWEN3_CODER_CONCAT, 1, 3, (2048, 2048), 0.7, 8150)
    tol = TOL[w.shape.dtype]
    g = GpuDrafter(w)
    try:
        draft, z = g.draft()
        ref = _oracle(w, shape_weights64(w.shape), g.state, 3, [0])
        err = check_logits(z.cpu().numpy(), ref["logits"], tol, w.name)
        strict, exempt = check_tokens(draft.cpu().numpy(), ref["logits"], tol, w.name)
        log(f"  logit err {err:.2e}, tokens strict {strict}/3, exempt {exempt}")
    finally:
        g.close()


def test_concat_rows_unsupported_entry_points():
    w = Workload("qwen3coder-concat-bf16-B2-K3-args", QWEN3_CODER_CONCAT, 2, 3, (60, 100), 0.7, 8190)
    g = GpuDrafter(w)
    torch = g.torch
    d = g.d
    try:
        tok = torch.empty((2, 3), dtype=torch.int32, device="cuda")
        with pytest.raises(g.pe.PeError) as e:
            g.pe.pe_draft_ar(g.ctx, 2, 3, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"], tok)
        assert e.value.status == g.pe.PE_ERR_UNSUPPORTED
        rows = torch.zeros((2, 3, w.shape.d_model), dtype=torch.float32, device="cuda")
        with pytest.raises(g.pe.PeError) as e:
            g.pe.pe_draft_rows(g.ctx, 2, 3, d["req_slot"], d["seq_len"], rows, tok)
        assert e.value.status == g.pe.PE_ERR_UNSUPPORTED
    finally:
        g.close()
