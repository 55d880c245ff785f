"""GPU parity of the parallel draft step (pe_draft_step / pe_draft_rows) against the oracle, plus the
method's invariants on the GPU.

Per request: logits within the row-relative tolerance (1e-4 fp32, 2e-2 bf16), draft tokens identical up
to the top-2-gap exemption, and this step's K/V rows appended to the cache within the same tolerance.
Workloads whose full oracle run would take minutes are checked on sampled requests (requests are
independent, so a sampled request's oracle result is exact for it).
"""

import numpy as np
import pytest

from synth import WORKLOADS, Workload, TINY_FP32, QWEN3_CODER, GPT_OSS_20B, make_state
from tests.gpu_util import (KV_TOL, TOL, GpuDrafter, check_logits, check_rows, check_tokens, log, oracle_draft,
                            shape_weights64)

pytestmark = pytest.mark.gpu


def _parity(g, requests, K=None, rows=None, rows_host=None, check_kv=True):
    w = g.w
    K = K or w.K
    tol = TOL[w.shape.dtype]
    draft, z = g.draft(K=K, rows=rows)
    W64 = shape_weights64(w.shape)
    req = list(requests)
    ref = oracle_draft(w, W64, g.state, K, req, rows=rows_host)
    err = check_logits(z.cpu().numpy()[req], ref["logits"], tol, w.name)
    strict, exempt = check_tokens(draft.cpu().numpy()[req], ref["logits"], tol, w.name)
    kv_err = 0.0
    if check_kv:
        for l in range(w.shape.n_layers):
            for i, b in enumerate(req):
                k, v = g.kv_rows(l, b, K)
                kt = KV_TOL[w.shape.dtype]
                kv_err = max(kv_err, check_rows(k, ref["k_new"][l][i], kt, f"{w.name} K rows l{l} b{b}"),
                             check_rows(v, ref["v_new"][l][i], kt, f"{w.name} V rows l{l} b{b}"))
    log(f"  {w.name}: requests {req[:6]}{'...' if len(req) > 6 else ''} logit err {err:.2e}, kv err {kv_err:.2e}, "
        f"tokens strict {strict}/{len(req) * K}, exempt {exempt}")
    return draft, z, ref


def _sample(w, state, n=3):
    rng = np.random.default_rng(w.seed + 7)
    pick = {0, w.B - 1, int(np.argmax(state["seq_len"]))}
    pick |= set(int(x) for x in rng.choice(w.B, size=min(n, w.B), replace=False))
    return sorted(pick)


FULL = ["tiny-fp32-B1-K4-L64", "qwen3coder-bf16-B1-K3-L2048"] + \
       [n for n, w in WORKLOADS.items() if "sweep" in w.tags]
SAMPLED = [n for n, w in WORKLOADS.items() if "churn" in w.tags or "large" in w.tags]


@pytest.mark.parametrize("name", FULL)
def test_draft_parity_full(name):
    w = WORKLOADS[name]
    log(f"draft parity {name}")
    g = GpuDrafter(w)
    try:
        _parity(g, range(w.B))
    finally:
        g.close()


@pytest.mark.parametrize("name", SAMPLED)
def test_draft_parity_sampled(name):
    w = WORKLOADS[name]
    log(f"draft parity (sampled requests) {name}")
    g = GpuDrafter(w)
    try:
        _parity(g, _sample(w, g.state))
    finally:
        g.close()


@pytest.mark.parametrize("shape", [TINY_FP32, QWEN3_CODER], ids=lambda s: s.name)
def test_empty_and_short_contexts(shape):
    # L_b = 0 (the request has no drafter context yet: row j sees only new rows 0..j) and tiny L_b
    w = Workload(f"{shape.name}-short-ctx", shape, 4, 3, (0, 3), 0.7, 7100)
    state = make_state(w)
    state["seq_len"][:] = [0, 1, 0, 3]
    g = GpuDrafter(w, state=state)
    try:
        _parity(g, range(w.B))
    finally:
        g.close()


def _random_rows(w, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((w.B, w.K, w.shape.d_model)).astype(np.float32)


@pytest.mark.parametrize("shape", [TINY_FP32, QWEN3_CODER], ids=lambda s: s.name)
def test_draft_rows_parity_and_causality(shape):
    """Invariant 3: under the causal mask, row j's output does not change when rows after j change.
    The rows are arbitrary (harness-drawn), fed through pe_draft_rows; bit-identical on the GPU."""
    import torch
    w = Workload(f"{shape.name}-rows", shape, 2, 5, (40, 90), 0.7, 7200)
    g = GpuDrafter(w)
    try:
        X = _random_rows(w, 1)
        Xd = torch.from_numpy(X).cuda()
        draft0, z0, _ = _parity(g, range(w.B), rows=Xd, rows_host=X.astype(np.float64), check_kv=False)
        z0 = z0.cpu().numpy()
        for j in range(w.K - 1):
            Xp = X.copy()
            Xp[:, j + 1:] += np.random.default_rng(10 + j).standard_normal(Xp[:, j + 1:].shape).astype(np.float32)
            _, zp = g.draft(rows=torch.from_numpy(Xp).cuda())
            zp = zp.cpu().numpy()
            assert np.array_equal(zp[:, : j + 1], z0[:, : j + 1]), f"row <= {j} changed"
            assert not np.array_equal(zp[:, j + 1:], z0[:, j + 1:])
        log("  causality holds bit-exactly")
    finally:
        g.close()


@pytest.mark.parametrize("shape", [TINY_FP32, QWEN3_CODER], ids=lambda s: s.name)
def test_k1_equals_row0_and_determinism(shape):
    """Invariant 2 on the GPU: K = 1 (plain EAGLE step, no placeholders) matches row 0 of the K-row
    step within tolerance; repeated runs are bit-identical."""
    w = Workload(f"{shape.name}-k1", shape, 3, 6, (100, 300), 0.7, 7300)
    g = GpuDrafter(w)
    tol = TOL[shape.dtype]
    try:
        d6, z6 = g.draft(K=6)
        d6b, z6b = g.draft(K=6)
        assert np.array_equal(z6.cpu().numpy(), z6b.cpu().numpy()) and np.array_equal(d6.cpu().numpy(),
                                                                                    d6b.cpu().numpy())
        _, _, ref = _parity(g, range(w.B), K=1)
        check_logits(z6.cpu().numpy()[:, 0], ref["logits"][:, 0], tol, "row 0 of K=6 vs oracle K=1")
        check_tokens(d6.cpu().numpy()[:, 0], ref["logits"][:, 0], tol, "row 0 token")
    finally:
        g.close()


@pytest.mark.parametrize("B,K", [(1, 1), (1, 2), (2, 1), (3, 1)], ids=lambda v: str(v))
def test_four_row_products_parity(B, K):
    """Draft steps of at most 4 rows (B (K + 1) <= 4; (3, 1) has 6) run the residual-stream projections on
    the 4-column weight packing; ragged contexts, parity against the oracle, K/V rows included."""
    w = Workload(f"qwen3coder-bf16-B{B}-K{K}-small", QWEN3_CODER, B, K, (60, 400), 0.7, 7400 + 10 * B + K)
    log(f"four-row products: B {B} K {K} (rows {B * (K + 1)})")
    g = GpuDrafter(w)
    try:
        _parity(g, range(w.B))
    finally:
        g.close()


@pytest.mark.parametrize("B,K", [(1, 3), (2, 2), (1, 4)], ids=lambda v: str(v))
def test_four_row_products_rows_path(B, K):
    """pe_draft_rows with B K <= 4 rows (the 4-column projections without the row build) and 5 rows
    (the 16-column ones), against the oracle on the same caller rows."""
    import torch
    w = Workload(f"qwen3coder-bf16-B{B}-K{K}-rows-small", QWEN3_CODER, B, K, (30, 200), 0.7, 7500 + 10 * B + K)
    log(f"four-row products, rows path: B {B} K {K}")
    g = GpuDrafter(w)
    try:
        X = _random_rows(w, 3)
        _parity(g, range(w.B), rows=torch.from_numpy(X).cuda(), rows_host=X.astype(np.float64), check_kv=False)
    finally:
        g.close()


@pytest.mark.parametrize("B,K", [(1, 8), (3, 5), (9, 3), (5, 12), (9, 11), (16, 7), (11, 11), (20, 7), (32, 8)],
                         ids=lambda v: str(v))
def test_stream_kernel_row_counts_parity(B, K):
    """Row counts around every projection-kernel boundary: layer rows B (K + 1) = 9 (small-batch kernel),
    18 / 36 / 65 / 108 / 128 (weight-stream kernel with 1, 2, 3 and 4 row blocks, 128 the largest) and
    132 / 160 / 288 (128 x 128 tiled kernel); LM-head rows B K = 8, 15, 27, 60, 99, 112 (stream kernel) and
    121, 140, 256 (tiled kernel). Ragged short contexts, sampled requests, K/V rows included."""
    w = Workload(f"qwen3coder-bf16-B{B}-K{K}-rowcounts", QWEN3_CODER, B, K, (60, 400), 0.7, 7600 + 20 * B + K)
    log(f"row counts: B {B} K {K} (layer rows {B * (K + 1)}, LM-head rows {B * K})")
    g = GpuDrafter(w)
    try:
        _parity(g, _sample(w, g.state))
    finally:
        g.close()


@pytest.mark.parametrize("K", [3, 4, 7, 8, 10, 11, 15], ids=lambda v: f"K{v}")
def test_gptoss_attention_row_tiles(K):
    """GPT-OSS-shaped drafter (head dimension 64, 8 query heads per kv head). Attention runs the K draft rows
    plus the trailing placeholder row, so a kv head has 8 (K + 1) query rows: K 3 / 4 / 7 / 8 / 10 / 11 / 15
    give 32 / 40 / 64 / 72 / 88 / 96 / 128 rows, i.e. 2 / 3 / 4 / 5 / 6 / 6 / 8 16-row tiles on 4- or
    8-wave workgroups (5 and 6 tiles leave waves without a row tile; 96 rows fill the last tile, 72 and 88
    do not; 128 is the most the configuration allows). The layer rows,
    3 (K + 1), reach the small-batch kernel (K 3, 4), the burst kernel (K 7, 8: 24 and 27 rows, whose
    reductions of 90 and 270 k-steps end in a short 16-k-step piece) and the weight-stream kernel (K 10,
    11, 15). Contexts 0, 37 and 700: a request with only its own rows,
    one whose keys end inside the first 128-key round, and one spread over several key splits with a
    ragged last round. Every request against the oracle, K/V rows included."""
    w = Workload(f"gptoss20b-bf16-B3-K{K}-rowtiles", GPT_OSS_20B, 3, K, (0, 700), 0.7, 7800 + K)
    state = make_state(w)
    state["seq_len"][:] = [0, 37, 700]
    log(f"GPT-OSS attention row tiles: K {K} ({8 * (K + 1)} query rows per kv head)")
    g = GpuDrafter(w, state=state)
    try:
        _parity(g, range(w.B))
    finally:
        g.close()
