"""pe_verify_static (greedy verify on the library's static scratch, no allocation) against pe_verify.

Two calls in a row on the same GPU, the second smaller than the first (so a stale tail of the first call's
scratch would show), each compared with pe_verify on the same inputs: every output bit-exact, and both
against the oracle's verify + compaction. Then a third call back at the first size.
"""

import numpy as np
import pytest

from synth import Workload, DrafterShape, make_state, plant_target_logits, random_draft, churn_finished
from synth.inputs import bf16_bits_to_f32
from tests.gpu_util import check_verify, log, run_verify, to_device
from tests.test_gpu_verify import VerifyCtx

pytestmark = pytest.mark.gpu

CASES = [  # (B, K, V, dtype): large, then smaller, then large again
    (128, 7, 151936, "bf16"),
    (5, 3, 4096, "f32"),
    (64, 10, 201088, "bf16"),
]


def _inputs(B, K, V, dtype, seed):
    s = DrafterShape(f"verify-only-{V}-{dtype}", 1, 32, 1, 1, 64, 32, V, dtype)
    w = Workload(f"static-verify-B{B}-K{K}", s, B, K, (100, 500), 0.6, seed, churn=0.2, new_ctx=(10, 20))
    st = make_state(w)
    draft = random_draft(w)
    T = plant_target_logits(w, draft, st["alpha"])
    fin = churn_finished(w, 0)
    return st, draft, T, fin


def _static(B, K, V, dtype, T_dev, draft_dev, fin_dev, slot_dev, seq_dev):
    import torch
    import eagle_drafting_amd as pe
    i32 = dict(dtype=torch.int32, device="cuda")
    names = ("accept_len", "cu_accept", "out_tokens", "keep_index", "n_keep", "req_slot_next", "seq_len_next",
             "last_token_next")
    sizes = (B, B + 1, B * (K + 1), B, 1, B, B, B)
    out = {n: torch.full((m,), -7, **i32) for n, m in zip(names, sizes)}
    pe.pe_verify_static(B, K, V, dtype, T_dev, draft_dev, fin_dev, slot_dev, seq_dev, *[out[n] for n in names],
                        stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def test_static_verify_matches_pe_verify_on_consecutive_calls():
    for i, (B, K, V, dtype) in enumerate(CASES):
        log(f"static verify call {i}: B {B} K {K} V {V} {dtype}")
        st, draft, T, fin = _inputs(B, K, V, dtype, 9100 + i)
        T_dev = to_device(T, dtype)
        d_dev, f_dev = to_device(draft, "i32"), to_device(fin, "u8")
        s_dev, q_dev = to_device(st["req_slot"], "i32"), to_device(st["seq_len"], "i32")
        got = _static(B, K, V, dtype, T_dev, d_dev, f_dev, s_dev, q_dev)
        ctx = VerifyCtx(V, dtype, B, K)
        try:
            ref = run_verify(ctx.pe, ctx.ctx, B, K, T_dev, d_dev, f_dev, s_dev, q_dev)
        finally:
            ctx.close()
        for k in ref:
            assert np.array_equal(got[k], ref[k]), f"call {i}: {k} differs from pe_verify"
        T_exact = T if dtype == "f32" else bf16_bits_to_f32(T)
        v, c = check_verify(got, T_exact, draft, fin, st["req_slot"], st["seq_len"])
        log(f"  equal to pe_verify and the oracle: accept_len mean {v['accept_len'].mean():.3f}, kept {c['n_keep']}")


def test_static_verify_rejects_bad_sizes():
    import torch
    import eagle_drafting_amd as pe
    z = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(pe.PeError) as e:
        pe.pe_verify_static(1025, 3, 4096, "bf16", z, z, None, z, z, z, z, z, z, z, z, z, z)
    assert e.value.status == pe.PE_ERR_INVALID
    with pytest.raises(pe.PeError) as e:
        pe.pe_verify_static(4, 3, 4100, "bf16", z, z, None, z, z, z, z, z, z, z, z, z, z)
    assert e.value.status == pe.PE_ERR_INVALID
