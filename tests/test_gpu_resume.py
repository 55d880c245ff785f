"""Snapshot -> resume: the drafter keeps no state of its own between calls.

Everything a draft + verify step reads or writes lives in caller-owned device memory: the K/V cache, the
batch metadata (req_slot, seq_len, last_token), the target hiddens and logits. A ctx holds only the packed
weights and a workspace whose contents do not outlive a call. So a copy of the cache and of the metadata
taken after some steps, restored later into a new ctx (whose workspace has meanwhile run unrelated work),
must reproduce every later output bit for bit: draft tokens, draft logits, verify and compaction outputs
and the final cache contents (the kernels are deterministic: fixed reduction orders, no float atomics).
The runs use the batch of a serving loop (kept requests in compacted order, freed slots refilled).
"""

from __future__ import annotations

import numpy as np
import pytest

from synth.inputs import churn_finished, kv_block, new_request, plant_target_logits, step_hiddens
from synth.workloads import QWEN3_CODER, Workload

from gpu_util import GpuDrafter, log, run_verify

pytestmark = pytest.mark.gpu

W = Workload("qwen3coder-bf16-B6-K5-L300to900-resume", QWEN3_CODER, 6, 5, (300, 900), (0.5, 0.9), 2300,
             churn=0.34, new_ctx=(100, 400), steps=6)


def _step(dr, st, step):
    """One draft + verify step on state st; returns its outputs (host arrays) and the next state."""
    import torch
    from synth.device import to_device
    w, s = dr.w, dr.w.shape
    B, K = w.B, w.K
    dstate = {"req_slot": to_device(st["req_slot"], "i32"), "seq_len": to_device(st["seq_len"], "i32"),
              "last_token": to_device(st["last_token"], "i32"),
              "target_hidden": to_device(st["target_hidden"], s.dtype)}
    draft_dev, z = dr.draft(dstate=dstate)
    draft = draft_dev.cpu().numpy()
    T = plant_target_logits(w, draft, st["alpha"], step)
    fin = churn_finished(w, step)
    got = run_verify(dr.pe, dr.ctx, B, K, to_device(T, s.dtype), draft_dev, to_device(fin, "u8"),
                     dstate["req_slot"], dstate["seq_len"])
    out = {"draft": draft, "logits": z.cpu().numpy(), **got}
    n_keep = int(got["n_keep"][0])
    kept = [int(i) for i in got["keep_index"][:n_keep]]
    nxt = {"req_slot": list(got["req_slot_next"][:n_keep]), "seq_len": list(got["seq_len_next"][:n_keep]),
           "last_token": list(got["last_token_next"][:n_keep]), "alpha": [st["alpha"][i] for i in kept]}
    free = [sl for sl in range(w.n_slots) if sl not in set(int(x) for x in nxt["req_slot"])]
    for i in range(B - n_keep):
        nr = new_request(w, step, i)
        for l in range(s.n_layers):
            for kind, cache in ((0, dr.kc[l]), (1, dr.vc[l])):
                cache[free[i], :, : nr["seq_len"], :] = to_device(kv_block(w, l, kind, nr["request_key"],
                                                                            nr["seq_len"]), s.dtype)
        nxt["req_slot"].append(free[i])
        nxt["seq_len"].append(nr["seq_len"])
        nxt["last_token"].append(nr["last_token"])
        nxt["alpha"].append(0.7)
    torch.cuda.synchronize()
    nst = {"req_slot": np.array(nxt["req_slot"], dtype=np.int32), "seq_len": np.array(nxt["seq_len"], dtype=np.int32),
           "last_token": np.array(nxt["last_token"], dtype=np.int32), "alpha": np.array(nxt["alpha"]),
           "target_hidden": step_hiddens(w, step + 1)}
    assert int(nst["seq_len"].max()) + K + 1 <= w.max_ctx
    return out, nst


def _new_ctx(dr):
    pe = dr.pe
    dr.ctx = pe.pe_init(dr.cfg, pe.make_weights(dr.dev, dr.w.shape.n_layers), pe.make_kv(dr.kc, dr.vc), dr.stream)


def test_snapshot_resume_bit_identical():
    import torch
    w = W
    dr = GpuDrafter(w)
    st = {k: np.array(v) for k, v in dr.state.items()}
    try:
        for step in range(2):
            _, st = _step(dr, st, step)
        log(f"snapshot after 2 steps: seq_len {st['seq_len'].tolist()} slots {st['req_slot'].tolist()}")
        snap_kv = [(k.clone(), v.clone()) for k, v in zip(dr.kc, dr.vc)]
        snap_st = {k: v.copy() for k, v in st.items()}

        first = []
        for step in range(2, 5):
            o, st = _step(dr, st, step)
            first.append(o)
        end_kv = [(k.clone(), v.clone()) for k, v in zip(dr.kc, dr.vc)]
        end_st = st

        # a new ctx; its workspace first runs a step on other inputs (which also writes the cache), then
        # the snapshot is restored and the same three steps run again
        dr.close()
        _new_ctx(dr)
        _step(dr, end_st, 5)
        for (k, v), (ks, vs) in zip(zip(dr.kc, dr.vc), snap_kv):
            k.copy_(ks)
            v.copy_(vs)
        torch.cuda.synchronize()
        st = snap_st
        for i, step in enumerate(range(2, 5)):
            o, st = _step(dr, st, step)
            for key, val in first[i].items():
                assert np.array_equal(o[key], val), f"step {step}: {key} differs after resume"
            log(f"step {step} after resume: every output bit-identical (accept_len {o['accept_len'].tolist()})")
        for l, ((k, v), (ke, ve)) in enumerate(zip(zip(dr.kc, dr.vc), end_kv)):
            assert torch.equal(k, ke) and torch.equal(v, ve), f"layer {l}: cache differs after resume"
        for key in ("req_slot", "seq_len", "last_token"):
            assert np.array_equal(st[key], end_st[key])
    finally:
        dr.close()
