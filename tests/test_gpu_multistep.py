"""GPU parity over several state-advancing draft + verify steps with churn, with the greedy verify and with
the sampled one (temperature > 0, seeded uniforms; its checks are those of test_gpu_verify_sampled).

Each step: pe_draft_step on the current batch (checked against the oracle's draft step on the oracle's own
copy of every request's context), target logits planted on the GPU's draft, pe_verify with random
finished flags (checked bit-exactly against the oracle's verify + compaction), then the next batch is
built the way a serving loop would: kept requests take req_slot_next / seq_len_next / last_token_next,
the freed cache slots go to new requests (their contexts written into the device cache), and every
request gets fresh target hiddens.

Cache reading followed by both sides: a draft step writes the K/V of its K rows and of one trailing
placeholder row at positions L_b .. L_b + K; after verify, positions up to the new seq_len (L_b +
accept_len, at most L_b + K + 1) are context, so the oracle appends its own rows 0 .. accept_len - 1 to
the request's context, and the GPU's later rows simply overwrite the rest. All-accepted steps (accept_len
= K + 1) are what reads the trailing row.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import pe_oracle as O
from synth.inputs import churn_finished, kv_block, new_request, plant_target_logits, step_hiddens, to_f64
from synth.workloads import QWEN3_CODER, TINY_FP32, Workload

from gpu_util import TOL, GpuDrafter, check_logits, check_tokens, check_verify, log, run_verify, shape_weights64

pytestmark = pytest.mark.gpu

MULTI = [
    Workload("tiny-fp32-B3-K4-L20to64-steps", TINY_FP32, 3, 4, (20, 64), 0.7, 1100, churn=0.34, new_ctx=(8, 40),
             steps=5),
    Workload("qwen3coder-bf16-B4-K3-L256to1024-steps", QWEN3_CODER, 4, 3, (256, 1024), (0.5, 0.9), 2100,
             churn=0.25, new_ctx=(128, 512), steps=3),
]


def _run(w: Workload, tau=None, steps=None, sample=None):
    """steps: how many steps to run (default w.steps). sample: check this many requests' drafts against the
    oracle each step instead of all of them; a checked request stays checked while it lives (its oracle
    context is grown by the oracle's own rows), and a finished one is replaced by a request that joins the
    batch at that step. Verify and the metadata rebuild are always checked for the whole batch."""
    import torch
    from synth.device import to_device

    s = w.shape
    tol = TOL[s.dtype]
    dr = GpuDrafter(w)
    W64 = shape_weights64(s)
    B, K, Hkv, hd = w.B, w.K, s.n_kv_heads, s.head_dim
    st = {k: np.array(v) for k, v in dr.state.items()}
    keys = list(range(B))                 # request keys (the context generator's identity)
    L0 = {b: int(st["seq_len"][b]) for b in range(B)}  # generated context length per key
    ext = {b: [[np.zeros((Hkv, 0, hd)) for _ in range(s.n_layers)] for _ in range(2)] for b in range(B)}
    checked = set(keys) if sample is None else {keys[i] for i in sorted({0, B // 2, B - 1})[:sample]}
    try:
        for step in range(steps or w.steps):
            log(f"{w.name} step {step}: seq_len {st['seq_len'].tolist()} slots {st['req_slot'].tolist()}")
            dstate = {"req_slot": to_device(st["req_slot"], "i32"), "seq_len": to_device(st["seq_len"], "i32"),
                      "last_token": to_device(st["last_token"], "i32"),
                      "target_hidden": to_device(st["target_hidden"], s.dtype)}
            draft_dev, z = dr.draft(dstate=dstate)
            draft = draft_dev.cpu().numpy()
            pos = [i for i in range(B) if keys[i] in checked]  # batch positions checked this step

            def ctx(l, j):
                key = keys[pos[j]]
                pre = [to_f64(kv_block(w, l, kind, key, L0[key]), s.dtype) for kind in (0, 1)]
                return tuple(np.concatenate([pre[kind], ext[key][kind][l]], axis=1) for kind in (0, 1))

            ref = O.draft_step(s, W64, {"last_token": st["last_token"][pos], "seq_len": st["seq_len"][pos],
                                        "target_hidden": to_f64(st["target_hidden"][pos], s.dtype)}, ctx, K,
                               tail=True)
            err = check_logits(z.cpu().numpy()[pos], ref["logits"], tol, f"step {step} logits")
            strict, exempt = check_tokens(draft[pos], ref["logits"], tol, f"step {step} tokens")
            log(f"  draft parity on requests {pos}: max row-rel err {err:.2e}, {strict}/{len(pos) * K} tokens "
                f"equal, {exempt} near-ties")

            T = plant_target_logits(w, draft, st["alpha"], step)
            fin = churn_finished(w, step)
            if tau is None:
                got = run_verify(dr.pe, dr.ctx, B, K, to_device(T, s.dtype), draft_dev, to_device(fin, "u8"),
                                 dstate["req_slot"], dstate["seq_len"])
                v, c = check_verify(got, to_f64(T, s.dtype), draft, fin, st["req_slot"], st["seq_len"])
            else:
                from test_gpu_verify_sampled import _check, _run as run_sampled, _uniforms
                Tx = to_f64(T, s.dtype)
                u_s, v_s = _uniforms(Tx, draft, tau, w.seed + 31 * step)
                got = run_sampled(dr.pe, dr.ctx, to_device(T, s.dtype), draft, tau, u_s, v_s, fin, st["req_slot"],
                                  st["seq_len"])
                v, c = _check(got, Tx, draft, tau, u_s, v_s, fin, st["req_slot"], st["seq_len"])
            log(f"  verify: accept_len {v['accept_len'].tolist()}, finished {fin.tolist()}, kept {c['n_keep']}")

            # the oracle's context grows by its own rows 0 .. accept_len - 1 of this step
            for j, b in enumerate(pos):
                a = int(v["accept_len"][b])
                for l in range(s.n_layers):
                    for kind, new in ((0, ref["k_new"][l]), (1, ref["v_new"][l])):
                        rows = new[j, :a].transpose(1, 0, 2)  # [Hkv, a, hd]
                        ext[keys[b]][kind][l] = np.concatenate([ext[keys[b]][kind][l], rows], axis=1)

            # next batch: kept requests in their compacted order, then new requests in the freed slots
            n_keep = c["n_keep"]
            kept = [int(i) for i in c["keep_index"][:n_keep]]
            nxt = {"req_slot": list(c["req_slot_next"][:n_keep]), "seq_len": list(c["seq_len_next"][:n_keep]),
                   "last_token": list(c["last_token_next"][:n_keep]), "alpha": [st["alpha"][i] for i in kept]}
            nkeys = [keys[i] for i in kept]
            free = [sl for sl in range(w.n_slots) if sl not in set(int(x) for x in nxt["req_slot"])]
            for i in range(B - n_keep):
                nr = new_request(w, step, i)
                slot = free[i]
                key = nr["request_key"]
                L0[key] = nr["seq_len"]
                ext[key] = [[np.zeros((Hkv, 0, hd)) for _ in range(s.n_layers)] for _ in range(2)]
                for l in range(s.n_layers):
                    for kind, cache in ((0, dr.kc[l]), (1, dr.vc[l])):
                        blk = to_device(kv_block(w, l, kind, key, nr["seq_len"]), s.dtype)
                        cache[slot, :, : nr["seq_len"], :] = blk
                nxt["req_slot"].append(slot)
                nxt["seq_len"].append(nr["seq_len"])
                nxt["last_token"].append(nr["last_token"])
                nxt["alpha"].append(float(np.mean(w.alpha)) if isinstance(w.alpha, tuple) else float(w.alpha))
                nkeys.append(key)
            torch.cuda.synchronize()
            # a checked request that finished is replaced by one that joins now
            gone = [k for k in checked if k not in set(nkeys)]
            fresh = [k for k in nkeys[n_keep:] if k not in checked]
            checked = (checked - set(gone)) | set(fresh[:len(gone)])
            keys = nkeys
            st = {"req_slot": np.array(nxt["req_slot"], dtype=np.int32),
                  "seq_len": np.array(nxt["seq_len"], dtype=np.int32),
                  "last_token": np.array(nxt["last_token"], dtype=np.int32),
                  "alpha": np.array(nxt["alpha"], dtype=np.float64),
                  "target_hidden": step_hiddens(w, step + 1)}
            # the next draft step writes K/V at positions seq_len .. seq_len + K
            assert int(st["seq_len"].max()) + K + 1 <= w.max_ctx
    finally:
        dr.close()


@pytest.mark.parametrize("w", MULTI, ids=lambda w: w.name)
def test_multistep_churn_parity(w):
    _run(w)


@pytest.mark.parametrize("w,tau", [(MULTI[0], 0.2), (MULTI[1], 0.1)], ids=lambda v: getattr(v, "name", str(v)))
def test_multistep_churn_sampled_verify(w, tau):
    _run(w, tau)


def test_multistep_churn_parity_high_concurrency():
    """The 32-request churn workload (K 7, contexts 512-4096, 10 % of the requests finish after every step
    and new ones with contexts 256-1024 take their slots) over four state-advancing steps: verify and the
    metadata rebuild of the whole batch bit-exact every step, drafts of three tracked requests against the
    oracle."""
    from synth import WORKLOADS
    _run(WORKLOADS["qwen3coder-bf16-B32-K7-L512to4096-churn"], steps=4, sample=3)


def test_multistep_catchup_parity():
    """State-advancing steps with catch-up: each step runs the previous verify's emitted tokens as real rows
    (with fresh target hiddens for each) and then the placeholders (pe_draft_catchup); the real rows' K/V
    become context, so the oracle grows each request's context by its own real rows only. Drafts against
    the oracle every step; verify bit-exact; the next step starts at P + n_real with the emitted tokens."""
    import torch
    from synth.device import to_device
    from synth.inputs import catchup_inputs

    w = Workload("qwen3coder-bf16-B4-K3-L256to1024-catchup-steps", QWEN3_CODER, 4, 3, (256, 1024), (0.5, 0.9), 2200,
                 steps=6)
    s = w.shape
    tol = TOL[s.dtype]
    B, K, R = w.B, w.K, w.K + 1
    dr = GpuDrafter(w, max_k=R + K - 1)
    W64 = shape_weights64(s)
    st = dr.state
    L0 = [int(x) for x in st["seq_len"]]
    ext = [[[np.zeros((s.n_kv_heads, 0, s.head_dim)) for _ in range(s.n_layers)] for _ in range(2)] for _ in range(B)]
    pos = np.array(L0, dtype=np.int32)                      # position of each request's first real row
    n_real = np.ones(B, dtype=np.int32)
    tokens = np.zeros((B, R), dtype=np.int32)
    tokens[:, 0] = st["last_token"]
    hid = catchup_inputs(w, R, 0)["target_hidden"]
    hid[:, 0] = st["target_hidden"]
    try:
        for step in range(3):
            log(f"catch-up step {step}: positions {pos.tolist()} n_real {n_real.tolist()}")
            pos_dev = to_device(pos, "i32")
            draft_dev = torch.full((B, K), -1, dtype=torch.int32, device="cuda")
            z = torch.empty((B, K, s.vocab), dtype=torch.float32, device="cuda")
            dr.pe.pe_draft_catchup(dr.ctx, B, K, R, dr.d["req_slot"], pos_dev, to_device(n_real, "i32"),
                                   to_device(tokens, "i32"), to_device(hid, s.dtype), draft_dev, z)
            torch.cuda.synchronize()
            draft = draft_dev.cpu().numpy()

            def ctx(l, b):
                pre = [to_f64(kv_block(w, l, kind, b, L0[b]), s.dtype) for kind in (0, 1)]
                return tuple(np.concatenate([pre[kind], ext[b][kind][l]], axis=1) for kind in (0, 1))

            ref = O.draft_step_catchup(s, W64, {"tokens": tokens, "target_hidden": to_f64(hid, s.dtype),
                                                "n_real": n_real, "seq_len": pos}, ctx, K)
            err = check_logits(z.cpu().numpy(), ref["logits"], tol, f"catch-up step {step} logits")
            strict, exempt = check_tokens(draft, ref["logits"], tol, f"catch-up step {step} tokens")
            log(f"  draft parity: max row-rel err {err:.2e}, {strict}/{B * K} tokens equal, {exempt} near-ties")

            T = plant_target_logits(w, draft, np.full(B, 0.7), step)
            fin = np.zeros(B, dtype=np.uint8)
            got = run_verify(dr.pe, dr.ctx, B, K, to_device(T, s.dtype), draft_dev, None, dr.d["req_slot"], pos_dev)
            v, c = check_verify(got, to_f64(T, s.dtype), draft, fin, st["req_slot"], pos)
            log(f"  verify: accept_len {v['accept_len'].tolist()}")

            # the real rows' K/V join the context; the emitted tokens are the next step's real rows
            for b in range(B):
                r = int(n_real[b])
                for l in range(s.n_layers):
                    for kind, new in ((0, ref["k_new"][l]), (1, ref["v_new"][l])):
                        ext[b][kind][l] = np.concatenate([ext[b][kind][l], new[b, :r].transpose(1, 0, 2)], axis=1)
            cu = c["cu_accept"]
            nxt = catchup_inputs(w, R, step + 1)
            for b in range(B):
                a = int(v["accept_len"][b])
                tokens[b, :a] = c["out_tokens"][cu[b]:cu[b] + a]
                tokens[b, a:] = 0
            pos = pos + n_real
            n_real = v["accept_len"].astype(np.int32)
            hid = nxt["target_hidden"]
            assert int(pos.max()) + R + K <= w.max_ctx
    finally:
        dr.close()
