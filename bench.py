"""Benchmark of the P-EAGLE parallel draft step + greedy verify on one MI355X.

One step = pe_draft_step (row build, 4 drafter layers, LM head, argmax: K draft tokens for each of B
requests in one pass) + pe_verify (target argmax over K+1 positions, accepted prefix, bonus token,
batch-metadata rebuild), over inputs already resident in HBM. Prints one JSON line.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--reps 100] [--workload NAME] [--no-targets]
                  [--no-cpu-baseline] [--cpu-seconds 20] [--churn-steps 16] [--variants] [--copy-calibration]

The headline workload is the largest one: the GPT-OSS-20B-shaped bf16 drafter, B = 64 requests, K = 10,
contexts 2048-8192. `targets` adds the Qwen3-Coder-shaped workloads the performance targets are stated on:
B 1 K 3 context 2048 and B 8 K 11 (draft step against 60 % of the HBM roofline), B 128 K 7 (LM head and MLP
GEMMs against 50 % of the bf16 MFMA peak), the latter also as a 16-step state-advancing run with churn.
Kernel times come from a separate pass with per-launch HIP events; the headline's timed loop records none.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE = "gptoss20b-bf16-B64-K10-L2048to8192"
TARGET_WORKLOADS = {
    "qwen_B1_K3": "qwen3coder-bf16-B1-K3-L2048",
    "qwen_B8_K11": "qwen3coder-bf16-B8-K11-L1024to4096",
    "qwen_B128_K7": "qwen3coder-bf16-B128-K7-L512to4096-churn",
}
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "draft tokens/s and draft+verify steps/s at B×K; % of HBM/MFMA roofline"
HBM_TARGET = 0.60              # draft step at B <= 8
MFMA_TARGET = 0.50             # LM-head / MLP GEMMs at B = 128


# ---------------------------------------------------------------------------------------------- work

def layer_rows(w):
    """Rows each drafter layer runs in a draft step: K draft rows plus the trailing placeholder row whose
    K/V an all-accepted verify keeps (position L + K)."""
    return w.B * (w.K + 1)


def algorithmic_bytes(w, state):
    """Bytes the step must move at minimum: every weight once, the gathered embedding rows, the target
    hiddens, each request's KV context (plus this step's rows) read once, this step's KV rows written once,
    and the target logits read once by verify. Activations, partials and logits dumps are not counted."""
    s = w.shape
    e = s.elem_bytes
    d, V, F = s.d_model, s.vocab, s.ffn_dim
    per_layer = s.qkv_dim * d + d * s.q_dim + 3 * d * F + 2 * d
    weights = (3 * d * d + s.n_layers * per_layer + d * V + d + 2 * d) * e
    L = state["seq_len"].astype(np.int64)
    kv_row = 2 * s.n_kv_heads * s.head_dim * e
    kv_read = s.n_layers * int((L + w.K + 1).sum()) * kv_row
    kv_write = s.n_layers * layer_rows(w) * kv_row
    inputs = w.B * d * e + w.B * 3 * d * e
    draft = weights + kv_read + kv_write + inputs
    verify = w.B * (w.K + 1) * V * e
    return {"draft": draft, "verify": verify, "step": draft + verify, "lm_head": d * V * e, "weights": weights,
            "kv_read": kv_read, "attention_per_layer": kv_read // s.n_layers,
            "qkv": s.qkv_dim * d * e, "o_proj": d * s.q_dim * e, "gate_up": 2 * F * d * e, "down": d * F * e,
            "rows": 3 * d * d * e}


def gemm_flops(w):
    """Flops per launch of each projection: 2 * rows * out * in."""
    s = w.shape
    d, F = s.d_model, s.ffn_dim
    M = layer_rows(w)
    return {"lm_head": 2.0 * w.B * w.K * d * s.vocab, "qkv": 2.0 * M * s.qkv_dim * d, "o_proj": 2.0 * M * d * s.q_dim,
            "gate_up": 2.0 * M * 2 * F * d, "down": 2.0 * M * d * F, "rows": 2.0 * w.B * d * 3 * d}


def attention_flops(w, state):
    """Score and value products of one layer: 4 * hd per (query head, row, visible key)."""
    s = w.shape
    L = state["seq_len"].astype(np.int64)
    rows = w.K + 1
    keys = (rows * L + rows * (rows + 1) // 2).sum()
    return 4.0 * s.n_q_heads * s.head_dim * float(keys)


def ridge_rows():
    return PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)


def kernel_roofline(name, us, launches, nbytes, flops, rows):
    """One kernel's average launch against the roofline that bounds it: HBM below the ridge (bytes per
    flop of a weight-streaming GEMM is 1 / rows), the bf16 MFMA peak above it."""
    secs = us * 1e-6
    gbs = nbytes / secs / 1e9
    tflops = flops / secs / 1e12
    mfma = rows > ridge_rows()
    return {"bound": "mfma" if mfma else "hbm", "avg_launch_us": us, "launches": launches,
            "achieved": tflops if mfma else gbs, "peak": PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if mfma else "GB/s", "frac": (tflops / PEAK_BF16_TFLOPS) if mfma else (gbs / PEAK_HBM_GBS),
            "hbm_frac": gbs / PEAK_HBM_GBS, "mfma_frac": tflops / PEAK_BF16_TFLOPS,
            "bytes_per_launch": nbytes, "flops_per_launch": flops}


KERNEL_SOURCES = {
    "lm_head": ("gemm.hip", "gemm_tiled.hip", "kernels.h", "common.h"),
    "attention": ("attention.hip", "kernels.h", "common.h"),
}


def kernel_source_digest(kernel="lm_head"):
    """sha256 over the sources that define a kernel family (the projections, or attention)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES.get(kernel, KERNEL_SOURCES["lm_head"]):
        h.update(open(os.path.join(ROOT, "eagle_drafting_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def traffic_from_profile(kernel, workload_name):
    """HBM bytes per launch of a kernel measured by rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, scaled by
    the plain-copy calibration), if the committed measurement was taken on this workload with the current
    sources of that kernel."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("workload") != workload_name or rec.get("kernel_src_sha256") != kernel_source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def pct(a, q):
    return float(np.percentile(np.asarray(a, dtype=np.float64), q))


# ------------------------------------------------------------------------------------------ workloads

class Run:
    """One workload's resident inputs, a pe ctx, and the step calls."""

    def __init__(self, pe, torch, name, weights=None):
        from synth import WORKLOADS, make_state
        from synth.device import config_args, upload_kv, upload_state, upload_weights
        self.pe, self.torch = pe, torch
        self.w = w = WORKLOADS[name]
        s = w.shape
        self.dev = weights if weights is not None else upload_weights(s)[0]
        self.state = make_state(w)
        self.kc, self.vc = upload_kv(w, self.state)
        self.d = upload_state(self.state, s.dtype)
        self.stream = torch.cuda.current_stream()
        self.ctx = pe.pe_init(pe.make_config(**config_args(w)), pe.make_weights(self.dev, s.n_layers),
                              pe.make_kv(self.kc, self.vc), self.stream.cuda_stream)
        i32 = dict(dtype=torch.int32, device="cuda")
        B, K = w.B, w.K
        self.draft = torch.empty((B, K), **i32)
        self.outs = [torch.empty(n, **i32) for n in (B, B + 1, B * (K + 1), B, 1, B, B, B)]
        self.draft_call()
        torch.cuda.synchronize()
        self.draft_host = self.draft.cpu().numpy()
        self.T_host, self.T, self.fin = self.plant()

    def plant(self):
        """Target logits planted on this drafter's own draft (the draft is deterministic, so every timed
        step sees the same acceptance pattern); churn workloads mark their first step's finished requests."""
        from synth import churn_finished, plant_target_logits
        from synth.device import to_device
        w = self.w
        T_host = plant_target_logits(w, self.draft_host, self.state["alpha"])
        fin = to_device(churn_finished(w, 0), "u8") if w.churn else None
        return T_host, to_device(T_host, w.shape.dtype), fin

    def draft_call(self):
        d, w = self.d, self.w
        self.pe.pe_draft_step(self.ctx, w.B, w.K, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"],
                              self.draft, None)

    def verify_call(self):
        self.pe.pe_verify(self.ctx, self.w.B, self.w.K, self.T, self.draft, self.fin, self.d["req_slot"],
                          self.d["seq_len"], *self.outs)

    def verify_sampled_call(self):
        """The sampling form of verify at temperature 0.3 (the pages' example request), seeded uniforms."""
        if not hasattr(self, "u_s"):
            torch, w = self.torch, self.w
            rng = np.random.default_rng(w.seed + 23)
            self.u_s = torch.from_numpy(rng.random((w.B, w.K), dtype=np.float32)).cuda()
            self.v_s = torch.from_numpy(rng.random((w.B, w.K + 1), dtype=np.float32)).cuda()
        self.pe.pe_verify_sampled(self.ctx, self.w.B, self.w.K, self.T, self.draft, 0.3, self.u_s, self.v_s, self.fin,
                                  self.d["req_slot"], self.d["seq_len"], *self.outs)

    def step(self):
        self.draft_call()
        self.verify_call()

    def timed(self, fn, n):
        """Total ms of n calls between two events on the library stream (no events in between)."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(n):
            fn()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def per_call(self, fn, n):
        """Each of n calls between its own pair of events: median, p10, p90 in microseconds."""
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        ev[0].record(self.stream)
        for i in range(n):
            fn()
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        us = [1e3 * ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
        return {"median": pct(us, 50), "p10": pct(us, 10), "p90": pct(us, 90), "mean": float(np.mean(us)), "n": n}

    def kernel_times(self, reps):
        """Average launch (us) and launches per step of every profiled kernel, from per-launch events in a
        pass of its own."""
        pe = self.pe
        pe.pe_profile_enable(self.ctx, (1 << pe.PE_PROF_COUNT) - 1)
        for _ in range(reps):
            self.step()
        out = {}
        names = {pe.PE_PROF_LM_HEAD: "lm_head", pe.PE_PROF_ATTENTION: "attention", pe.PE_PROF_GATE_UP: "gate_up",
                 pe.PE_PROF_VERIFY_SCAN: "verify_scan", pe.PE_PROF_QKV: "qkv", pe.PE_PROF_O_PROJ: "o_proj",
                 pe.PE_PROF_DOWN: "down", pe.PE_PROF_ROWS: "rows"}
        for kid, name in names.items():
            tot, n = pe.pe_profile_read(self.ctx, kid)
            out[name] = {"avg_us": 1e3 * tot / max(n, 1), "launches_per_step": n / reps}
        pe.pe_profile_enable(self.ctx, 0)
        return out

    def rooflines(self, kern):
        w = self.w
        ab = algorithmic_bytes(w, self.state)
        fl = gemm_flops(w)
        M = layer_rows(w)
        out = {}
        for name in ("lm_head", "qkv", "o_proj", "gate_up", "down", "rows"):
            rows = w.B * w.K if name == "lm_head" else (w.B if name == "rows" else M)
            k = kern[name]
            out[name] = kernel_roofline(name, k["avg_us"], k["launches_per_step"], ab[name], fl[name], rows)
        k = kern["attention"]
        out["attention"] = kernel_roofline("attention", k["avg_us"], k["launches_per_step"], ab["attention_per_layer"],
                                           attention_flops(w, self.state), 0)
        k = kern["verify_scan"]
        out["verify_scan"] = kernel_roofline("verify_scan", k["avg_us"], k["launches_per_step"], ab["verify"], 0.0, 0)
        return out

    def close(self):
        self.pe.pe_destroy(self.ctx)
        del self.T, self.kc, self.vc, self.d
        self.torch.cuda.empty_cache()


def churn_run(r, n_steps):
    """n_steps state-advancing draft + verify steps with churn: after each verify the kept requests take
    req_slot_next / seq_len_next / last_token_next, the finished ones' slots go to new requests (contexts
    written into the cache beforehand), every request gets fresh target hiddens, and the target logits are
    planted on each step's draft on the device (the target model's stand-in; not timed). Device time of
    draft + verify per step from events around them; the host work between steps is not in it."""
    torch, pe, w = r.torch, r.pe, r.w
    from synth import churn_finished
    from synth.device import to_device
    from synth.inputs import kv_block, new_request
    s = w.shape
    B, K, V = w.B, w.K, s.vocab
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 99)
    T_base = r.T.clone()
    rowmax1 = (T_base[:, :K].float().amax(-1) + 1.0).to(T_base.dtype)
    slot = r.state["req_slot"].astype(np.int32).copy()
    seq = r.state["seq_len"].astype(np.int32).copy()
    last = r.state["last_token"].astype(np.int32).copy()
    alpha = torch.from_numpy(r.state["alpha"].astype(np.float32)).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    draft = torch.empty((B, K), **i32)
    outs = [torch.empty(n, **i32) for n in (B, B + 1, B * (K + 1), B, 1, B, B, B)]
    dev_us, acc_all = [], []
    for step in range(n_steps):
        assert int(seq.max()) + K + 1 <= w.max_ctx  # this step writes K/V at positions seq .. seq + K
        d_slot, d_seq, d_last = to_device(slot, "i32"), to_device(seq, "i32"), to_device(last, "i32")
        hid = torch.randn((B, 3 * s.d_model), generator=gen, device="cuda").to(torch.bfloat16)
        fin_h = churn_finished(w, step)
        fin = to_device(fin_h, "u8")
        T = T_base.clone()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(r.stream)
        pe.pe_draft_step(r.ctx, B, K, d_slot, d_seq, d_last, hid, draft, None)
        e[1].record(r.stream)
        hit = torch.rand((B, K), generator=gen, device="cuda") < alpha[:, None]
        other = torch.randint(0, V - 1, (B, K), generator=gen, device="cuda", dtype=torch.int32)
        other = other + (other >= draft).to(torch.int32)
        tok = torch.where(hit, draft, other).long()
        T[:, :K].scatter_(2, tok.unsqueeze(-1), rowmax1.unsqueeze(-1))
        e[2].record(r.stream)
        pe.pe_verify(r.ctx, B, K, T, draft, fin, d_slot, d_seq, *outs)
        e[3].record(r.stream)
        torch.cuda.synchronize()
        dev_us.append(1e3 * (e[0].elapsed_time(e[1]) + e[2].elapsed_time(e[3])))
        acc = outs[0].cpu().numpy()
        acc_all.append(acc.copy())
        n_keep = int(outs[4].cpu().numpy()[0])
        keep_slot = outs[5].cpu().numpy()[:n_keep]
        nxt_slot = list(keep_slot)
        nxt_seq = list(outs[6].cpu().numpy()[:n_keep])
        nxt_last = list(outs[7].cpu().numpy()[:n_keep])
        free = [sl for sl in range(w.n_slots) if sl not in set(int(x) for x in keep_slot)]
        for i in range(B - n_keep):
            nr = new_request(w, step, i)
            sl = free[i]
            for l in range(s.n_layers):
                r.kc[l][sl, :, :nr["seq_len"], :] = to_device(kv_block(w, l, 0, nr["request_key"], nr["seq_len"]),
                                                              s.dtype)
                r.vc[l][sl, :, :nr["seq_len"], :] = to_device(kv_block(w, l, 1, nr["request_key"], nr["seq_len"]),
                                                              s.dtype)
            nxt_slot.append(sl)
            nxt_seq.append(nr["seq_len"])
            nxt_last.append(nr["last_token"])
        slot = np.array(nxt_slot, dtype=np.int32)
        seq = np.array(nxt_seq, dtype=np.int32)
        last = np.array(nxt_last, dtype=np.int32)
    acc_all = np.concatenate(acc_all)
    return {"steps": n_steps, "B": B, "K": K, "device_us_per_step": {"median": pct(dev_us, 50), "p10": pct(dev_us, 10),
                                                                     "p90": pct(dev_us, 90)},
            "request_steps_per_s": B * 1e6 / pct(dev_us, 50),
            "draft_tokens_per_s": B * K * 1e6 / pct(dev_us, 50),
            "mean_accept_len": float(acc_all.mean()), "alpha_hat": float((acc_all - 1).sum() / (acc_all.size * K)),
            "finished_per_step": int(churn_finished(w, 0).sum())}


def latency_vs_depth(r, reps, depths=(1, 3, 7, 11)):
    """Draft latency against the draft depth K on the same requests and contexts: one parallel pass
    (pe_draft_step) against K autoregressive passes (pe_draft_ar), the comparison the pages make between
    parallel and autoregressive drafting. HIP events on the library stream."""
    from synth.device import config_args
    pe, torch, w = r.pe, r.torch, r.w
    s = w.shape
    depths = [k for k in depths if w.ctx[1] + k + 1 <= w.max_ctx]
    ctx = pe.pe_init(pe.make_config(**config_args(w, max_k=max(depths))), pe.make_weights(r.dev, s.n_layers),
                     pe.make_kv(r.kc, r.vc), r.stream.cuda_stream)
    out = {"B": w.B, "K": depths, "parallel_us": [], "autoregressive_us": []}
    d = r.d
    for K in depths:
        tok = torch.empty((w.B, K), dtype=torch.int32, device="cuda")
        for fn, key in ((pe.pe_draft_step, "parallel_us"), (pe.pe_draft_ar, "autoregressive_us")):
            def call():
                fn(ctx, w.B, K, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"], tok, None)
            for _ in range(3):
                call()
            out[key].append(1e3 * r.timed(call, reps) / reps)
    pe.pe_destroy(ctx)
    out["autoregressive_over_parallel"] = [a / p for a, p in zip(out["autoregressive_us"], out["parallel_us"])]
    return out


def variants(r, reps):
    """Catch-up, concatenated-row and FP8-weight draft steps on the same requests (opt-in)."""
    import dataclasses
    from synth.device import config_args, to_device, upload_weights
    from synth.inputs import catchup_inputs
    pe, torch, w = r.pe, r.torch, r.w
    s = w.shape
    d = r.d
    out = {}
    tok = torch.empty((w.B, w.K), dtype=torch.int32, device="cuda")
    max_k = min(16, 128 // (s.n_q_heads // s.n_kv_heads) - 1)
    R = min(w.K + 1, max_k + 1 - w.K)
    if R >= 1:
        ctx = pe.pe_init(pe.make_config(**config_args(w, max_k=R + w.K - 1)), pe.make_weights(r.dev, s.n_layers),
                         pe.make_kv(r.kc, r.vc), r.stream.cuda_stream)
        inp = catchup_inputs(w, R)
        nr, tk, hd = to_device(inp["n_real"], "i32"), to_device(inp["tokens"], "i32"), to_device(inp["target_hidden"], s.dtype)
        call = lambda: pe.pe_draft_catchup(ctx, w.B, w.K, R, d["req_slot"], d["seq_len"], nr, tk, hd, tok, None)
        call()
        out["catchup_step"] = {"R": R, "rows_per_request": R + w.K, "draft_us": 1e3 * r.timed(call, reps) / reps}
        pe.pe_destroy(ctx)
    sc = dataclasses.replace(s, name=s.name + "-concat", row_concat=True, weight_seed=s.weight_seed + 100)
    wc = dataclasses.replace(w, shape=sc)
    devc, _ = upload_weights(sc)
    ctx = pe.pe_init(pe.make_config(**config_args(wc)), pe.make_weights(devc, sc.n_layers), pe.make_kv(r.kc, r.vc),
                     r.stream.cuda_stream)
    call = lambda: pe.pe_draft_step(ctx, w.B, w.K, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"],
                                    tok, None)
    call()
    out["concat_rows_step"] = {"draft_us": 1e3 * r.timed(call, reps) / reps}
    pe.pe_destroy(ctx)
    del devc
    ctx = pe.pe_init(pe.make_config(**{**config_args(w), "weight_fp8": 1}), pe.make_weights(r.dev, s.n_layers),
                     pe.make_kv(r.kc, r.vc), r.stream.cuda_stream)
    call = lambda: pe.pe_draft_step(ctx, w.B, w.K, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"],
                                    tok, None)
    call()
    out["fp8_weights_step"] = {"draft_us": 1e3 * r.timed(call, reps) / reps}
    pe.pe_destroy(ctx)
    torch.cuda.empty_cache()
    return out


def copy_bandwidth(torch):
    """A plain 1 GiB device-to-device copy (read + write bytes / time): the part's measured streaming rate,
    reported beside the 8 TB/s peak."""
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * src.numel() * 2 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


# ------------------------------------------------------------------------------------------ CPU side

def host_info():
    info = {"nproc": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = int(blas[0].get("num_threads", 1))
    except Exception:  # threadpoolctl missing: the BLAS is not reported
        pass
    return info


def oracle_step(w, W64, state, T_host, req, K):
    """The oracle's draft step + verify + compaction for the requests `req` of workload w (requests are
    independent), on their own contexts."""
    from oracle import pe_oracle as O
    from synth.inputs import kv_block, to_f64
    s = w.shape
    seq = state["seq_len"][req]
    ctxs = {}

    def ctx(l, i):
        if (l, i) not in ctxs:
            b = req[i]
            ctxs[(l, i)] = (to_f64(kv_block(w, l, 0, b, int(seq[i])), s.dtype),
                            to_f64(kv_block(w, l, 1, b, int(seq[i])), s.dtype))
        return ctxs[(l, i)]

    for l in range(s.n_layers):  # contexts are inputs: generated before the timing
        for i in range(len(req)):
            ctx(l, i)
    st = {"last_token": state["last_token"][req], "target_hidden": to_f64(state["target_hidden"][req], s.dtype),
          "seq_len": seq}
    Tq = to_f64(T_host[req], s.dtype)
    t0 = time.perf_counter()
    out = O.draft_step(s, W64, st, ctx, K)
    v = O.verify(Tq, out["draft"])
    O.compact(v, state["req_slot"][req], seq)
    return time.perf_counter() - t0, out


def cpu_baseline(runs_cfg, budget_s):
    """The oracle as it stands (float64 NumPy, all BLAS threads), timed on this host: the median of three
    draft + verify + compaction runs over a sample of the headline workload's requests; plus the same with one
    thread on the tiny workload and the Qwen-shaped B 1 K 3 (median of five) and B 8 K 11 (one request,
    median of three) workloads. Also the argmax rule's strict-match and exempt counts of the
    GPU's drafts on the sampled requests."""
    from synth.inputs import make_weights, to_f64
    info = host_info()
    head = runs_cfg["headline"]
    w = head["w"]
    s = w.shape
    W64 = {k: to_f64(v, s.dtype) for k, v in make_weights(s).items()}
    n = 1
    dt, out = oracle_step(w, W64, head["state"], head["T_host"], [0], w.K)
    while n < w.B and dt * (n * 2) / n * 3 < budget_s:  # grow the sample while three runs fit the budget
        n *= 2
        dt, out = oracle_step(w, W64, head["state"], head["T_host"], list(range(n)), w.K)
    req = list(range(n))
    times = [dt] + [oracle_step(w, W64, head["state"], head["T_host"], req, w.K)[0] for _ in range(2)]
    med = float(np.median(times))
    tol = 2e-2 if s.dtype == "bf16" else 1e-4
    z = out["logits"].reshape(-1, s.vocab)
    tok = head["draft"][req].reshape(-1)
    srt = np.sort(z, axis=-1)
    exempt = (srt[:, -1] - srt[:, -2]) < tol * np.abs(z).max(-1)
    strict = tok == np.argmax(z, axis=-1)
    res = {"value": n * w.K / med, "unit": "draft tokens/s", "cores": info.get("blas_threads", info["nproc"]),
           "kind": "oracle",
           "sample": f"{n} of the {w.B} requests of {w.name} (K {w.K}) as one batch: float64 NumPy draft step + "
                     f"verify + compaction, median of 3 runs ({', '.join(f'{t:.2f}' for t in times)} s)",
           "steps_per_s_of_sample": 1.0 / med, "host": info,
           "argmax_rule": {"rows": int(z.shape[0]), "strict_match": int(strict.sum()), "exempt": int(exempt.sum()),
                           "strict_rate": float(strict.mean())}}
    del W64
    one = {}
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # threadpoolctl missing: no one-thread runs
        threadpool_limits = None
    if threadpool_limits is not None:
        from synth import WORKLOADS, TINY_FP32, make_state, plant_target_logits, random_draft
        cases = [("tiny-fp32-B1-K4-L64", None), ("qwen3coder-bf16-B1-K3-L2048", None),
                 ("qwen3coder-bf16-B8-K11-L1024to4096", [0])]
        Wq = None
        for name, sub in cases:
            wc = WORKLOADS[name]
            if wc.shape is TINY_FP32:
                Wc = {k: to_f64(v, wc.shape.dtype) for k, v in make_weights(wc.shape).items()}
            else:
                if Wq is None:
                    Wq = {k: to_f64(v, wc.shape.dtype) for k, v in make_weights(wc.shape).items()}
                Wc = Wq
            stc = make_state(wc)
            Tc = plant_target_logits(wc, random_draft(wc), stc["alpha"])
            rq = sub or list(range(wc.B))
            nrun = 3 if sub else 5  # the two single-request workloads: median of five runs
            with threadpool_limits(limits=1):
                ts = [oracle_step(wc, Wc, stc, Tc, rq, wc.K)[0] for _ in range(nrun)]
            one[name] = {"requests": len(rq), "median_s": float(np.median(ts)), "runs": nrun,
                         "draft_tokens_per_s": len(rq) * wc.K / float(np.median(ts)), "threads": 1}
        del Wq
    res["one_thread"] = one
    return res


# ----------------------------------------------------------------------------------------------- main

def measure(r, steps, warmup, reps):
    """Timed whole steps (no events inside), per-step distribution, draft / verify alone, kernel pass."""
    for _ in range(warmup):
        r.step()
    wall0 = time.perf_counter()
    ms = r.timed(r.step, steps)
    wall = time.perf_counter() - wall0
    out = {"ms_per_step": ms / steps, "wall_ms_per_step": 1e3 * wall / steps,
           "step_us": r.per_call(r.step, reps), "draft_us": r.per_call(r.draft_call, reps),
           "verify_us": r.per_call(r.verify_call, reps)}
    r.verify_sampled_call()
    out["verify_sampled_us"] = r.per_call(r.verify_sampled_call, reps)
    r.verify_call()  # leave the greedy verify's outputs (accept lengths) in place
    out["kernels"] = r.kernel_times(max(10, reps // 5))
    out["rooflines"] = r.rooflines(out["kernels"])
    return out


def target_entry(r, m):
    w = r.w
    ab = algorithmic_bytes(w, r.state)
    t_draft = m["draft_us"]["median"]
    e = {"workload": w.name, "B": w.B, "K": w.K, "ms_per_step": m["ms_per_step"],
         "step_us": m["step_us"], "t_draft_us": m["draft_us"], "t_verify_us": m["verify_us"],
         "t_verify_sampled_us": m["verify_sampled_us"],
         "draft_tokens_per_s": w.B * w.K / (m["ms_per_step"] * 1e-3), "steps_per_s": 1e3 / m["ms_per_step"],
         "draft_hbm_frac": ab["draft"] / (t_draft * 1e-6) / (PEAK_HBM_GBS * 1e9),
         "algorithmic_MB": {k: v / 1e6 for k, v in ab.items()},
         "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()
                         if kk in ("avg_launch_us", "launches", "bound", "frac", "hbm_frac", "mfma_frac")}
                     for k, v in m["rooflines"].items()}}
    acc = r.outs[0].cpu().numpy()
    e["mean_accept_len"] = float(acc.mean())
    e["alpha_hat"] = float((acc - 1).sum() / (acc.size * w.K))
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=100, help="calls timed one by one for the distributions")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-targets", action="store_true", help="skip the target workloads (e.g. under a profiler)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--churn-steps", type=int, default=16)
    ap.add_argument("--variants", action="store_true",
                    help="also time catch-up, concatenated-row and FP8 steps (headline workload and the B = 1 target)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="start with the 1 GiB device copy (the known-size kernel that scales HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: this path runs on one GPU (each request's draft and verify are independent; "
              f"scale-out is data-parallel over requests and is not built). --gpus {args.gpus} is not supported.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import eagle_drafting_amd as pe
    torch.cuda.set_device(0)

    def note(msg):
        print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)

    copy_gbs = copy_bandwidth(torch) if args.copy_calibration else None
    note(f"headline {args.workload}")
    r = Run(pe, torch, args.workload)
    w, s = r.w, r.w.shape
    m = measure(r, args.steps, args.warmup, args.reps)
    ab = algorithmic_bytes(w, r.state)
    acc = r.outs[0].cpu().numpy()
    rl = m["rooflines"]
    dominant = max(("lm_head", "attention", "gate_up", "qkv", "down", "o_proj"),
                   key=lambda k: rl[k]["avg_launch_us"] * rl[k]["launches"])
    roof = dict(rl[dominant])
    roof["kernel"] = dominant
    roof["traffic"] = traffic_from_profile(dominant, w.name)
    headline_cpu = {"w": w, "state": r.state, "T_host": r.T_host, "draft": r.draft.cpu().numpy()}
    result = {
        "metric": METRIC,
        "value": w.B * w.K / (m["ms_per_step"] * 1e-3),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) hiddens/KV, planted target logits)",
        "config": {"workload": w.name, "drafter_shape": s.name, "B": w.B, "K": w.K, "context": list(w.ctx),
                   "layers": s.n_layers, "d": s.d_model, "vocab": s.vocab},
        "steps_per_s": 1e3 / m["ms_per_step"],
        "request_steps_per_s": w.B * 1e3 / m["ms_per_step"],
        "wall_ms_per_step": m["wall_ms_per_step"],
        "step_us": m["step_us"],
        "t_draft_us": m["draft_us"],
        "t_verify_us": m["verify_us"],
        "t_verify_sampled_us": m["verify_sampled_us"],
        "step_hbm_frac": ab["step"] / (m["ms_per_step"] * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "draft_hbm_frac": ab["draft"] / (m["draft_us"]["median"] * 1e-6) / (PEAK_HBM_GBS * 1e9),
        "algorithmic_MB": {k: v / 1e6 for k, v in ab.items()},
        "mean_accept_len": float(acc.mean()),
        "alpha_hat": float((acc - 1).sum() / (acc.size * w.K)),
        "roofline": roof,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()
                        if kk in ("avg_launch_us", "launches", "bound", "frac", "hbm_frac", "mfma_frac")}
                    for k, v in rl.items()},
        "device_flags": pe.pe_device_flags(r.ctx),
    }
    if args.variants:
        note("variants on the headline workload")
        result["variants"] = variants(r, max(10, args.steps // 2))
    r.close()
    del r

    if not args.no_targets:
        targets = {}
        qwen_dev = None
        for key, name in TARGET_WORKLOADS.items():
            note(f"target {name}")
            from synth import WORKLOADS
            from synth.device import upload_weights
            if qwen_dev is None:
                qwen_dev = upload_weights(WORKLOADS[name].shape)[0]
            rt = Run(pe, torch, name, weights=qwen_dev)
            mt = measure(rt, args.steps, args.warmup, args.reps)
            e = target_entry(rt, mt)
            if rt.w.B <= 8:
                e["target"] = {"what": "draft step >= 60 % of the 8 TB/s roofline",
                               "t_draft_max_us": algorithmic_bytes(rt.w, rt.state)["draft"] / (HBM_TARGET * PEAK_HBM_GBS * 1e9) * 1e6,
                               "met": e["draft_hbm_frac"] >= HBM_TARGET}
            if rt.w.B == 1:
                e["draft_latency_vs_depth"] = latency_vs_depth(rt, max(10, args.steps // 2))
                if args.variants:
                    e.update(variants(rt, max(10, args.steps // 2)))
            if rt.w.B >= 128:
                ks = e["kernels"]
                e["target"] = {"what": "LM-head and MLP GEMMs >= 50 % of the bf16 MFMA peak",
                               "lm_head_mfma_frac": ks["lm_head"]["mfma_frac"],
                               "gate_up_mfma_frac": ks["gate_up"]["mfma_frac"],
                               "down_mfma_frac": ks["down"]["mfma_frac"],
                               "lm_head_max_us": gemm_flops(rt.w)["lm_head"] / (MFMA_TARGET * PEAK_BF16_TFLOPS * 1e12) * 1e6,
                               "gate_up_max_us": gemm_flops(rt.w)["gate_up"] / (MFMA_TARGET * PEAK_BF16_TFLOPS * 1e12) * 1e6,
                               "met": min(ks["lm_head"]["mfma_frac"], ks["gate_up"]["mfma_frac"],
                                          ks["down"]["mfma_frac"]) >= MFMA_TARGET}
                note(f"churn run {args.churn_steps} steps")
                e["churn_run"] = churn_run(rt, args.churn_steps)
            targets[key] = e
            rt.close()
            del rt
        del qwen_dev
        torch.cuda.empty_cache()
        result["targets"] = targets
        result["hbm_copy_GBps"] = copy_bandwidth(torch)
    elif copy_gbs is not None:
        result["hbm_copy_GBps"] = copy_gbs
    if not args.no_cpu_baseline:
        note("cpu baseline")
        result["cpu_baseline"] = cpu_baseline({"headline": headline_cpu}, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
