"""Benchmark of the P-EAGLE parallel draft step + greedy verify on one MI355X.

One step = pe_draft_step (row build, 4 drafter layers, LM head, argmax: K draft tokens for each of B
requests in one pass) + pe_verify (target argmax over K+1 positions, accepted prefix, bonus token,
batch-metadata rebuild), over inputs already resident in HBM. Prints one JSON line.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload NAME] [--no-cpu-baseline] [--no-depth-sweep]

The default workload is the Qwen3-Coder-30B-A3B-shaped bf16 drafter at B = 1, K = 3, context 2048.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE = "qwen3coder-bf16-B1-K3-L2048"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "draft tokens/s and draft+verify steps/s at B×K; % of HBM/MFMA roofline"


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
    kv_read = s.n_layers * int((L + w.K).sum()) * kv_row
    kv_write = s.n_layers * w.B * w.K * kv_row
    inputs = w.B * d * e + w.B * 3 * d * e
    draft = weights + kv_read + kv_write + inputs
    verify = w.B * (w.K + 1) * V * e
    lm_head = d * V * e
    return {"draft": draft, "verify": verify, "step": draft + verify, "lm_head": lm_head,
            "weights": weights, "kv_read": kv_read}


def lm_head_flops(w):
    return 2.0 * w.B * w.K * w.shape.d_model * w.shape.vocab


def lm_head_roofline(w, ab, lm_us, lm_n, traffic):
    """Roofline of the dominant kernel, the LM head: one weight read of V x d bf16 and 2 (B K) d V flops
    per launch. Its intensity is B K flop per byte, so it is bound by HBM below the ridge
    (2.5 PFLOP/s / 8 TB/s = 312.5 rows) and by the bf16 MFMA rate above it."""
    secs = lm_us * 1e-6
    gbs = ab["lm_head"] / secs / 1e9
    tflops = lm_head_flops(w) / secs / 1e12
    mfma = w.B * w.K > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    r = {"bound": "mfma" if mfma else "hbm",
         "kernel": "LM-head GEMM with fused argmax partials",
         "achieved": tflops if mfma else gbs,
         "peak": PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBS,
         "unit": "TFLOP/s" if mfma else "GB/s",
         "traffic": traffic,
         "bytes_per_launch": ab["lm_head"],
         "flops_per_launch": lm_head_flops(w),
         "avg_launch_us": lm_us,
         "launches": lm_n,
         "hbm_frac": gbs / PEAK_HBM_GBS,
         "mfma_frac": tflops / PEAK_BF16_TFLOPS}
    r["frac"] = r["achieved"] / r["peak"]
    return r


def latency_vs_depth(pe, torch, w, cfg_args, dev, kc, vc, d, stream, reps, depths=(1, 3, 7, 11)):
    """Draft latency against the draft depth K on the same requests and contexts: one parallel pass
    (pe_draft_step) against K autoregressive passes (pe_draft_ar), the comparison the pages make between
    parallel and autoregressive drafting. Timed with HIP events on the library stream, outside the
    step's timed region. bf16 drafters only (the autoregressive entry point needs one)."""
    s = w.shape
    if s.dtype != "bf16":
        return None
    depths = [k for k in depths if w.ctx[1] + k + 1 <= w.max_ctx]
    ctx = pe.pe_init(pe.make_config(**cfg_args(w, max_k=max(depths))), pe.make_weights(dev, s.n_layers),
                     pe.make_kv(kc, vc), stream.cuda_stream)
    out = {"B": w.B, "K": depths, "parallel_us": [], "autoregressive_us": []}
    for K in depths:
        tok = torch.empty((w.B, K), dtype=torch.int32, device="cuda")
        for fn, key in ((pe.pe_draft_step, "parallel_us"), (pe.pe_draft_ar, "autoregressive_us")):
            def call():
                fn(ctx, w.B, K, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"], tok, None)
            for _ in range(3):
                call()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            out[key].append(1e3 * e0.elapsed_time(e1) / reps)
    pe.pe_destroy(ctx)
    out["autoregressive_over_parallel"] = [a / p for a, p in zip(out["autoregressive_us"], out["parallel_us"])]
    return out


def catchup_latency(pe, torch, w, cfg_args, dev, kc, vc, d, stream, reps):
    """Latency of a multi-row catch-up step (pe_draft_catchup) beside the plain step on the same requests:
    R = K + 1 token / hidden pairs per request (room for a fully accepted previous step; fewer where the
    config's largest max_k, 16 and 128 query rows per kv head, caps R + K - 1), real-row counts drawn
    uniformly in 1..R, so every request runs R + K rows. bf16 drafters only."""
    from synth.device import to_device
    from synth.inputs import catchup_inputs
    s = w.shape
    if s.dtype != "bf16":
        return None
    K = w.K
    max_k = min(16, 128 // (s.n_q_heads // s.n_kv_heads) - 1)
    R = min(K + 1, max_k + 1 - K)
    if R < 1:
        return None
    ctx = pe.pe_init(pe.make_config(**cfg_args(w, max_k=R + K - 1)), pe.make_weights(dev, s.n_layers),
                     pe.make_kv(kc, vc), stream.cuda_stream)
    inp = catchup_inputs(w, R)
    n_real = to_device(inp["n_real"], "i32")
    tokens = to_device(inp["tokens"], "i32")
    hid = to_device(inp["target_hidden"], s.dtype)
    tok = torch.empty((w.B, K), dtype=torch.int32, device="cuda")
    out = {"B": w.B, "K": K, "R": R, "rows_per_request": R + K, "mean_n_real": float(inp["n_real"].mean())}
    calls = {"catchup_us": lambda: pe.pe_draft_catchup(ctx, w.B, K, R, d["req_slot"], d["seq_len"], n_real, tokens,
                                                        hid, tok, None),
             "plain_step_us": lambda: pe.pe_draft_step(ctx, w.B, K, d["req_slot"], d["seq_len"], d["last_token"],
                                                       d["target_hidden"], tok, None)}
    for key, call in calls.items():
        for _ in range(3):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        out[key] = 1e3 * e0.elapsed_time(e1) / reps
    pe.pe_destroy(ctx)
    return out


def concat_rows_latency(pe, torch, w, cfg_args, kc, vc, d, stream, reps):
    """Latency of the draft step with concatenated input rows ([embedding || hidden] into layer 0's
    attention; its QKV reads 2d columns) beside the same workload's summed rows: a drafter of the same
    shape with row_concat set (own seeded weights), the same requests and contexts. bf16 drafters only."""
    import dataclasses
    from synth.device import upload_weights
    s = w.shape
    if s.dtype != "bf16":
        return None
    sc = dataclasses.replace(s, name=s.name + "-concat", row_concat=True, weight_seed=s.weight_seed + 100)
    wc = dataclasses.replace(w, shape=sc)
    dev, _ = upload_weights(sc)
    ctx = pe.pe_init(pe.make_config(**cfg_args(wc)), pe.make_weights(dev, sc.n_layers), pe.make_kv(kc, vc),
                     stream.cuda_stream)
    tok = torch.empty((w.B, w.K), dtype=torch.int32, device="cuda")

    def call():
        pe.pe_draft_step(ctx, w.B, w.K, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"], tok, None)
    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    pe.pe_destroy(ctx)
    del dev
    return {"B": w.B, "K": w.K, "draft_us": 1e3 * e0.elapsed_time(e1) / reps}


def fp8_weights_latency(pe, torch, w, cfg_args, dev, kc, vc, d, stream, reps):
    """Draft step with FP8 drafter weights (weight_fp8: E4M3 codes with per-row scales, half the weight
    bytes) on the same requests, beside the bf16 step. Reports the step and the LM head's average launch."""
    s = w.shape
    if s.dtype != "bf16":
        return None
    ctx = pe.pe_init(pe.make_config(**{**cfg_args(w), "weight_fp8": 1}), pe.make_weights(dev, s.n_layers),
                     pe.make_kv(kc, vc), stream.cuda_stream)
    tok = torch.empty((w.B, w.K), dtype=torch.int32, device="cuda")

    def call():
        pe.pe_draft_step(ctx, w.B, w.K, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"], tok, None)
    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    pe.pe_profile_enable(ctx, 1 << pe.PE_PROF_LM_HEAD)
    for _ in range(reps):
        call()
    lm_ms, lm_n = pe.pe_profile_read(ctx, pe.PE_PROF_LM_HEAD)
    pe.pe_destroy(ctx)
    lm_us = 1e3 * lm_ms / max(lm_n, 1)
    lm_bytes = s.vocab * s.d_model + s.vocab * 4  # E4M3 codes + one float32 scale per row
    return {"B": w.B, "K": w.K, "draft_us": 1e3 * e0.elapsed_time(e1) / reps, "lm_head_us": lm_us,
            "lm_head_GBps": lm_bytes / (lm_us * 1e-6) / 1e9}


def kernel_source_digest():
    """sha256 over the sources that define the projection kernels (the LM head among them)."""
    h = hashlib.sha256()
    for name in ("gemm.hip", "kernels.h", "common.h"):
        h.update(open(os.path.join(ROOT, "eagle_drafting_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def traffic_from_profile(workload_name):
    """HBM bytes per LM-head launch measured by rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, scaled by
    the plain-copy calibration), if the committed measurement was taken with the current kernel source."""
    path = os.path.join(ROOT, "profiles", "lm_head_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("workload") != workload_name or rec.get("kernel_src_sha256") != kernel_source_digest():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, state, target_logits_host, target_seconds):
    """The oracle, as it stands, on this host: repeated draft + verify + compact steps of the same
    workload until about target_seconds of work."""
    from oracle import pe_oracle as O
    from synth.inputs import kv_block, make_weights, to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the visible CPUs
        threads = os.cpu_count() or 1
    s = w.shape
    W = {k: to_f64(v, s.dtype) for k, v in make_weights(s).items()}
    ctx_cache = {}

    def ctx(l, b):
        if (l, b) not in ctx_cache:
            L = int(state["seq_len"][b])
            ctx_cache[(l, b)] = (to_f64(kv_block(w, l, 0, b, L), s.dtype), to_f64(kv_block(w, l, 1, b, L), s.dtype))
        return ctx_cache[(l, b)]

    for l in range(s.n_layers):
        for b in range(w.B):
            ctx(l, b)
    st = {"last_token": state["last_token"], "target_hidden": to_f64(state["target_hidden"], s.dtype),
          "seq_len": state["seq_len"]}
    T = to_f64(target_logits_host, s.dtype)
    n, t0 = 0, time.perf_counter()
    while True:
        out = O.draft_step(s, W, st, ctx, w.K)
        v = O.verify(T, out["draft"])
        O.compact(v, state["req_slot"], state["seq_len"])
        n += 1
        el = time.perf_counter() - t0
        if el >= target_seconds or n >= 200:
            break
    return {"value": w.B * w.K * n / el, "unit": "draft tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} full draft+verify steps of {w.name} (float64 NumPy oracle), {el:.1f} s",
            "steps_per_s": n / el}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the catch-up and concatenated-row timings (e.g. under a profiler)")
    ap.add_argument("--no-depth-sweep", action="store_true",
                    help="skip the parallel vs autoregressive latency sweep over K (e.g. under a profiler)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference kernel for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: this path runs on one GPU (each request's draft and verify are independent; "
              f"scale-out is data-parallel over requests and is not built). --gpus {args.gpus} is not supported.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import eagle_drafting_amd as pe
    from synth import WORKLOADS, churn_finished, make_state, plant_target_logits
    from synth.device import config_args, to_device, upload_kv, upload_state, upload_weights

    w = WORKLOADS[args.workload]
    s = w.shape
    torch.cuda.set_device(0)
    dev, _ = upload_weights(s)
    state = make_state(w)
    kc, vc = upload_kv(w, state)
    d = upload_state(state, s.dtype)
    stream = torch.cuda.current_stream()
    ctx = pe.pe_init(pe.make_config(**config_args(w)), pe.make_weights(dev, s.n_layers), pe.make_kv(kc, vc),
                     stream.cuda_stream)
    B, K, V = w.B, w.K, s.vocab
    i32 = dict(dtype=torch.int32, device="cuda")
    draft = torch.empty((B, K), **i32)
    outs = [torch.empty(n, **i32) for n in (B, B + 1, B * (K + 1), B, 1, B, B, B)]

    # target logits planted on this drafter's own draft tokens (the draft is deterministic, so every
    # timed step sees the same acceptance pattern)
    pe.pe_draft_step(ctx, B, K, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"], draft, None)
    torch.cuda.synchronize()
    draft_host = draft.cpu().numpy()
    T_host = plant_target_logits(w, draft_host, state["alpha"])
    T = to_device(T_host, s.dtype)
    fin = to_device(churn_finished(w, 0), "u8") if w.churn else None

    def draft_call():
        pe.pe_draft_step(ctx, B, K, d["req_slot"], d["seq_len"], d["last_token"], d["target_hidden"], draft, None)

    def verify_call():
        pe.pe_verify(ctx, B, K, T, draft, fin, d["req_slot"], d["seq_len"], *outs)

    for _ in range(args.warmup):
        draft_call()
        verify_call()
    pe.pe_profile_enable(ctx, 1 << pe.PE_PROF_LM_HEAD)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        draft_call()
        verify_call()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev0.elapsed_time(ev1)
    lm_ms, lm_n = pe.pe_profile_read(ctx, pe.PE_PROF_LM_HEAD)
    ms_step = ms / args.steps
    accept = outs[0].cpu().numpy()

    # breakdown (outside the timed region): draft alone, verify alone, then per-kernel events
    pe.pe_profile_enable(ctx, 0)
    reps = max(10, args.steps // 2)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    for _ in range(reps):
        draft_call()
    e[1].record(stream)
    for _ in range(reps):
        verify_call()
    e[2].record(stream)
    torch.cuda.synchronize()
    t_draft = e[0].elapsed_time(e[1]) / reps
    t_verify = e[1].elapsed_time(e[2]) / reps
    pe.pe_profile_enable(ctx, (1 << 4) - 1)
    for _ in range(reps):
        draft_call()
        verify_call()
    kern = {}
    for name, kid in (("lm_head", pe.PE_PROF_LM_HEAD), ("attention", pe.PE_PROF_ATTENTION),
                      ("gate_up", pe.PE_PROF_GATE_UP), ("verify_scan", pe.PE_PROF_VERIFY_SCAN)):
        tot, n = pe.pe_profile_read(ctx, kid)
        kern[name] = {"avg_us": 1e3 * tot / max(n, 1), "launches": n}
    pe.pe_profile_enable(ctx, 0)

    # verify in its sampling form at temperature 0.3 (the pages' example request), seeded uniforms
    rng = np.random.default_rng(w.seed + 23)
    u_s = torch.from_numpy(rng.random((B, K), dtype=np.float32)).cuda()
    v_s = torch.from_numpy(rng.random((B, K + 1), dtype=np.float32)).cuda()

    def verify_sampled_call():
        pe.pe_verify_sampled(ctx, B, K, T, draft, 0.3, u_s, v_s, fin, d["req_slot"], d["seq_len"], *outs)

    for _ in range(3):
        verify_sampled_call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        verify_sampled_call()
    e1.record(stream)
    torch.cuda.synchronize()
    t_verify_sampled = e0.elapsed_time(e1) / reps

    depth = None if args.no_depth_sweep else latency_vs_depth(pe, torch, w, config_args, dev, kc, vc, d, stream, reps)
    catchup = concat = fp8 = None
    if not args.no_variants:
        catchup = catchup_latency(pe, torch, w, config_args, dev, kc, vc, d, stream, reps)
        concat = concat_rows_latency(pe, torch, w, config_args, kc, vc, d, stream, reps)
        fp8 = fp8_weights_latency(pe, torch, w, config_args, dev, kc, vc, d, stream, reps)

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    flags = pe.pe_device_flags(ctx)
    pe.pe_destroy(ctx)

    ab = algorithmic_bytes(w, state)
    lm_us = 1e3 * lm_ms / max(lm_n, 1)
    traffic = traffic_from_profile(w.name)
    result = {
        "metric": METRIC,
        "value": B * K / (ms_step * 1e-3),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) hiddens/KV, planted target logits)",
        "config": {"workload": w.name, "drafter_shape": s.name, "B": B, "K": K,
                   "context": list(w.ctx), "layers": s.n_layers, "d": s.d_model, "vocab": V},
        "steps_per_s": 1e3 / ms_step,
        "request_steps_per_s": B * 1e3 / ms_step,
        "wall_ms_per_step": 1e3 * wall / args.steps,
        "t_draft_us": 1e3 * t_draft,
        "t_verify_us": 1e3 * t_verify,
        "t_verify_sampled_us": 1e3 * t_verify_sampled,
        "step_hbm_frac": ab["step"] / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "draft_hbm_frac": ab["draft"] / (t_draft * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "algorithmic_MB": {k: v / 1e6 for k, v in ab.items()},
        "mean_accept_len": float(accept.mean()),
        "alpha_hat": float((accept - 1).sum() / (accept.size * K)),
        "kernels": kern,
        "roofline": lm_head_roofline(w, ab, lm_us, lm_n, traffic),
        "device_flags": flags,
        "draft_latency_vs_depth": depth,
        "catchup_step": catchup,
        "concat_rows_step": concat,
        "fp8_weights_step": fp8,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, state, T_host, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
