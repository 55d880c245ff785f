"""Diagnostic (test infrastructure): how far bf16 activations alone move the drafter from the float64 oracle.

The bf16 drafter's kernels keep the residual stream, every accumulation and the softmax statistics in
float32, and round to bf16 at these points only: the normalised operand of every normalised projection
(x * g before the 1/RMS row scale), the rotated queries, the cache keys and values, the unnormalised
softmax weights of the attention's value product, the attention output and the SwiGLU output. This script
runs the oracle's forward with bf16 round-to-nearest-even at exactly those points (float64 everywhere else,
softmax weights relative to the row's global maximum) and reports, per layer, the largest per-(row, kv head)
relative K/V difference and the largest per-row relative logit difference against the plain oracle, both
for all points together and for each point alone.

  python -m oracle.bf16_rounding_budget [B K R]   (default: the 15-row catch-up case B 8 K 7 R 8)

It is not used by any test; its numbers are quoted where the K/V tolerance of the catch-up test is
discussed. Runs on the CPU in well under a minute (a few requests of the Qwen3-Coder-shaped drafter).
"""

from __future__ import annotations

import math
import os
import sys

import numpy as np

if __package__ in (None, ""):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle import pe_oracle as O  # noqa: E402

POINTS = ("xg", "q", "kv", "p", "o", "a")


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of float values, via float32 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32).astype(np.float64)


def draft_rows_bf16_points(shape, W, X, seq_len, kv_context, points=POINTS):
    """The oracle's draft_rows with bf16 rounding at the given points (see the module docstring)."""
    B, K, d = X.shape
    Hq, Hkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    G = Hq // Hkv
    eps = shape.rms_eps
    rb = (lambda name, v: round_bf16(v) if name in points else v)
    x = X.reshape(B * K, d).astype(np.float64, copy=True)
    pos = (np.asarray(seq_len, dtype=np.int64)[:, None] + np.arange(K)[None, :]).reshape(-1)

    def normed(v, g):
        # the kernels' form of RMSNorm: (bf16(x * g) . W) * 1/RMS(x)
        return rb("xg", v * g), 1.0 / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)

    k_all, v_all = [], []
    for l in range(shape.n_layers):
        xg, r = normed(x, W[f"l{l}.attn_norm"])
        qkv = O.linear(xg, W[f"l{l}.wqkv"]) * r
        q = O.rope(qkv[:, : Hq * hd].reshape(B * K, Hq, hd), pos, shape.rope_base)
        k = O.rope(qkv[:, Hq * hd: (Hq + Hkv) * hd].reshape(B * K, Hkv, hd), pos, shape.rope_base)
        v = qkv[:, (Hq + Hkv) * hd:].reshape(B * K, Hkv, hd)
        q, k, v = rb("q", q), rb("kv", k), rb("kv", v)
        o = np.empty_like(q)
        for b in range(B):
            k_ctx, v_ctx = kv_context(l, b)
            L = k_ctx.shape[1]
            for h in range(Hq):
                g = h // G
                keys = np.concatenate([k_ctx[g], k[b * K:(b + 1) * K, g]], axis=0)
                vals = np.concatenate([v_ctx[g], v[b * K:(b + 1) * K, g]], axis=0)
                for j in range(K):
                    s = keys[: L + j + 1] @ q[b * K + j, h] / math.sqrt(hd)
                    p = np.exp(s - s.max())
                    o[b * K + j, h] = (rb("p", p) @ vals[: L + j + 1]) / p.sum()
        x = x + O.linear(rb("o", o).reshape(B * K, Hq * hd), W[f"l{l}.wo"])
        xg, r = normed(x, W[f"l{l}.mlp_norm"])
        a = rb("a", O.silu(O.linear(xg, W[f"l{l}.wgate"]) * r) * (O.linear(xg, W[f"l{l}.wup"]) * r))
        x = x + O.linear(a, W[f"l{l}.wdown"])
        k_all.append(k.reshape(B, K, Hkv, hd))
        v_all.append(v.reshape(B, K, Hkv, hd))
    xg, r = normed(x, W["final_norm"])
    return {"logits": (O.linear(xg, W["lm_head"]) * r).reshape(B, K, -1), "k_new": k_all, "v_new": v_all}


def _per_head(a, b):
    return np.abs(a - b).max(-1) / np.abs(b).max(-1)


def main(argv):
    from synth import QWEN3_CODER, Workload, make_state
    from synth.inputs import catchup_inputs, kv_block, make_weights, to_f64
    B, K, R = (int(v) for v in argv[:3]) if len(argv) >= 3 else (8, 7, 8)
    # the catch-up parity test's workload of the same (B, K, R)
    w = Workload(f"qwen3coder-bf16-B{B}-K{K}-R{R}-catchup", QWEN3_CODER, B, K, (60, 400), 0.7, 7800 + 40 * B + K + R)
    s = w.shape
    W = {k: to_f64(v, s.dtype) for k, v in make_weights(s).items()}
    st = make_state(w)
    inp = catchup_inputs(w, R)
    req = list(range(B)) if B <= 4 else sorted({0, 1, B // 2, B - 1})
    seq = st["seq_len"][req]

    def ctx(l, i):
        return (to_f64(kv_block(w, l, 0, req[i], int(seq[i])), s.dtype),
                to_f64(kv_block(w, l, 1, req[i], int(seq[i])), s.dtype))

    X = O.build_rows_catchup(W, inp["tokens"][req], to_f64(inp["target_hidden"][req], s.dtype),
                             inp["n_real"][req], K)
    ref = O.draft_rows(s, W, X, seq, ctx)
    print(f"{w.name}: requests {req}, n_real {inp['n_real'][req].tolist()}, {X.shape[1]} rows each")
    for pts in [POINTS] + [(p,) for p in POINTS]:
        f = draft_rows_bf16_points(s, W, X, seq, ctx, pts)
        zl = np.abs(f["logits"] - ref["logits"]).max(-1) / np.abs(ref["logits"]).max(-1)
        kv = " ".join(f"l{l} {max(_per_head(f['k_new'][l], ref['k_new'][l]).max(), _per_head(f['v_new'][l], ref['v_new'][l]).max()):.2e}"
                      for l in range(s.n_layers))
        print(f"  bf16 at {'+'.join(pts):16s} logits {zl.max():.2e} | K/V per head {kv}")


if __name__ == "__main__":
    main(sys.argv[1:])
