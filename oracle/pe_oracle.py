"""CPU oracle of the P-EAGLE parallel draft step and the greedy verify step. TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this module. The GPU
path never calls it; it shares no code with the HIP kernels or their host library.

Everything is computed in float64 with plain NumPy, in the order the method describes. Sources (page
titles; sections):
  [AWS-P]  "Parallelize speculative decoding with P-EAGLE on Amazon SageMaker AI" (Chinese translation of
           the AWS post): solution overview -> "sequential dependency in autoregressive EAGLE",
           "how P-EAGLE breaks the chain", "step-by-step drafting process".
  [AWS-S]  Korean summary of the same post, detail items 3 (core idea) and 8 (internals).
  [LESSON] "EAGLE-3 speculative decoding in production" (Korean lesson): concept section (speedup
           formula and worked example), break-even section, production recipe (alpha measurement).
  [JP]     Japanese commentary on the same AWS post, section "implementation and performance" (fused
           kernels that rebuild the batch metadata).

Readings where the pages leave a step open (each is listed with its reason in the design notes):
  * row 0 = fc(concat(h_low, h_mid, h_high)) + E[last_token] (a sum, not a concatenation);
    rows 1..K-1 = h_shared + emb_mask, without fc;
  * decoder layer = pre-RMSNorm GQA attention + pre-RMSNorm SwiGLU MLP, residual stream, no biases;
  * RoPE: rotate-half pairs (i, i + hd/2), inv_freq_i = base^(-2i/hd), position of row j = L_b + j;
    cached context keys are already rotated;
  * row j attends to the L_b context positions and to new rows 0..j (causal inside the K block);
    q head h reads kv head floor(h / G);
  * LM head is untied; draft token = argmax with ties to the lowest index;
  * verify is greedy exact match; the bonus token comes from the same target pass;
  * the drafter's cache after verify keeps positions L_b .. L_b + accept_len - 1 (verify advances seq_len
    by accept_len). accept_len can be K + 1, so a step that is followed by verify also runs one more
    placeholder row at position L_b + K (after the K draft rows, so it changes none of them) and keeps
    only its K/V: draft_step(..., tail=True).

  * concatenated rows (the variant that follows the pages' word "concatenated" literally): row =
    [embedding || hidden], 2d wide into layer 0's attention, each half RMS-normalised with its own gain,
    and the hidden half alone is the residual stream (the pages do not say which part carries the
    residual; the hidden half is the one that has the model's width and meaning);
  * FP8 drafter weights: every projection matrix stored as E4M3 codes with one float32 scale per output
    row (largest magnitude / 448), the product y = s_n * (q_n . x); activations, norms, embeddings and
    the KV cache stay bf16 / fp32. The pages give FP8 as the deployment precision of the target, not
    the drafter's scaling scheme; per-row scales are the plainest reading;
  * multi-row catch-up (a step that first re-runs the positions a verify accepted): each real row pairs
    an emitted token with the target hidden states that produced it, as the pages' position 1 does for
    the one token; the pages do not describe this step, so its logits are parity unpinned against the
    pages (pinned against the separately written single-row passes and against the plain step);
  * autoregressive drafting (the baseline parallel drafting replaces) feeds back the drafter's hidden
    state after its last layer (before the final norm) plus the embedding of the token it just drafted;
    the pages name the dependency but not which hidden state, so this reading is parity unpinned
    against the pages (it is pinned against the separately written loop-by-loop pass).

Parity status: each function below is pinned by tests under tests/ (closed forms, invariants, special
cases, brute force on tiny inputs). The full-step logit values have no printed worked example on the
pages; beyond the invariants they are pinned by the separately written sequential single-row step.
"""

from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------------------------------
# [LESSON] concept section: tokens per target pass = 1 + K*alpha; speedup = (1 + K*alpha) / (1 + eps)
# [LESSON] break-even section: S = 1  <=>  alpha = eps / K


def tokens_per_target_pass(K: int, alpha: float) -> float:
    return 1.0 + K * alpha


def speedup(K: int, alpha: float, eps: float) -> float:
    return tokens_per_target_pass(K, alpha) / (1.0 + eps)


def breakeven_alpha(eps: float, K: int) -> float:
    return eps / K


def alpha_hat(accept_len: np.ndarray, K: int) -> float:
    """[LESSON] production recipe: alpha = accepted draft tokens per request / draft length.
    accept_len counts the bonus token, so accepted drafts = accept_len - 1."""
    a = np.asarray(accept_len, dtype=np.int64)
    return float((a - 1).sum()) / (a.size * K)


def expected_accept_len_iid(p: float, K: int) -> float:
    """E[accept_len] when each of the K positions matches independently with probability p and
    acceptance stops at the first mismatch: sum_{i=0..K} p^i (textbook geometric prefix)."""
    return float(sum(p ** i for i in range(K + 1)))


# --------------------------------------------------------------------------------------------------
# building blocks


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def rope_angles(pos: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """angles [P, hd/2] = pos * base^(-2i/hd)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE. x [P, H, hd] at positions pos [P]."""
    hd = x.shape[-1]
    h = hd // 2
    ang = rope_angles(pos, hd, base)
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def argmax_first(z: np.ndarray) -> np.ndarray:
    """argmax over the last axis; among equal maxima the lowest index (numpy's documented rule)."""
    return np.argmax(z, axis=-1).astype(np.int32)


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x . W^T with W stored [out, in]."""
    return x @ w.T


# --------------------------------------------------------------------------------------------------
# [AWS-P] step-by-step drafting process, step 2: build the K input positions


def build_rows(W: dict, last_token: np.ndarray, target_hidden: np.ndarray, K: int) -> np.ndarray:
    """X [B, K, d].

    Position 1 of the pages (row 0 here) has real context: the token just produced by the target plus
    the hidden states captured from three target layers (low, middle, high; concatenated to 3d).
    Positions 2..K (rows 1..K-1) carry no real input: the learned shared hidden state h_shared stands in
    for the drafter's previous hidden state and the learned mask-token embedding emb_mask for the
    unknown previous token ([AWS-P] "how P-EAGLE breaks the chain").
    """
    B = last_token.shape[0]
    d = W["emb_mask"].shape[0]
    X = np.empty((B, K, d), dtype=np.float64)
    X[:, 0, :] = linear(target_hidden, W["fc"]) + W["embed"][last_token]
    X[:, 1:, :] = (W["h_shared"] + W["emb_mask"])[None, None, :]
    return X


# --------------------------------------------------------------------------------------------------
# attention of one request


def attention_request(q: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray, k_new: np.ndarray,
                      v_new: np.ndarray) -> np.ndarray:
    """One request's GQA attention.

    q [K, Hq, hd] (rotated); k_ctx, v_ctx [Hkv, L, hd] (context, keys already rotated);
    k_new, v_new [K, Hkv, hd] (this step's rows, keys rotated). Row j sees all L context positions and
    new rows 0..j. Returns o [K, Hq, hd].
    """
    K, Hq, hd = q.shape
    Hkv, L, _ = k_ctx.shape
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(hd)
    o = np.empty_like(q)
    for h in range(Hq):
        g = h // G
        keys = np.concatenate([k_ctx[g], k_new[:, g, :]], axis=0)  # [L + K, hd]
        vals = np.concatenate([v_ctx[g], v_new[:, g, :]], axis=0)
        for j in range(K):
            n = L + j + 1
            s = keys[:n] @ q[j, h] * scale
            p = np.exp(s - s.max())
            p /= p.sum()
            o[j, h] = p @ vals[:n]
    return o


# --------------------------------------------------------------------------------------------------
# the drafter forward over prebuilt rows


def draft_rows(shape, W: dict, X: np.ndarray, seq_len: np.ndarray, kv_context, E: np.ndarray = None) -> dict:
    """Run rows X [B, K, d] through the drafter's layers and LM head.

    kv_context(layer, b) -> (k_ctx [Hkv, L_b, hd], v_ctx [Hkv, L_b, hd]) float64.
    E [B, K, d] (concatenated rows only): the embedding half of each row. Layer 0's attention then reads
    [RMSNorm(e) with gain embed_norm || RMSNorm(x) with gain l0.attn_norm] through wqkv[0] [qkv, 2d];
    the residual stream is x alone.
    Returns logits [B, K, V], draft [B, K], hidden [B, K, d] (before the final norm) and the rotated
    keys / values of the new rows per layer (k_new[l], v_new[l] [B, K, Hkv, hd]).
    """
    B, K, d = X.shape
    Hq, Hkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    eps = shape.rms_eps
    x = X.reshape(B * K, d).astype(np.float64, copy=True)
    pos = (np.asarray(seq_len, dtype=np.int64)[:, None] + np.arange(K)[None, :]).reshape(-1)
    k_new_all, v_new_all = [], []
    for l in range(shape.n_layers):
        u = rms_norm(x, W[f"l{l}.attn_norm"], eps)
        if l == 0 and E is not None:
            u = np.concatenate([rms_norm(E.reshape(B * K, d), W["embed_norm"], eps), u], axis=1)
        qkv = linear(u, W[f"l{l}.wqkv"])
        q = qkv[:, : Hq * hd].reshape(B * K, Hq, hd)
        k = qkv[:, Hq * hd: (Hq + Hkv) * hd].reshape(B * K, Hkv, hd)
        v = qkv[:, (Hq + Hkv) * hd:].reshape(B * K, Hkv, hd)
        q = rope(q, pos, shape.rope_base)
        k = rope(k, pos, shape.rope_base)
        o = np.empty_like(q)
        for b in range(B):
            rows = slice(b * K, (b + 1) * K)
            k_ctx, v_ctx = kv_context(l, b)
            o[rows] = attention_request(q[rows], k_ctx, v_ctx, k[rows], v[rows])
        x = x + linear(o.reshape(B * K, Hq * hd), W[f"l{l}.wo"])
        u = rms_norm(x, W[f"l{l}.mlp_norm"], eps)
        a = silu(linear(u, W[f"l{l}.wgate"])) * linear(u, W[f"l{l}.wup"])
        x = x + linear(a, W[f"l{l}.wdown"])
        k_new_all.append(k.reshape(B, K, Hkv, hd))
        v_new_all.append(v.reshape(B, K, Hkv, hd))
    z = linear(rms_norm(x, W["final_norm"], eps), W["lm_head"])
    logits = z.reshape(B, K, -1)
    return {"logits": logits, "draft": argmax_first(logits), "hidden": x.reshape(B, K, d),
            "k_new": k_new_all, "v_new": v_new_all}


def draft_step(shape, W: dict, state: dict, kv_context, K: int, tail: bool = False) -> dict:
    """[AWS-P] step 2: build K rows per request, one forward pass, K draft tokens at once.

    tail=True also runs one placeholder row after the K draft rows; its K/V (k_new, v_new then hold K + 1
    rows) fill the cache position an all-accepted verify keeps; logits, draft and hidden stay K rows."""
    X = build_rows(W, state["last_token"], state["target_hidden"], K + 1 if tail else K)
    out = draft_rows(shape, W, X, state["seq_len"], kv_context)
    if tail:
        for key in ("logits", "draft", "hidden"):
            out[key] = out[key][:, :K]
    out["rows"] = X
    return out


def fp8_e4m3_round(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest value of the FP8 E4M3 format (1 sign, 4 exponent bits with bias 7,
    3 mantissa bits; largest finite 448; subnormals step 2^-9), ties to the even mantissa. Inputs must lie
    within +-464 (the caller scales them into +-448); returns the rounded values as float64."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # spacing of representable values around a: 2^(e - 3) for a in [2^e, 2^(e+1)), e >= -6; 2^-9 below 2^-6
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = np.exp2(e - 3.0)
    q = a / step
    r = np.floor(q)
    frac = q - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2.0) == 1.0))
    r = r + up
    out = np.where(a > 0, r * step, 0.0)
    return np.copysign(np.minimum(out, 448.0), x)


def quantize_fp8_rows(W: np.ndarray) -> np.ndarray:
    """Per-output-row FP8 weights, dequantized: s_n = max_k |W[n, k]| / 448 (float32), q = E4M3 rounding of
    float32(W[n, k] / s_n) (float32 division, as the repack computes it), returned as q * s_n in float64.
    A row of zeros keeps scale 1 (and stays zero)."""
    W32 = np.asarray(W, dtype=np.float32)
    amax = np.abs(W32).max(axis=1) if W32.ndim == 2 else np.abs(W32).max()
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = fp8_e4m3_round((W32 / s[:, None]).astype(np.float32))
    return q * s.astype(np.float64)[:, None]


def weights_fp8(shape, W: dict) -> dict:
    """The drafter with every projection matrix (fc, wqkv, wo, wgate, wup, wdown, lm_head) replaced by its
    per-row FP8 dequantization; embeddings, placeholders and norm gains unchanged."""
    out = dict(W)
    for k, v in W.items():
        base = k.split(".")[-1]
        if base in ("fc", "wqkv", "wo", "wgate", "wup", "wdown", "lm_head"):
            out[k] = quantize_fp8_rows(v)
    return out


def build_rows_concat(W: dict, last_token: np.ndarray, target_hidden: np.ndarray, K: int) -> tuple:
    """The pages' literal wording: each position's input is its token embedding concatenated with a
    hidden state ([AWS-P] step-by-step drafting process: position 1 joins the real token's embedding to the
    captured target hidden states, positions 2..K join emb_mask to h_shared). Returns the two halves,
    E [B, K, d] (embedding) and H [B, K, d] (hidden: fc of the three captured states for row 0, h_shared
    after); the row is [E || H]."""
    B = last_token.shape[0]
    d = W["emb_mask"].shape[0]
    E = np.empty((B, K, d), dtype=np.float64)
    H = np.empty((B, K, d), dtype=np.float64)
    E[:, 0, :] = W["embed"][last_token]
    H[:, 0, :] = linear(target_hidden, W["fc"])
    E[:, 1:, :] = W["emb_mask"][None, None, :]
    H[:, 1:, :] = W["h_shared"][None, None, :]
    return E, H


def draft_step_concat(shape, W: dict, state: dict, kv_context, K: int, tail: bool = False) -> dict:
    """draft_step with concatenated input rows (build_rows_concat; layer 0 reads [E || H], the residual
    stream starts as H). tail as in draft_step."""
    E, H = build_rows_concat(W, state["last_token"], state["target_hidden"], K + 1 if tail else K)
    out = draft_rows(shape, W, H, state["seq_len"], kv_context, E=E)
    if tail:
        for key in ("logits", "draft", "hidden"):
            out[key] = out[key][:, :K]
    return out


def build_rows_catchup(W: dict, tokens: np.ndarray, target_hidden: np.ndarray, n_real: np.ndarray,
                       K: int) -> np.ndarray:
    """X [B, R + K, d] for a step that first catches up on several real positions.

    Request b's rows 0..n_real[b]-1 are real, each built like the pages' position 1: fc of the three
    captured target hidden states that produced token tokens[b, i], plus that token's embedding. Every
    later row is the placeholder h_shared + emb_mask ([AWS-P] "how P-EAGLE breaks the chain"). With
    n_real = 1 and R = 1 this is build_rows with K + 1 rows.
    tokens [B, R], target_hidden [B, R, 3d]; entries past n_real[b] are ignored.
    """
    B, R = tokens.shape
    d = W["emb_mask"].shape[0]
    X = np.empty((B, R + K, d), dtype=np.float64)
    X[:, :, :] = (W["h_shared"] + W["emb_mask"])[None, None, :]
    for b in range(B):
        r = int(n_real[b])
        X[b, :r, :] = linear(target_hidden[b, :r], W["fc"]) + W["embed"][tokens[b, :r]]
    return X


def draft_step_catchup(shape, W: dict, state: dict, kv_context, K: int) -> dict:
    """One parallel draft step whose input starts with several real positions (multi-row catch-up).

    After a verify that emitted a tokens, the target has computed a hidden state for each of them; the
    step re-runs those a positions as real rows (the exact drafter K/V for what was accepted) and then the
    K - 1 placeholder rows of the parallel step. Request b's first row sits at position seq_len[b]; its
    drafts come from rows n_real[b] - 1 (the last real row: the next token) .. n_real[b] + K - 2.
    Every request runs R + K rows (R = tokens.shape[1]); the rows after the drafted ones only fill cache
    positions the causal mask hides from every drafted row.

    state: seq_len [B], tokens [B, R], target_hidden [B, R, 3d], n_real [B] in 1..R.
    Returns logits [B, K, V], draft [B, K], hidden [B, K, d] of the drafted rows, the built rows, and
    k_new / v_new per layer [B, R + K, Hkv, hd] of every row.
    """
    n_real = np.asarray(state["n_real"], dtype=np.int64)
    X = build_rows_catchup(W, np.asarray(state["tokens"]), state["target_hidden"], n_real, K)
    out = draft_rows(shape, W, X, state["seq_len"], kv_context)
    B = X.shape[0]
    rows = n_real[:, None] - 1 + np.arange(K)[None, :]
    bi = np.arange(B)[:, None]
    for key in ("logits", "draft", "hidden"):
        out[key] = out[key][bi, rows]
    out["rows"] = X
    return out


def draft_autoregressive(shape, W: dict, state: dict, kv_context, K: int, tail: bool = False,
                         feed: np.ndarray = None) -> dict:
    """Autoregressive EAGLE-style drafting of K tokens, the chain that parallel drafting removes ([AWS-P]
    "sequential dependency in autoregressive EAGLE": each draft token needs the previous pass's hidden
    state and token, so K tokens take K forward passes).

    Pass 0 runs the parallel step's row 0 (fc(concat(h)) + E[last_token]) at position L_b. Pass i >= 1
    runs one row per request at position L_b + i: the drafter's own hidden state of pass i - 1 (the
    residual stream after the last layer, before the final norm) plus the embedding of the token pass
    i - 1 drafted; it attends to the context and to the rows of passes 0..i-1. feed [B, K] optionally
    replaces the token fed back after pass i (row i of feed), e.g. to follow another implementation's
    choice at a near-tie. tail=True runs one more pass (layers only) at position L_b + K, so the cache holds
    K/V for every position an all-accepted verify keeps, as the parallel step's placeholder row does.

    Returns logits [B, K, V], draft [B, K], hidden [B, K, d] and k_new / v_new per layer [B, K(+1), Hkv, hd].
    """
    B = state["last_token"].shape[0]
    seq = np.asarray(state["seq_len"], dtype=np.int64)
    row0 = build_rows(W, state["last_token"], state["target_hidden"], 1)[:, 0]
    logits, draft, hidden = [], [], []
    k_new = [[] for _ in range(shape.n_layers)]
    v_new = [[] for _ in range(shape.n_layers)]

    def ctx_with_passes(l, b):
        k_ctx, v_ctx = kv_context(l, b)
        if not k_new[l]:
            return k_ctx, v_ctx
        k_add = np.stack([kn[b] for kn in k_new[l]], axis=1)  # [Hkv, passes, hd]
        v_add = np.stack([vn[b] for vn in v_new[l]], axis=1)
        return np.concatenate([k_ctx, k_add], axis=1), np.concatenate([v_ctx, v_add], axis=1)

    row = row0
    for i in range(K + 1 if tail else K):
        out = draft_rows(shape, W, row[:, None, :], seq + i, ctx_with_passes)
        for l in range(shape.n_layers):
            k_new[l].append(out["k_new"][l][:, 0])
            v_new[l].append(out["v_new"][l][:, 0])
        if i == K:
            break
        logits.append(out["logits"][:, 0])
        draft.append(out["draft"][:, 0])
        hidden.append(out["hidden"][:, 0])
        tok = draft[-1] if feed is None else np.asarray(feed)[:, i]
        row = hidden[-1] + W["embed"][tok]
    return {"logits": np.stack(logits, axis=1), "draft": np.stack(draft, axis=1),
            "hidden": np.stack(hidden, axis=1),
            "k_new": [np.stack(k, axis=1) for k in k_new], "v_new": [np.stack(v, axis=1) for v in v_new]}


# --------------------------------------------------------------------------------------------------
# written separately, loop by loop: one sequential EAGLE-style draft for one request


def eagle_step_sequential(shape, W: dict, token: int, hid3: np.ndarray, L: int, kv_ctx_layers,
                          row: np.ndarray = None, full: bool = False) -> tuple:
    """One autoregressive EAGLE draft pass for a single request ([AWS-P] "sequential dependency in
    autoregressive EAGLE"): the input is the embedding of the token just produced plus the projected
    target hidden states; one row goes through the layers at position L; the LM head gives one token.
    kv_ctx_layers[l] = (k [Hkv, >= L, hd], v [Hkv, >= L, hd]): the first L positions are the context.
    row: a prebuilt input row used instead of fc(hid3) + E[token] (a later autoregressive pass).

    Written with explicit per-head and per-key loops, independently of draft_rows. Returns
    (token, logits [V]); with full=True also the hidden state after the last layer (before the final
    norm) and this row's rotated keys and values per layer ([Hkv, hd] each).
    """
    d = shape.d_model
    Hq, Hkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    G = Hq // Hkv
    half = hd // 2
    eps = shape.rms_eps
    if row is None:
        fc = W["fc"]
        x = np.array([float(np.dot(fc[r], hid3)) for r in range(d)]) + W["embed"][token]
    else:
        x = np.array(row, dtype=np.float64)
    k_rows, v_rows = [], []

    def norm(v, g):
        return v * (1.0 / math.sqrt(float(np.dot(v, v)) / d + eps)) * g

    def rot(vec):
        out = vec.copy()
        for i in range(half):
            theta = L * shape.rope_base ** (-(2.0 * i) / hd)
            c, s = math.cos(theta), math.sin(theta)
            out[i] = vec[i] * c - vec[i + half] * s
            out[i + half] = vec[i + half] * c + vec[i] * s
        return out

    for l in range(shape.n_layers):
        k_ctx, v_ctx = kv_ctx_layers[l]
        u = norm(x, W[f"l{l}.attn_norm"])
        wqkv = W[f"l{l}.wqkv"]
        attn = np.zeros(Hq * hd)
        k_self = [rot(wqkv[(Hq + g) * hd:(Hq + g + 1) * hd] @ u) for g in range(Hkv)]
        v_self = [wqkv[(Hq + Hkv + g) * hd:(Hq + Hkv + g + 1) * hd] @ u for g in range(Hkv)]
        k_rows.append(np.array(k_self))
        v_rows.append(np.array(v_self))
        for h in range(Hq):
            qh = rot(wqkv[h * hd:(h + 1) * hd] @ u)
            g = h // G
            scores = [float(np.dot(qh, k_ctx[g, t])) / math.sqrt(hd) for t in range(L)]
            scores.append(float(np.dot(qh, k_self[g])) / math.sqrt(hd))
            m = max(scores)
            wts = [math.exp(sc - m) for sc in scores]
            tot = sum(wts)
            acc = np.zeros(hd)
            for t in range(L):
                acc += wts[t] * v_ctx[g, t]
            acc += wts[L] * v_self[g]
            attn[h * hd:(h + 1) * hd] = acc / tot
        x = x + W[f"l{l}.wo"] @ attn
        u = norm(x, W[f"l{l}.mlp_norm"])
        gate = W[f"l{l}.wgate"] @ u
        up = W[f"l{l}.wup"] @ u
        act = np.array([gv / (1.0 + math.exp(-gv)) * uv for gv, uv in zip(gate, up)])
        x = x + W[f"l{l}.wdown"] @ act
    z = W["lm_head"] @ norm(x, W["final_norm"])
    best = 0
    for v in range(1, z.shape[0]):
        if z[v] > z[best]:
            best = v
    if full:
        return best, z, x, k_rows, v_rows
    return best, z


# --------------------------------------------------------------------------------------------------
# [AWS-P] step-by-step drafting process, final sentence: the target verifies all K candidates in one
# pass with the standard acceptance rule. Greedy reading: accept while the draft equals the target's
# argmax; the target's argmax at the first mismatch (or after K matches) is the bonus token.


def verify(target_logits: np.ndarray, draft: np.ndarray) -> dict:
    """target_logits [B, K+1, V] (position i predicts the token after draft i-1; i = 0 follows the
    last target token), draft [B, K]. Returns t [B, K+1], n [B] (accepted drafts), accept_len [B] = n+1,
    bonus [B]."""
    t = argmax_first(target_logits)
    B, K = draft.shape
    n = np.empty(B, dtype=np.int32)
    for b in range(B):
        i = 0
        while i < K and draft[b, i] == t[b, i]:
            i += 1
        n[b] = i
    accept_len = n + 1
    bonus = t[np.arange(B), n]
    return {"t": t, "n": n, "accept_len": accept_len.astype(np.int32), "bonus": bonus.astype(np.int32)}


# --------------------------------------------------------------------------------------------------
# The same acceptance rule in its sampling form (temperature > 0; the pages' example request uses 0.3):
# standard speculative sampling. A draft x drawn from q is accepted with probability min(1, p(x) / q(x));
# on a rejection the emitted token is drawn from the normalised residual max(0, p - q); after K
# acceptances the bonus token is drawn from p at position K. Reading: the parallel drafter drafts
# greedily, so q is a point mass at the draft token; then a draft x is accepted with probability p(x) and
# a rejection draws from p with x removed. The uniforms are inputs (u for the acceptance tests, v for the
# draws), so the rule is deterministic given them.


def softmax_temperature(z: np.ndarray, temperature: float) -> np.ndarray:
    """p = softmax(z / temperature) along the last axis, float64."""
    x = np.asarray(z, dtype=np.float64) / temperature
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def draw_inverse_cdf(w: np.ndarray, v: float) -> int:
    """The smallest x with w[0] + ... + w[x] > v * sum(w), for weights w >= 0 and v in [0, 1)."""
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    return int(np.searchsorted(c, v * c[-1], side="right"))


def verify_sampled(target_logits: np.ndarray, draft: np.ndarray, temperature: float, u: np.ndarray,
                   v: np.ndarray) -> dict:
    """target_logits [B, K+1, V], draft [B, K], uniforms u [B, K] and v [B, K+1] in [0, 1).

    Position i accepts draft[b, i] iff u[b, i] < p_i(draft[b, i]), p_i = softmax(T[b, i] / temperature).
    At the first rejection n, the emitted token is drawn with v[b, n] from p_n without draft[b, n];
    after K acceptances the bonus token is drawn with v[b, K] from p_K. Returns the same fields as verify:
    t [B, K+1] (emitted tokens at positions 0..n, -1 after), n, accept_len = n + 1, bonus."""
    B, K = draft.shape
    t = np.full((B, K + 1), -1, dtype=np.int64)
    n = np.empty(B, dtype=np.int32)
    for b in range(B):
        i = 0
        while True:
            p = softmax_temperature(target_logits[b, i], temperature)
            if i == K:
                t[b, i] = draw_inverse_cdf(p, v[b, i])
                break
            x = int(draft[b, i])
            if u[b, i] < p[x]:
                t[b, i] = x
                i += 1
                continue
            r = p.copy()
            r[x] = 0.0
            t[b, i] = draw_inverse_cdf(r, v[b, i])
            break
        n[b] = i
    bonus = t[np.arange(B), n]
    return {"t": t, "n": n, "accept_len": (n + 1).astype(np.int32), "bonus": bonus.astype(np.int32)}


def compact(v: dict, req_slot: np.ndarray, seq_len: np.ndarray, finished=None) -> dict:
    """Batch-metadata rebuild after verify ([JP] implementation and performance: the metadata the
    serving loop needs for the next step).

    cu_accept [B+1]: exclusive prefix sum of accept_len; out_tokens: request b's accepted tokens (the
    target argmax prefix t[b, 0..n_b]) at cu_accept[b]...; seq_len' = seq_len + accept_len;
    last_token' = bonus; surviving (not finished) requests keep their order.
    """
    acc = v["accept_len"]
    B = acc.shape[0]
    cu = np.zeros(B + 1, dtype=np.int32)
    for b in range(B):
        cu[b + 1] = cu[b] + acc[b]
    out = np.empty(cu[B], dtype=np.int32)
    for b in range(B):
        for i in range(acc[b]):
            out[cu[b] + i] = v["t"][b, i]
    seq_next_all = (np.asarray(seq_len) + acc).astype(np.int32)
    fin = np.zeros(B, dtype=bool) if finished is None else np.asarray(finished).astype(bool)
    keep = [b for b in range(B) if not fin[b]]
    keep_index = np.array(keep, dtype=np.int32)
    return {"cu_accept": cu, "out_tokens": out, "keep_index": keep_index, "n_keep": len(keep),
            "req_slot_next": np.asarray(req_slot, dtype=np.int32)[keep_index],
            "seq_len_next": seq_next_all[keep_index],
            "last_token_next": v["bonus"][keep_index].astype(np.int32)}
