"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test names the passage or the mathematical fact it relies on. Expected values here never come
from the oracle itself: they are printed on the pages (tests/golden), closed forms, hand-computed
values, textbook special cases, or a brute-force recount written differently.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import pe_oracle as O
from synth import DrafterShape, Workload, make_weights, make_state, random_draft, plant_target_logits
from synth.inputs import to_f64, kv_block

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# a tiny drafter: 2 layers, GQA with G = 2, small vocab
MINI = DrafterShape("mini-f32", 2, 32, 4, 2, 8, 48, 64, "f32")


def _weights64(shape, seed):
    raw = make_weights(shape, seed=seed)
    return {k: to_f64(v, shape.dtype) for k, v in raw.items()}


def _ctx(shape, L, seed, nlayers=None):
    rng = np.random.default_rng(seed)
    n = shape.n_layers if nlayers is None else nlayers
    return [(rng.standard_normal((shape.n_kv_heads, L, shape.head_dim)),
             rng.standard_normal((shape.n_kv_heads, L, shape.head_dim))) for _ in range(n)]


# ---------------------------------------------------------------- speedup formula (lesson, concept)

def test_speedup_worked_example_from_page():
    g = json.load(open(os.path.join(GOLDEN, "lesson_speedup.json")))["speedup_worked_example"]
    K, a, e = g["K"], g["alpha"], g["verify_overhead"]
    assert O.tokens_per_target_pass(K, a) == pytest.approx(g["tokens_per_target_pass"], abs=1e-12)
    s = O.speedup(K, a, e)
    assert s == pytest.approx(g["numerator"] / g["denominator"], abs=1e-12)
    assert round(s, 1) == g["speedup_as_printed"]


def test_breakeven_worked_example_from_page():
    g = json.load(open(os.path.join(GOLDEN, "lesson_speedup.json")))["breakeven_worked_example"]
    a = O.breakeven_alpha(g["verify_overhead"], g["K"])
    assert a == pytest.approx(g["alpha_breakeven_as_printed"], abs=1e-12)
    # at the break-even alpha the speedup is exactly 1 (closed form)
    assert O.speedup(g["K"], a, g["verify_overhead"]) == pytest.approx(1.0, abs=1e-12)


def test_alpha_hat_identity():
    # production recipe: alpha = accepted drafts per request / draft length, so that
    # mean accepted tokens per target pass = 1 + K * alpha exactly.
    rng = np.random.default_rng(5)
    for K in (1, 3, 7, 11):
        acc = rng.integers(1, K + 2, size=97)
        assert acc.mean() == pytest.approx(O.tokens_per_target_pass(K, O.alpha_hat(acc, K)), abs=1e-12)


def test_expected_accept_len_closed_form():
    # geometric prefix: sum_{i=0..K} p^i = (1 - p^(K+1)) / (1 - p)
    for p, K in ((0.7, 4), (0.6, 7), (0.85, 11)):
        assert O.expected_accept_len_iid(p, K) == pytest.approx((1 - p ** (K + 1)) / (1 - p), rel=1e-12)
    assert O.expected_accept_len_iid(1.0, 5) == 6.0


# ---------------------------------------------------------------- verify / accept (greedy)

def _planted(K, V, pattern, rng):
    """Target logits whose argmax at position i equals draft[i] iff pattern[i] == '1'."""
    draft = rng.integers(0, V, size=K)
    T = rng.standard_normal((K + 1, V)) * 0.1
    tgt = []
    for i in range(K):
        tok = int(draft[i]) if pattern[i] == "1" else (int(draft[i]) + 1 + int(rng.integers(0, V - 1))) % V
        T[i, tok] = 5.0
        tgt.append(tok)
    bonus_tok = int(rng.integers(0, V))
    T[K, bonus_tok] = 5.0
    tgt.append(bonus_tok)
    return T, draft, tgt


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_verify_brute_force_all_patterns(K):
    V = 16
    rng = np.random.default_rng(100 + K)
    for bits in itertools.product("01", repeat=K):
        pattern = "".join(bits)
        T, draft, tgt = _planted(K, V, pattern, rng)
        v = O.verify(T[None], draft[None])
        first_zero = pattern.find("0")
        n_expect = K if first_zero < 0 else first_zero
        assert v["n"][0] == n_expect
        assert v["accept_len"][0] == n_expect + 1
        assert v["bonus"][0] == tgt[n_expect]
        # output identical to the target's greedy tokens
        assert list(v["t"][0, : n_expect + 1]) == tgt[: n_expect + 1]


def test_verify_invariant_all_match_and_first_mismatch():
    rng = np.random.default_rng(7)
    for K in (1, 4, 10):
        T, draft, _ = _planted(K, 50, "1" * K, rng)
        assert O.verify(T[None], draft[None])["accept_len"][0] == K + 1
        T, draft, _ = _planted(K, 50, "0" + "1" * (K - 1), rng)
        assert O.verify(T[None], draft[None])["accept_len"][0] == 1


def test_argmax_ties_lowest_index():
    z = np.array([[0.0, 3.0, 1.0, 3.0, 3.0], [2.0, 2.0, 2.0, 2.0, 2.0]])
    assert list(O.argmax_first(z)) == [1, 0]


def test_compact_against_recount():
    rng = np.random.default_rng(11)
    for B, K in ((1, 3), (5, 4), (33, 7)):
        T = rng.standard_normal((B, K + 1, 20))
        draft = rng.integers(0, 20, size=(B, K))
        # make roughly half the positions match
        t0 = T.argmax(-1)
        m = rng.random((B, K)) < 0.6
        draft[m] = t0[:, :K][m]
        v = O.verify(T, draft)
        fin = (rng.random(B) < 0.3).astype(np.uint8)
        slot = rng.permutation(B + 3)[:B]
        seq = rng.integers(10, 100, size=B)
        c = O.compact(v, slot, seq, fin)
        assert list(c["cu_accept"]) == [0] + list(np.cumsum(v["accept_len"]))
        toks = [int(x) for b in range(B) for x in t0[b, : v["accept_len"][b]]]
        assert list(c["out_tokens"]) == toks
        keep = [b for b, f in enumerate(fin) if f == 0]
        assert list(c["keep_index"]) == keep and c["n_keep"] == len(keep)
        assert list(c["req_slot_next"]) == [slot[b] for b in keep]
        assert list(c["seq_len_next"]) == [seq[b] + v["accept_len"][b] for b in keep]
        assert list(c["last_token_next"]) == [t0[b, v["n"][b]] for b in keep]


def test_planted_generator_acceptance_statistics():
    # per-position i.i.d. planting with probability p gives E[accept_len] = sum_i p^i (C-11 reading);
    # checked within 5 sigma over many requests
    w = Workload("stat", MINI, 4000, 5, (8, 8), 0.7, 77)
    st = make_state(w)
    draft = random_draft(w)
    T = plant_target_logits(w, draft, st["alpha"])
    acc = O.verify(T, draft)["accept_len"].astype(np.float64)
    mu = O.expected_accept_len_iid(0.7, 5)
    assert abs(acc.mean() - mu) < 5 * acc.std() / math.sqrt(acc.size)


# ---------------------------------------------------------------- building blocks

def test_linear_orientation_hand_example():
    W = np.array([[1.0, 2.0], [3.0, 4.0]])
    assert list(O.linear(np.array([[1.0, 1.0]]), W)[0]) == [3.0, 7.0]


def test_rms_norm_hand_example_and_closed_form():
    out = O.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert out == pytest.approx([3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rel=1e-15)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)) * 3
    g = 1 + 0.02 * rng.standard_normal(64)
    eps = 1e-6
    y = O.rms_norm(x, g, eps) / g
    ms = np.mean(x * x, -1)
    assert np.mean(y * y, -1) == pytest.approx(ms / (ms + eps), rel=1e-12)


def test_silu_closed_forms():
    assert O.silu(np.array(0.0)) == 0.0
    assert float(O.silu(np.array(1.0))) == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)
    x = np.linspace(-6, 6, 25)
    assert O.silu(x) - O.silu(-x) == pytest.approx(x, abs=1e-12)


def test_rope_hand_values_pin_pairing_and_frequencies():
    # hd = 4, base 10000: inv_freq = [1, 10000^(-1/2)] = [1, 0.01]; rotate-half pairs (0,2) and (1,3)
    e0 = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    y = O.rope(e0, np.array([1]), 10000.0)[0, 0]
    assert y == pytest.approx([math.cos(1.0), 0.0, math.sin(1.0), 0.0], abs=1e-15)
    e1 = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    y = O.rope(e1, np.array([100]), 10000.0)[0, 0]
    assert y == pytest.approx([0.0, math.cos(1.0), 0.0, math.sin(1.0)], abs=1e-13)
    e2 = np.array([[[0.0, 0.0, 1.0, 0.0]]])
    y = O.rope(e2, np.array([1]), 10000.0)[0, 0]
    assert y == pytest.approx([-math.sin(1.0), 0.0, math.cos(1.0), 0.0], abs=1e-15)


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 2, 16))
    assert np.array_equal(O.rope(x, np.zeros(3, dtype=int), 10000.0), x)
    y = O.rope(x, np.array([5, 77, 4000]), 10000.0)
    assert np.linalg.norm(y, axis=-1) == pytest.approx(np.linalg.norm(x, axis=-1), rel=1e-12)
    q, k = rng.standard_normal((1, 1, 16)), rng.standard_normal((1, 1, 16))
    d1 = np.sum(O.rope(q, np.array([9]), 1e4) * O.rope(k, np.array([3]), 1e4))
    d2 = np.sum(O.rope(q, np.array([1009]), 1e4) * O.rope(k, np.array([1003]), 1e4))
    assert d1 == pytest.approx(d2, rel=1e-9)


# ---------------------------------------------------------------- attention

def _attn_brute(q, k_ctx, v_ctx, k_new, v_new):
    """per-key loop, with an explicit mask test"""
    K, Hq, hd = q.shape
    Hkv, L, _ = k_ctx.shape
    G = Hq // Hkv
    o = np.zeros_like(q)
    for j in range(K):
        for h in range(Hq):
            g = h // G
            num = np.zeros(hd)
            den = 0.0
            allk = [(k_ctx[g, t], v_ctx[g, t], t) for t in range(L)] + \
                   [(k_new[i, g], v_new[i, g], L + i) for i in range(K)]
            m = max(float(np.dot(q[j, h], kk)) / math.sqrt(hd) for kk, _, pos in allk if pos <= L + j)
            for kk, vv, pos in allk:
                if pos > L + j:
                    continue
                wgt = math.exp(float(np.dot(q[j, h], kk)) / math.sqrt(hd) - m)
                num += wgt * vv
                den += wgt
            o[j, h] = num / den
    return o


def test_attention_matches_brute_force():
    rng = np.random.default_rng(3)
    for (K, Hq, Hkv, hd, L) in ((1, 2, 1, 4, 0), (3, 4, 2, 8, 5), (4, 8, 2, 8, 9)):
        q = rng.standard_normal((K, Hq, hd))
        kc, vc = rng.standard_normal((Hkv, L, hd)), rng.standard_normal((Hkv, L, hd))
        kn, vn = rng.standard_normal((K, Hkv, hd)), rng.standard_normal((K, Hkv, hd))
        assert O.attention_request(q, kc, vc, kn, vn) == pytest.approx(_attn_brute(q, kc, vc, kn, vn),
                                                                       rel=1e-12, abs=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(4)
    # one key (L = 0, K = 1): softmax of a single score is 1, output is that value row exactly
    q = rng.standard_normal((1, 4, 8))
    kn, vn = rng.standard_normal((1, 2, 8)), rng.standard_normal((1, 2, 8))
    o = O.attention_request(q, np.zeros((2, 0, 8)), np.zeros((2, 0, 8)), kn, vn)
    assert np.array_equal(o[0, :2], np.repeat(vn[0, :1], 2, 0)) and np.array_equal(o[0, 2:], np.repeat(vn[0, 1:], 2, 0))
    # identical keys: uniform weights, output = mean of the visible values
    L, K = 6, 3
    key = rng.standard_normal(8)
    kc = np.tile(key, (1, L, 1))
    kn = np.tile(key, (K, 1, 1))
    vc, vn = rng.standard_normal((1, L, 8)), rng.standard_normal((K, 1, 8))
    o = O.attention_request(rng.standard_normal((K, 2, 8)), kc, vc, kn, vn)
    allv = np.concatenate([vc[0], vn[:, 0]], 0)
    for j in range(K):
        assert o[j, 0] == pytest.approx(allv[: L + j + 1].mean(0), rel=1e-12)


# ---------------------------------------------------------------- row building and whole-step invariants

def test_build_rows_structure():
    # "Paris" example: K = 4, position 1 is real, positions 2..4 are the learned placeholders
    W = _weights64(MINI, 9)
    st = make_state(Workload("r", MINI, 3, 4, (5, 5), 0.7, 9))
    hid = to_f64(st["target_hidden"], "f32")
    X = O.build_rows(W, st["last_token"], hid, 4)
    for j in (1, 2, 3):
        assert np.array_equal(X[:, j], np.broadcast_to(W["h_shared"] + W["emb_mask"], X[:, j].shape))
    assert X[:, 0] == pytest.approx(hid @ W["fc"].T + W["embed"][st["last_token"]], rel=1e-14)
    W0 = dict(W, fc=np.zeros_like(W["fc"]))
    X0 = O.build_rows(W0, st["last_token"], hid, 4)
    assert np.array_equal(X0[:, 0], W["embed"][st["last_token"]])


def _step(shape, W, tokens, hid, seq, ctx, K):
    st = {"last_token": np.asarray(tokens), "target_hidden": hid, "seq_len": np.asarray(seq)}
    return O.draft_step(shape, W, st, lambda l, b: ctx[b][l], K)


def test_k1_parallel_equals_sequential_eagle_step():
    # invariant 2: with K = 1 there are no placeholders; the step is one autoregressive EAGLE pass
    W = _weights64(MINI, 21)
    rng = np.random.default_rng(21)
    for L in (0, 1, 7):
        tok = int(rng.integers(0, MINI.vocab))
        hid = rng.standard_normal((1, 3 * MINI.d_model))
        ctx = _ctx(MINI, L, 100 + L)
        out = _step(MINI, W, [tok], hid, [L], [ctx], 1)
        t_seq, z_seq = O.eagle_step_sequential(MINI, W, tok, hid[0], L, ctx)
        assert out["logits"][0, 0] == pytest.approx(z_seq, rel=1e-10, abs=1e-12)
        assert out["draft"][0, 0] == t_seq


def test_row0_of_k_block_equals_k1_step():
    W = _weights64(MINI, 22)
    rng = np.random.default_rng(22)
    hid = rng.standard_normal((2, 3 * MINI.d_model))
    ctx = [_ctx(MINI, 4, 1), _ctx(MINI, 9, 2)]
    a = _step(MINI, W, [3, 40], hid, [4, 9], ctx, 1)
    b = _step(MINI, W, [3, 40], hid, [4, 9], ctx, 5)
    assert b["logits"][:, 0] == pytest.approx(a["logits"][:, 0], rel=1e-12, abs=1e-13)


def test_causality_later_rows_do_not_change_earlier_rows():
    # invariant 3: under the causal mask, perturbing rows j' > j leaves rows <= j unchanged
    W = _weights64(MINI, 23)
    rng = np.random.default_rng(23)
    K = 5
    st = {"last_token": np.array([7, 11]), "target_hidden": rng.standard_normal((2, 3 * MINI.d_model)),
          "seq_len": np.array([6, 3])}
    ctx = [_ctx(MINI, 6, 3), _ctx(MINI, 3, 4)]
    X = O.build_rows(W, st["last_token"], st["target_hidden"], K)
    base = O.draft_rows(MINI, W, X, st["seq_len"], lambda l, b: ctx[b][l])
    for j in range(K - 1):
        Xp = X.copy()
        Xp[:, j + 1:] += rng.standard_normal(Xp[:, j + 1:].shape)
        pert = O.draft_rows(MINI, W, Xp, st["seq_len"], lambda l, b: ctx[b][l])
        assert np.allclose(pert["logits"][:, : j + 1], base["logits"][:, : j + 1], rtol=1e-13, atol=1e-13)
        assert not np.allclose(pert["logits"][:, j + 1:], base["logits"][:, j + 1:])
        for l in range(MINI.n_layers):
            assert np.allclose(pert["k_new"][l][:, : j + 1], base["k_new"][l][:, : j + 1], rtol=1e-13, atol=1e-13)


def test_tail_row_leaves_the_draft_unchanged_and_fills_position_L_plus_K():
    # the trailing placeholder row (run so that an all-accepted verify finds K/V at L + K) comes after the
    # K draft rows: their logits are those of the plain K-row step, and its layer-0 key is the closed form
    # rope(W_k . RMSNorm(h_shared + emb_mask), L + K)
    W = _weights64(MINI, 25)
    rng = np.random.default_rng(25)
    K = 3
    hid = rng.standard_normal((2, 3 * MINI.d_model))
    seq = [5, 2]
    ctx = [_ctx(MINI, 5, 8), _ctx(MINI, 2, 9)]
    st = {"last_token": np.array([4, 9]), "target_hidden": hid, "seq_len": np.array(seq)}
    plain = O.draft_step(MINI, W, st, lambda l, b: ctx[b][l], K)
    tail = O.draft_step(MINI, W, st, lambda l, b: ctx[b][l], K, tail=True)
    assert tail["logits"].shape == plain["logits"].shape
    assert np.allclose(tail["logits"], plain["logits"], rtol=1e-13, atol=1e-13)
    assert np.array_equal(tail["draft"], plain["draft"])
    for l in range(MINI.n_layers):
        assert tail["k_new"][l].shape[1] == K + 1
        assert np.allclose(tail["k_new"][l][:, :K], plain["k_new"][l], rtol=1e-13, atol=1e-13)
    Hq, Hkv, hd = MINI.n_q_heads, MINI.n_kv_heads, MINI.head_dim
    x = W["h_shared"] + W["emb_mask"]
    u = x / np.sqrt(np.mean(x * x) + MINI.rms_eps) * W["l0.attn_norm"]
    k = (W["l0.wqkv"][Hq * hd:(Hq + Hkv) * hd] @ u).reshape(Hkv, hd)
    for b in range(2):
        pos = seq[b] + K
        inv = MINI.rope_base ** (-np.arange(hd // 2) * 2.0 / hd)
        c, s_ = np.cos(pos * inv), np.sin(pos * inv)
        want = np.concatenate([k[:, :hd // 2] * c - k[:, hd // 2:] * s_, k[:, hd // 2:] * c + k[:, :hd // 2] * s_], -1)
        assert np.allclose(tail["k_new"][0][b, K], want, rtol=1e-12, atol=1e-12)


def test_requests_are_independent():
    # a request's draft depends only on its own state and cache
    W = _weights64(MINI, 24)
    rng = np.random.default_rng(24)
    hid = rng.standard_normal((3, 3 * MINI.d_model))
    ctx = [_ctx(MINI, 4, 5), _ctx(MINI, 8, 6), _ctx(MINI, 2, 7)]
    full = _step(MINI, W, [1, 2, 3], hid, [4, 8, 2], ctx, 3)
    one = _step(MINI, W, [2], hid[1:2], [8], ctx[1:2], 3)
    assert one["logits"][0] == pytest.approx(full["logits"][1], rel=1e-12, abs=1e-13)


# ---------------------------------------------------------------- the shared input generator

def test_bf16_rounding_nearest_even():
    from synth import bf16_bits
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    assert list(bf16_bits(x)) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]


def test_kv_blocks_reproducible_per_request():
    w = Workload("kv", MINI, 3, 2, (4, 9), 0.7, 31)
    a = kv_block(w, 1, 0, 2, 5)
    b = kv_block(w, 1, 0, 2, 5)
    assert np.array_equal(a, b) and not np.array_equal(a, kv_block(w, 1, 1, 2, 5))


# ---------------------------------------------------------------- autoregressive drafting (the baseline)

def _ar(shape, W, tokens, hid, seq, ctx, K, tail=False, feed=None):
    st = {"last_token": np.asarray(tokens), "target_hidden": hid, "seq_len": np.asarray(seq)}
    return O.draft_autoregressive(shape, W, st, lambda l, b: ctx[b][l], K, tail=tail, feed=feed)


def _ar_loops(shape, W, tok, hid, L, ctx, K):
    """The same chain from the separately written loop-by-loop pass: pass i runs at position L + i over
    the context plus the K/V of passes 0..i-1, on the row h_{i-1} + E[t_{i-1}]."""
    ctx = [(k.copy(), v.copy()) for k, v in ctx]
    toks, zs, row = [], [], None
    for i in range(K):
        t, z, x, k_rows, v_rows = O.eagle_step_sequential(shape, W, tok, hid, L + i, ctx, row=row, full=True)
        toks.append(t)
        zs.append(z)
        ctx = [(np.concatenate([k, kr[:, None, :]], axis=1), np.concatenate([v, vr[:, None, :]], axis=1))
               for (k, v), kr, vr in zip(ctx, k_rows, v_rows)]
        row = x + W["embed"][t]
    return toks, np.stack(zs)


def test_autoregressive_chain_matches_loop_by_loop_passes():
    # the vectorised chain (draft_rows per pass, context grown by each pass's K/V) against the explicit
    # per-head, per-key loops of eagle_step_sequential, pass by pass
    W = _weights64(MINI, 31)
    rng = np.random.default_rng(31)
    for L, K in ((0, 3), (5, 4)):
        tok = int(rng.integers(0, MINI.vocab))
        hid = rng.standard_normal((1, 3 * MINI.d_model))
        ctx = _ctx(MINI, L, 300 + L)
        out = _ar(MINI, W, [tok], hid, [L], [ctx], K)
        toks, zs = _ar_loops(MINI, W, tok, hid[0], L, ctx, K)
        assert out["draft"][0].tolist() == toks
        assert out["logits"][0] == pytest.approx(zs, rel=1e-9, abs=1e-12)


def test_autoregressive_k1_and_pass0_equal_the_parallel_step():
    # K = 1: one pass, the same as the parallel step with K = 1; for any K, pass 0 sees only the context
    # and itself, so it equals the parallel step's row 0
    W = _weights64(MINI, 32)
    rng = np.random.default_rng(32)
    toks = rng.integers(0, MINI.vocab, size=2)
    hid = rng.standard_normal((2, 3 * MINI.d_model))
    ctx = [_ctx(MINI, 4, 320), _ctx(MINI, 9, 321)]
    ar1 = _ar(MINI, W, toks, hid, [4, 9], ctx, 1)
    pe1 = _step(MINI, W, toks, hid, [4, 9], ctx, 1)
    assert np.array_equal(ar1["logits"], pe1["logits"])
    ar3 = _ar(MINI, W, toks, hid, [4, 9], ctx, 3)
    pe3 = _step(MINI, W, toks, hid, [4, 9], ctx, 3)
    assert np.array_equal(ar3["logits"][:, 0], pe3["logits"][:, 0])
    assert ar3["logits"].shape == (2, 3, MINI.vocab)


def test_autoregressive_tail_and_feed():
    # the tail pass adds the K/V of position L + K and changes no output; a feed equal to the drafted
    # tokens changes nothing, a different feed changes every later pass but not pass 0
    W = _weights64(MINI, 33)
    rng = np.random.default_rng(33)
    tok = [int(rng.integers(0, MINI.vocab))]
    hid = rng.standard_normal((1, 3 * MINI.d_model))
    ctx = [_ctx(MINI, 6, 330)]
    a = _ar(MINI, W, tok, hid, [6], ctx, 3)
    t = _ar(MINI, W, tok, hid, [6], ctx, 3, tail=True)
    assert np.array_equal(a["logits"], t["logits"])
    assert a["k_new"][0].shape[1] == 3 and t["k_new"][0].shape[1] == 4
    assert np.array_equal(t["k_new"][1][:, :3], a["k_new"][1][:, :3])
    # the tail row is the pass-3 row h_2 + E[d_2] at position L + 3: check its layer-0 key by hand
    x = a["hidden"][0, 2] + W["embed"][a["draft"][0, 2]]
    u = O.rms_norm(x[None], W["l0.attn_norm"], MINI.rms_eps)
    k = O.linear(u, W["l0.wqkv"])[0, MINI.n_q_heads * MINI.head_dim:(MINI.n_q_heads + MINI.n_kv_heads) * MINI.head_dim]
    k = O.rope(k.reshape(1, MINI.n_kv_heads, MINI.head_dim), np.array([9]), MINI.rope_base)[0]
    assert t["k_new"][0][0, 3] == pytest.approx(k, rel=1e-12, abs=1e-12)
    same = _ar(MINI, W, tok, hid, [6], ctx, 3, feed=a["draft"])
    assert np.array_equal(same["logits"], a["logits"])
    other = (a["draft"] + 1) % MINI.vocab
    f = _ar(MINI, W, tok, hid, [6], ctx, 3, feed=other)
    assert np.array_equal(f["logits"][:, 0], a["logits"][:, 0])
    assert not np.allclose(f["logits"][:, 1], a["logits"][:, 1])


# ---------------------------------------------------------------- multi-row catch-up step

def _catchup(shape, W, tokens, hid, n_real, seq, ctx, K):
    st = {"tokens": np.asarray(tokens), "target_hidden": hid, "n_real": np.asarray(n_real),
          "seq_len": np.asarray(seq)}
    return O.draft_step_catchup(shape, W, st, lambda l, b: ctx[b][l], K)


def _real_row_passes(shape, W, toks, hid, L, ctx):
    """Real rows one at a time with the separately written single-row pass: row i at position L + i over
    the context plus the K/V of rows 0..i-1. Returns the last pass's logits, per-row K/V and the context
    grown by every row but the last."""
    ctx = [(k.copy(), v.copy()) for k, v in ctx]
    ks, vs, z, grown = [], [], None, None
    for i, (t, h) in enumerate(zip(toks, hid)):
        if i == len(toks) - 1:
            grown = [(k.copy(), v.copy()) for k, v in ctx]
        _, z, _, k_rows, v_rows = O.eagle_step_sequential(shape, W, int(t), h, L + i, ctx, full=True)
        ks.append(k_rows)
        vs.append(v_rows)
        ctx = [(np.concatenate([k, kr[:, None, :]], axis=1), np.concatenate([v, vr[:, None, :]], axis=1))
               for (k, v), kr, vr in zip(ctx, k_rows, v_rows)]
    return z, ks, vs, grown


def test_catchup_real_rows_match_single_row_passes():
    # each real row is an ordinary EAGLE input (token + the hidden states that produced it) at its own
    # position; the rows of one request see each other causally, so row i equals a single-row pass over
    # the context grown by rows 0..i-1; the last real row's logits are draft 0
    W = _weights64(MINI, 41)
    rng = np.random.default_rng(41)
    R, K = 3, 3
    toks = rng.integers(0, MINI.vocab, size=(2, R))
    hid = rng.standard_normal((2, R, 3 * MINI.d_model))
    n_real, seq = [3, 2], [5, 0]
    ctx = [_ctx(MINI, 5, 410), _ctx(MINI, 0, 411)]
    out = _catchup(MINI, W, toks, hid, n_real, seq, ctx, K)
    assert out["logits"].shape == (2, K, MINI.vocab) and out["k_new"][0].shape[1] == R + K
    for b in range(2):
        r = n_real[b]
        z, ks, vs, _ = _real_row_passes(MINI, W, toks[b, :r], hid[b, :r], seq[b], ctx[b])
        assert out["logits"][b, 0] == pytest.approx(z, rel=1e-9, abs=1e-12)
        for i in range(r):
            for l in range(MINI.n_layers):
                assert out["k_new"][l][b, i] == pytest.approx(ks[i][l], rel=1e-9, abs=1e-12)
                assert out["v_new"][l][b, i] == pytest.approx(vs[i][l], rel=1e-9, abs=1e-12)


def test_catchup_drafts_equal_the_plain_step_on_the_grown_context():
    # after the real rows 0..r-2 have joined the context (single-row passes), the catch-up step's K drafts
    # are those of a plain parallel step whose row 0 is the last real row, at position L + r - 1
    W = _weights64(MINI, 42)
    rng = np.random.default_rng(42)
    R, K = 4, 3
    toks = rng.integers(0, MINI.vocab, size=(2, R))
    hid = rng.standard_normal((2, R, 3 * MINI.d_model))
    n_real, seq = [4, 2], [3, 6]
    ctx = [_ctx(MINI, 3, 420), _ctx(MINI, 6, 421)]
    out = _catchup(MINI, W, toks, hid, n_real, seq, ctx, K)
    for b in range(2):
        r = n_real[b]
        _, _, _, grown = _real_row_passes(MINI, W, toks[b, :r], hid[b, :r], seq[b], ctx[b])
        plain = _step(MINI, W, [toks[b, r - 1]], hid[b, r - 1][None], [seq[b] + r - 1], [grown], K)
        assert out["logits"][b] == pytest.approx(plain["logits"][0], rel=1e-9, abs=1e-12)
        assert out["draft"][b].tolist() == plain["draft"][0].tolist()


def test_catchup_with_one_real_row_is_the_plain_step():
    # n_real = 1 and R = 1: the K + 1 rows of the plain step with its trailing placeholder row, exactly;
    # padding entries past n_real (R = 3) change nothing
    W = _weights64(MINI, 43)
    rng = np.random.default_rng(43)
    K = 3
    toks = rng.integers(0, MINI.vocab, size=(2, 1))
    hid = rng.standard_normal((2, 1, 3 * MINI.d_model))
    ctx = [_ctx(MINI, 4, 430), _ctx(MINI, 2, 431)]
    out = _catchup(MINI, W, toks, hid, [1, 1], [4, 2], ctx, K)
    st = {"last_token": toks[:, 0], "target_hidden": hid[:, 0], "seq_len": np.asarray([4, 2])}
    ref = O.draft_step(MINI, W, st, lambda l, b: ctx[b][l], K, tail=True)
    # (the same arithmetic; the fc product runs per request here, so only the summation order differs)
    assert out["logits"] == pytest.approx(ref["logits"], rel=1e-12, abs=1e-14)
    for l in range(MINI.n_layers):
        assert out["k_new"][l] == pytest.approx(ref["k_new"][l], rel=1e-12, abs=1e-14)
    toks3 = np.concatenate([toks, rng.integers(0, MINI.vocab, size=(2, 2))], axis=1)
    hid3 = np.concatenate([hid, rng.standard_normal((2, 2, 3 * MINI.d_model))], axis=1)
    pad = _catchup(MINI, W, toks3, hid3, [1, 1], [4, 2], ctx, K)
    assert np.array_equal(pad["logits"], out["logits"])
    assert np.array_equal(pad["k_new"][0][:, :K + 1], out["k_new"][0])


# ---------------------------------------------------------------- concatenated input rows

MINI_CAT = DrafterShape("mini-f32-concat", 2, 32, 4, 2, 8, 48, 64, "f32", row_concat=True)


def test_concat_rows_with_zero_embeddings_reduce_to_the_sum_step():
    # with a zero embedding table and mask, the embedding half normalises to zero, so layer 0 sees only
    # the hidden half through wqkv[0][:, d:]: the pinned sum-of-rows step with that matrix and zero
    # embeddings
    W = _weights64(MINI_CAT, 51)
    W["embed"] = np.zeros_like(W["embed"])
    W["emb_mask"] = np.zeros_like(W["emb_mask"])
    Ws = {k: v for k, v in W.items() if k != "embed_norm"}
    Ws["l0.wqkv"] = W["l0.wqkv"][:, MINI.d_model:]
    rng = np.random.default_rng(51)
    toks = rng.integers(0, MINI.vocab, size=2)
    hid = rng.standard_normal((2, 3 * MINI.d_model))
    ctx = [_ctx(MINI, 5, 510), _ctx(MINI, 0, 511)]
    st = {"last_token": toks, "target_hidden": hid, "seq_len": np.asarray([5, 0])}
    cat = O.draft_step_concat(MINI_CAT, W, st, lambda l, b: ctx[b][l], 3, tail=True)
    ref = O.draft_step(MINI, Ws, st, lambda l, b: ctx[b][l], 3, tail=True)
    assert cat["logits"] == pytest.approx(ref["logits"], rel=1e-12, abs=1e-14)
    for l in range(MINI.n_layers):
        assert cat["k_new"][l] == pytest.approx(ref["k_new"][l], rel=1e-12, abs=1e-14)


def test_concat_rows_layer0_keys_by_hand():
    # the order [embedding || hidden], the two gains and the placeholder halves, checked on layer 0's
    # keys of rows 0 and 1 computed here directly from the definitions
    W = _weights64(MINI_CAT, 52)
    rng = np.random.default_rng(52)
    d, Hq, Hkv, hd = MINI.d_model, MINI.n_q_heads, MINI.n_kv_heads, MINI.head_dim
    tok = int(rng.integers(0, MINI.vocab))
    hid = rng.standard_normal((1, 3 * d))
    L = 4
    ctx = [_ctx(MINI, L, 520)]
    out = O.draft_step_concat(MINI_CAT, W, {"last_token": np.asarray([tok]), "target_hidden": hid,
                                            "seq_len": np.asarray([L])}, lambda l, b: ctx[b][l], 2)

    def norm(v, g):
        return v / math.sqrt(float(v @ v) / d + MINI.rms_eps) * g

    rows = [(W["embed"][tok], W["fc"] @ hid[0]), (W["emb_mask"], W["h_shared"])]
    for j, (e, h) in enumerate(rows):
        u = np.concatenate([norm(e, W["embed_norm"]), norm(h, W["l0.attn_norm"])])
        k = (W["l0.wqkv"] @ u)[Hq * hd:(Hq + Hkv) * hd].reshape(Hkv, hd)
        half = hd // 2
        for g in range(Hkv):
            rot = np.empty(hd)
            for i in range(half):
                th = (L + j) * MINI.rope_base ** (-2.0 * i / hd)
                rot[i] = k[g, i] * math.cos(th) - k[g, i + half] * math.sin(th)
                rot[i + half] = k[g, i + half] * math.cos(th) + k[g, i] * math.sin(th)
            assert out["k_new"][0][0, j, g] == pytest.approx(rot, rel=1e-10, abs=1e-12)


def test_concat_embedding_enters_only_through_layer0_attention():
    # the residual stream is the hidden half: with wqkv[0]'s embedding columns zeroed, neither the
    # embedding table nor the mask embedding changes any output
    W = _weights64(MINI_CAT, 54)
    W["l0.wqkv"] = W["l0.wqkv"].copy()
    W["l0.wqkv"][:, :MINI.d_model] = 0.0
    rng = np.random.default_rng(54)
    hid = rng.standard_normal((2, 3 * MINI.d_model))
    ctx = [_ctx(MINI, 2, 540), _ctx(MINI, 6, 541)]
    st = {"last_token": np.asarray([3, 9]), "target_hidden": hid, "seq_len": np.asarray([2, 6])}
    a = O.draft_step_concat(MINI_CAT, W, st, lambda l, b: ctx[b][l], 3)
    W2 = dict(W)
    W2["embed"] = W["embed"] * 3.0 + 0.5
    W2["emb_mask"] = W["emb_mask"] - 2.0
    b = O.draft_step_concat(MINI_CAT, W2, st, lambda l, b_: ctx[b_][l], 3)
    assert np.array_equal(a["logits"], b["logits"])


def test_concat_rows_causality():
    # invariant 3 holds with concatenated rows: changing the token of request 0 changes row 0 onwards,
    # and rows after j never reach row j (perturb the hidden half of the placeholders via h_shared)
    W = _weights64(MINI_CAT, 53)
    rng = np.random.default_rng(53)
    hid = rng.standard_normal((1, 3 * MINI.d_model))
    ctx = [_ctx(MINI, 3, 530)]
    st = {"last_token": np.asarray([7]), "target_hidden": hid, "seq_len": np.asarray([3])}
    a = O.draft_step_concat(MINI_CAT, W, st, lambda l, b: ctx[b][l], 3)
    W2 = dict(W)
    W2["h_shared"] = W["h_shared"] + 1.0
    b = O.draft_step_concat(MINI_CAT, W2, st, lambda l, b_: ctx[b_][l], 3)
    assert np.array_equal(a["logits"][:, 0], b["logits"][:, 0])
    assert not np.allclose(a["logits"][:, 1], b["logits"][:, 1])


# ---------------------------------------------------------------- FP8 weights

def _e4m3_values():
    """Every finite E4M3 value from its bit fields: (-1)^s 2^(e-7) (1 + m/8) for e >= 1, (-1)^s m 2^-9 for
    e = 0; exponent 15 with mantissa 7 is NaN."""
    vals = []
    for code in range(256):
        sgn, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals.append((-v if sgn else v, m & 1))
    return vals


def test_fp8_rounding_brute_force_nearest_even():
    vals = _e4m3_values()
    grid = np.array(sorted(set(v for v, _ in vals)))
    mids = (grid[1:] + grid[:-1]) / 2
    rng = np.random.default_rng(61)
    xs = np.concatenate([grid, mids, rng.uniform(-464, 464, 3000), rng.uniform(-0.02, 0.02, 1000)])
    xs = xs[np.abs(xs) <= 464]
    got = O.fp8_e4m3_round(xs)
    for x, g in zip(xs, got):
        d = [(abs(v - x), odd, v) for v, odd in vals]
        dmin = min(t[0] for t in d)
        best = [t for t in d if t[0] == dmin]
        want = min(best, key=lambda t: t[1])[2] if len(best) > 1 else best[0][2]
        if x == 0:
            want = 0.0
        assert g == want, (x, g, want)


def test_fp8_rounding_hand_values():
    x = np.array([1.0, 1.0625, 1.1875, 448.0, 464.0, 2.0 ** -9, 3 * 2.0 ** -10, -0.5, 0.1, 300.0])
    want = np.array([1.0, 1.0, 1.25, 448.0, 448.0, 2.0 ** -9, 2.0 ** -8, -0.5, 0.1015625, 288.0])
    assert np.array_equal(O.fp8_e4m3_round(x), want)


def test_fp8_row_quantization_scale_and_round_trip():
    rng = np.random.default_rng(62)
    W = rng.standard_normal((6, 40)).astype(np.float32) * 0.02
    W[3] = 0.0
    D = O.quantize_fp8_rows(W)
    # the largest element of each nonzero row maps to +-448 s exactly; a zero row stays zero
    amax = np.abs(W).max(axis=1)
    for n in (0, 1, 2, 4, 5):
        assert np.abs(D[n]).max() == np.float64(np.float32(amax[n] / np.float32(448.0))) * 448.0
    assert not D[3].any()
    # quantizing the dequantized weights changes nothing; doubling a row doubles its dequantization
    assert np.array_equal(O.quantize_fp8_rows(D.astype(np.float32)), D)
    W2 = W.copy()
    W2[1] *= 2
    assert np.array_equal(O.quantize_fp8_rows(W2)[1], 2 * D[1])
    # relative error of a normal-range value is at most half a mantissa step (2^-4)
    big = np.abs(W) > amax[:, None] / 448 * 2.0 ** -6
    assert np.all(np.abs(D - W)[big] <= np.abs(W)[big] * 2.0 ** -4 * (1 + 1e-6))


# ---------------------------------------------------------------- sampled verify (temperature > 0)

def test_draw_inverse_cdf_brute_force():
    w = np.array([0.0, 1.0, 0.0, 2.0, 1.0, 0.0])
    for v in np.linspace(0.0, 0.999, 37):
        # brute force: walk the bins of total 4 and stop at the first whose right edge passes v * 4
        acc, want = 0.0, None
        for x, wx in enumerate(w):
            acc += wx
            if acc > v * 4.0:
                want = x
                break
        assert O.draw_inverse_cdf(w, v) == want


def test_sampled_verify_emits_the_target_distribution():
    # speculative sampling's defining property: whatever the (greedy) draft, the token emitted at the first
    # position is distributed as p_0 = softmax(T_0 / temperature), and after an acceptance the next one as
    # p_1; the acceptance rate of draft x is p_0(x). Checked by Monte Carlo against scipy's softmax.
    from scipy.special import softmax
    rng = np.random.default_rng(41)
    V, K, tau = 6, 2, 0.7
    T = rng.standard_normal((1, K + 1, V)) * 1.5
    draft = np.array([[int(np.argsort(T[0, 0])[-2]), int(np.argmax(T[0, 1]))]])  # not the argmax at position 0
    N = 40000
    p0 = softmax(T[0, 0] / tau)
    p1 = softmax(T[0, 1] / tau)
    first, second, acc0 = np.zeros(V), np.zeros(V), 0
    for _ in range(N):
        u = rng.random((1, K))
        v = rng.random((1, K + 1))
        out = O.verify_sampled(T, draft, tau, u, v)
        first[out["t"][0, 0]] += 1
        if out["n"][0] >= 1:
            acc0 += 1
            second[out["t"][0, 1]] += 1
    sig = np.sqrt(p0 * (1 - p0) / N)
    assert np.all(np.abs(first / N - p0) < 5 * sig + 1e-12)
    assert abs(acc0 / N - p0[draft[0, 0]]) < 5 * math.sqrt(p0[draft[0, 0]] * (1 - p0[draft[0, 0]]) / N)
    n1 = second.sum()
    sig1 = np.sqrt(p1 * (1 - p1) / n1)
    assert np.all(np.abs(second / n1 - p1) < 5 * sig1 + 1e-12)


def test_sampled_verify_near_zero_temperature_is_greedy():
    # with logit gaps far above the temperature, p is one-hot at the argmax: the sampled rule reduces to
    # the greedy one (accept while the draft equals the argmax, bonus = argmax at the first mismatch)
    rng = np.random.default_rng(42)
    B, K, V = 64, 4, 16
    T = np.stack([rng.permutation(V) for _ in range(B * (K + 1))]).reshape(B, K + 1, V).astype(np.float64)
    T = T + rng.standard_normal(T.shape) * 0.01
    t_greedy = O.argmax_first(T)
    draft = np.where(rng.random((B, K)) < 0.7, t_greedy[:, :K], (t_greedy[:, :K] + 1) % V)
    u = rng.uniform(0.01, 0.99, (B, K))
    v = rng.uniform(0.01, 0.99, (B, K + 1))
    s = O.verify_sampled(T, draft, 1e-3, u, v)
    g = O.verify(T, draft)
    assert np.array_equal(s["accept_len"], g["accept_len"])
    assert np.array_equal(s["bonus"], g["bonus"])
    for b in range(B):
        assert np.array_equal(s["t"][b, :g["accept_len"][b]], g["t"][b, :g["accept_len"][b]])


def test_weights_fp8_quantizes_exactly_the_projection_matrices():
    # the FP8 reading stores the seven projection matrices (fc, every layer's wqkv / wo / wgate / wup / wdown,
    # lm_head) as per-row E4M3 codes; everything else (embedding table, mask embedding, shared hidden, norm
    # gains) keeps its exact value. Checked key by key on a 2-layer drafter.
    W = _weights64(MINI, 63)
    Q = O.weights_fp8(MINI, W)
    assert set(Q) == set(W)
    proj = {"fc", "lm_head"} | {f"l{l}.{n}" for l in range(MINI.n_layers)
                                for n in ("wqkv", "wo", "wgate", "wup", "wdown")}
    assert proj <= set(W) and len(proj) == 2 + 5 * MINI.n_layers
    for k, v in W.items():
        if k in proj:
            assert Q[k].shape == v.shape
            assert not np.array_equal(Q[k], v), f"{k}: not quantized"
            # every row is the per-row quantization of that source row alone
            for n in (0, v.shape[0] // 2, v.shape[0] - 1):
                assert np.array_equal(Q[k][n], O.quantize_fp8_rows(v[n:n + 1])[0]), (k, n)
            # and every value sits on its row's E4M3 grid: q / s is an E4M3 value
            s = np.float64(np.float32(np.abs(v.astype(np.float32)).max(axis=1)) / np.float32(448.0))
            codes = Q[k] / s[:, None]
            assert np.array_equal(O.fp8_e4m3_round(codes), codes), k
        else:
            assert np.array_equal(Q[k], v), f"{k}: changed by the FP8 conversion"
