"""The oracle's pins catch plausible mistakes (CPU, no GPU).

Each case plants one mistake in a copy of the oracle's source (a dropped term, a wrong sign or index, a
transposed operand, an off-by-one), loads that copy as a module of its own, points the pins of
tests/test_oracle_pins.py at it and requires at least one pin to fail. A control case loads the unmodified
source the same way and requires every pin to pass, so a failure is due to the planted mistake and not to
the harness. Every planted snippet must occur exactly once in the oracle's source, so a rewrite of the
oracle that removes it fails here loudly instead of silently testing nothing.
"""

from __future__ import annotations

import inspect
import types

import pytest

from oracle import pe_oracle as O
import tests.test_oracle_pins as P

# (name, original snippet, planted replacement)
MUTATIONS = [
    ("dropped attention residual",
     'x = x + linear(o.reshape(B * K, Hq * hd), W[f"l{l}.wo"])',
     'x = linear(o.reshape(B * K, Hq * hd), W[f"l{l}.wo"])'),
    ("dropped MLP residual",
     'x = x + linear(a, W[f"l{l}.wdown"])',
     'x = linear(a, W[f"l{l}.wdown"])'),
    ("GQA head map interleaved instead of grouped",
     "        g = h // G\n        keys = np.concatenate",
     "        g = h % Hkv\n        keys = np.concatenate"),
    ("RoPE rotation sign",
     "x1 * c - x2 * s, x2 * c + x1 * s",
     "x1 * c + x2 * s, x2 * c - x1 * s"),
    ("RoPE frequency exponent",
     "inv_freq = base ** (-2.0 * i / head_dim)",
     "inv_freq = base ** (-1.0 * i / head_dim)"),
    ("keys not rotated",
     "k = rope(k, pos, shape.rope_base)",
     "k = k"),
    ("causal mask off by one (row sees the next row)",
     "n = L + j + 1\n            s = keys[:n]",
     "n = L + j + 2\n            s = keys[:n]"),
    ("missing 1/sqrt(hd) score scale",
     "s = keys[:n] @ q[j, h] * scale",
     "s = keys[:n] @ q[j, h]"),
    ("missing final norm",
     'z = linear(rms_norm(x, W["final_norm"], eps), W["lm_head"])',
     'z = linear(x, W["lm_head"])'),
    ("row 0 without the token embedding",
     'X[:, 0, :] = linear(target_hidden, W["fc"]) + W["embed"][last_token]',
     'X[:, 0, :] = linear(target_hidden, W["fc"])'),
    ("placeholder rows without the mask embedding",
     'X[:, 1:, :] = (W["h_shared"] + W["emb_mask"])[None, None, :]',
     'X[:, 1:, :] = W["h_shared"][None, None, :]'),
    ("row positions start one late",
     "pos = (np.asarray(seq_len, dtype=np.int64)[:, None] + np.arange(K)[None, :]).reshape(-1)",
     "pos = (np.asarray(seq_len, dtype=np.int64)[:, None] + np.arange(1, K + 1)[None, :]).reshape(-1)"),
    ("RMSNorm without eps",
     "return x / np.sqrt(ms + eps) * g",
     "return x / np.sqrt(ms) * g"),
    ("SiLU sign",
     "return x / (1.0 + np.exp(-x))",
     "return x / (1.0 + np.exp(x))"),
    ("gate and up swapped",
     'a = silu(linear(u, W[f"l{l}.wgate"])) * linear(u, W[f"l{l}.wup"])',
     'a = silu(linear(u, W[f"l{l}.wup"])) * linear(u, W[f"l{l}.wgate"])'),
    ("argmax ties to the highest index",
     "return np.argmax(z, axis=-1).astype(np.int32)",
     "return (z.shape[-1] - 1 - np.argmax(z[..., ::-1], axis=-1)).astype(np.int32)"),
    ("verify counts matches past the first mismatch",
     "        n[b] = i\n    accept_len = n + 1",
     "        n[b] = int((draft[b] == t[b, :K]).sum())\n    accept_len = n + 1"),
    ("bonus token taken one position late",
     "bonus = t[np.arange(B), n]\n    return {\"t\": t, \"n\": n, \"accept_len\": accept_len",
     "bonus = t[np.arange(B), np.minimum(n + 1, K)]\n    return {\"t\": t, \"n\": n, \"accept_len\": accept_len"),
    ("seq_len advanced by the accepted drafts only",
     "seq_next_all = (np.asarray(seq_len) + acc).astype(np.int32)",
     "seq_next_all = (np.asarray(seq_len) + acc - 1).astype(np.int32)"),
    ("compaction keeps the finished requests",
     "keep = [b for b in range(B) if not fin[b]]",
     "keep = [b for b in range(B) if fin[b]]"),
    ("speedup divides by 1 - eps",
     "return tokens_per_target_pass(K, alpha) / (1.0 + eps)",
     "return tokens_per_target_pass(K, alpha) / (1.0 - eps)"),
    ("sampled verify: acceptance test inverted",
     "if u[b, i] < p[x]:",
     "if u[b, i] > p[x]:"),
    ("sampled verify: residual keeps the rejected draft",
     "            r[x] = 0.0\n",
     "            r[x] = r[x]\n"),
    ("sampled verify: temperature multiplies the logits",
     "x = np.asarray(z, dtype=np.float64) / temperature",
     "x = np.asarray(z, dtype=np.float64) * temperature"),
    ("FP8 rounding: ties away from zero",
     "up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2.0) == 1.0))",
     "up = frac >= 0.5"),
    ("FP8 scale for a 240 maximum",
     "amax / np.float32(448.0)",
     "amax / np.float32(240.0)"),
    ("FP8 weights leave the LM head in bf16",
     '("fc", "wqkv", "wo", "wgate", "wup", "wdown", "lm_head")',
     '("fc", "wqkv", "wo", "wgate", "wup", "wdown")'),
    ("autoregressive feedback without the drafted token's embedding",
     'row = hidden[-1] + W["embed"][tok]',
     "row = hidden[-1]"),
    ("concatenated rows: halves in the wrong order",
     'u = np.concatenate([rms_norm(E.reshape(B * K, d), W["embed_norm"], eps), u], axis=1)',
     'u = np.concatenate([u, rms_norm(E.reshape(B * K, d), W["embed_norm"], eps)], axis=1)'),
    ("catch-up drafts taken from the row after the last real row",
     "rows = n_real[:, None] - 1 + np.arange(K)[None, :]",
     "rows = np.minimum(n_real[:, None] + np.arange(K)[None, :], X.shape[1] - 1)"),
]


def _pins():
    """Every pin of test_oracle_pins as a zero-argument callable (parametrized pins once per value)."""
    out = []
    for name, fn in inspect.getmembers(P, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != P.__name__:
            continue
        params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not params:
            out.append((name, fn, ()))
            continue
        argnames, values = params[0].args[0], params[0].args[1]
        nargs = len([a for a in argnames.split(",") if a.strip()]) if isinstance(argnames, str) else len(argnames)
        for v in values:
            out.append((f"{name}[{v}]", fn, tuple(v) if nargs > 1 else (v,)))
    # cheap pins first, the Monte Carlo ones last
    slow = ("sampled_verify_emits", "fp8_rounding_brute", "planted_generator")
    return sorted(out, key=lambda t: any(s in t[0] for s in slow))


def _load(src: str) -> types.ModuleType:
    mod = types.ModuleType("pe_oracle_planted")
    mod.__file__ = O.__file__
    exec(compile(src, O.__file__, "exec"), mod.__dict__)
    return mod


def _failing_pins(monkeypatch, mod, stop_at_first=True):
    monkeypatch.setattr(P, "O", mod)
    failed = []
    for name, fn, args in _pins():
        try:
            fn(*args)
        except Exception as e:  # an assertion, or the planted mistake breaking a shape
            failed.append((name, type(e).__name__))
            if stop_at_first:
                break
    return failed


def test_unmodified_oracle_passes_every_pin_when_loaded_the_same_way(monkeypatch):
    assert _failing_pins(monkeypatch, _load(inspect.getsource(O)), stop_at_first=False) == []


@pytest.mark.parametrize("name,orig,planted", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(monkeypatch, name, orig, planted):
    src = inspect.getsource(O)
    assert src.count(orig) == 1, f"snippet for '{name}' occurs {src.count(orig)} times in the oracle"
    failed = _failing_pins(monkeypatch, _load(src.replace(orig, planted)))
    assert failed, f"no pin fails with the planted mistake '{name}'"
