"""Drafter shapes and synthetic workloads.

The shapes follow the drafter the P-EAGLE pages describe (a 4-layer head over a Qwen3-Coder-30B-A3B or
GPT-OSS-20B target; "Parallelize speculative decoding with P-EAGLE on Amazon SageMaker AI", solution
overview, step-by-step drafting process) plus a tiny fp32 shape for exact checks. Concurrency, draft
depth and acceptance ranges follow the pages' benchmark tables (concurrency 1-128, K in {3, 7, 11},
acceptance 0.5-0.85). The pages' own benchmark suites (HumanEval, SPEED-Bench, MT-Bench) are not used;
these seeded synthetic inputs stand in for them.
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class DrafterShape:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    dtype: str  # "f32" or "bf16": weights, KV cache, target hiddens and target logits
    weight_seed: int = 0  # seed of this synthetic drafter's weights (shared by every workload on it)
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    # input rows as the concatenation [embedding || hidden] (2d wide into layer 0's attention) instead of
    # their sum; layer 0's wqkv is then [qkv_dim, 2d] and the embedding half has its own RMSNorm gain
    row_concat: bool = False

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_dim(self) -> int:
        return self.q_dim + 2 * self.kv_dim

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


TINY_FP32 = DrafterShape("tiny-fp32", 1, 256, 4, 4, 64, 512, 4096, "f32", 1000)
QWEN3_CODER = DrafterShape("qwen3-coder-30b-a3b-shaped", 4, 2048, 32, 4, 128, 6144, 151936, "bf16", 2000)
QWEN3_CODER_CONCAT = DrafterShape("qwen3-coder-30b-a3b-shaped-concat", 4, 2048, 32, 4, 128, 6144, 151936, "bf16",
                                  2100, row_concat=True)
GPT_OSS_20B = DrafterShape("gpt-oss-20b-shaped", 4, 2880, 64, 8, 64, 8640, 201088, "bf16", 5000)


@dataclass(frozen=True)
class Workload:
    """One batch of drafting requests.

    ctx: inclusive range of the per-request drafter context length L_b (uniform integers).
    alpha: per-position probability that the target's argmax is planted on the draft token; a pair
        means one value per request, drawn uniformly from that range.
    churn: fraction of requests that finish after each step and are replaced by new requests whose
        context length is drawn from new_ctx.
    """

    name: str
    shape: DrafterShape
    B: int
    K: int
    ctx: tuple
    alpha: object
    seed: int
    churn: float = 0.0
    new_ctx: tuple = (0, 0)
    steps: int = 1
    tags: tuple = field(default_factory=tuple)

    @property
    def M(self) -> int:
        return self.B * self.K

    @property
    def n_slots(self) -> int:
        # a few spare slots so the slot indirection is exercised (live slots are a random subset)
        return self.B + max(1, self.B // 4)

    @property
    def max_ctx(self) -> int:
        need = self.ctx[1] + max(self.steps, 2) * (self.K + 1)
        return ((need + 63) // 64) * 64


def _build():
    w = []
    w.append(Workload("tiny-fp32-B1-K4-L64", TINY_FP32, 1, 4, (64, 64), 0.7, 1000, tags=("small",)))
    w.append(Workload("qwen3coder-bf16-B1-K3-L2048", QWEN3_CODER, 1, 3, (2048, 2048), 0.7, 2000,
                      tags=("headline",)))
    i = 0
    for K in (3, 7, 11):
        for B in (1, 4, 8):
            w.append(Workload(f"qwen3coder-bf16-B{B}-K{K}-L1024to4096", QWEN3_CODER, B, K, (1024, 4096),
                              (0.5, 0.85), 3000 + i, tags=("sweep",)))
            i += 1
    for i, B in enumerate((32, 128)):
        w.append(Workload(f"qwen3coder-bf16-B{B}-K7-L512to4096-churn", QWEN3_CODER, B, 7, (512, 4096), 0.6,
                          4000 + i, churn=0.1, new_ctx=(256, 1024), steps=16, tags=("churn",)))
    w.append(Workload("gptoss20b-bf16-B64-K10-L2048to8192", GPT_OSS_20B, 64, 10, (2048, 8192), 0.7, 5000,
                      tags=("large",)))
    return {x.name: x for x in w}


WORKLOADS = _build()


def workload(name: str) -> Workload:
    return WORKLOADS[name]
