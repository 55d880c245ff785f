"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This package draws numbers and lays them out; it computes nothing of the drafting method
itself (no norms, projections, attention, argmax or acceptance logic).
"""

from .workloads import (  # noqa: F401
    DrafterShape,
    Workload,
    TINY_FP32,
    QWEN3_CODER,
    GPT_OSS_20B,
    WORKLOADS,
    workload,
)
from .inputs import (  # noqa: F401
    bf16_bits,
    bf16_bits_to_f32,
    round_bf16,
    make_weights,
    make_state,
    make_kv_cache,
    plant_target_logits,
    random_draft,
    churn_finished,
)
