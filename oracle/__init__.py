"""CPU oracle of the Dual-Flow Transformer grouped decode step.

TEST INFRASTRUCTURE. This package is a plain, slow, float64 restatement of
what the decode step computes. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.
It shares no code with the HIP library: its only dependency in this
repository is the seeded input generator (``synth``).
"""
from .dualflow import (  # noqa: F401
    Model, Cache, StepResult,
    decode_bf16, round_to, layer_norm, gelu, softmax,
    attention_one, attention_dual, mix_head, topk_ids,
    decode_step, prefill_primary, run_tiny,
)
