"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the benchmark."""
from .synth import (  # noqa: F401
    BLOCK,
    Workload,
    bf16_bits,
    build_inputs,
    config_8b_decode,
    config_long_layer,
    config_mixed_step,
    config_prefill,
    config_prefill_r64,
    config_serving_mix,
    config_tiny_f32,
    decode_workload,
    mixed_workload,
    prefill_workload,
    round_bf16,
)
