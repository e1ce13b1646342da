"""Seeded synthetic verify batches shared by the oracle, the tests and the bench.

Holds no attention arithmetic: it only draws and lays out inputs.
"""
from .synth import (  # noqa: F401
    BF16_NAN, CONFIGS, CONFIG_SEEDS, FP8_KV_SCALE, FP8_NAN, LATENT, NOPE, PAGE, SHARP_Q_SCALE,
    ConfigSpec, SparsePool, bf16_bits_to_fp8_codes, fp8_cache,
    KvUpdateInputs, VerifyInputs, bf16_bits_to_f32, build_inputs, f32_to_bf16_bits, make_config,
    make_kv_update_inputs, ramp_scores, referenced_kv_bytes,
)
