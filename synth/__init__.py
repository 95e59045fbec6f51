"""Seeded synthetic inputs shared by the oracle and the GPU path (no loss arithmetic)."""
from .inputs import (CONFIGS, KDConfig, bf16_bits_to_f32, f32_to_bf16_bits,  # noqa: F401
                     get_config, make_inputs, make_teacher_cache, row_prefix)
