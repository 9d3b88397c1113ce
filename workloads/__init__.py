"""Seeded synthetic workloads shared by the oracle's tests, the GPU tests and
the benchmark. Holds shapes and random draws only, no attention arithmetic."""
from .configs import (CONFIGS, GQLA_CONFIGS, PAGE, DecodeConfig, GqlaConfig, bytes_per_token,
                      MLA_SCALE, GQA_SCALE)
from .gen import (make_inputs, make_gqla_inputs, config_inputs, f32_to_bf16_bits, draw_seqlens,
                  BF16_NAN)

__all__ = ["CONFIGS", "GQLA_CONFIGS", "GqlaConfig", "make_gqla_inputs", "PAGE", "DecodeConfig", "bytes_per_token", "MLA_SCALE",
           "GQA_SCALE", "make_inputs", "config_inputs", "f32_to_bf16_bits",
           "draw_seqlens", "BF16_NAN"]
