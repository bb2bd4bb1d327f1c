"""Seeded synthetic inputs (weights W and calibration activations X) for the GPTQ layer path.

This package draws random numbers and encodes them as fp32 or bf16 bit patterns. It holds none of
the quantization method's arithmetic, so both the CPU oracle and the GPU path may read from it.
"""
from .workloads import (  # noqa: F401
    SEGMENT_ROWS,
    LayerConfig,
    CONFIGS,
    config_by_name,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    gen_w,
    gen_x,
    gen_layer,
    custom_config,
    MLPConfig,
    MLP_CONFIGS,
    mlp_config_by_name,
    gen_mlp,
)
