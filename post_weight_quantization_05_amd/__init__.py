"""GPTQ per-layer quantization on MI355X (gfx950): HIP kernels behind the C ABI of libgptq_mi355x.so.

The Python layer only marshals arguments; see include/gptq_mi355x.h for the ABI.
"""
from ._lib import (  # noqa: F401
    GPTQ_BF16, GPTQ_F32, GPTQ_FACTOR_INVERSE_RECHOL, GPTQ_FACTOR_R_FORM, GPTQ_FACTOR_REVERSED, GPTQ_GRID_ASYMMETRIC,
    GPTQ_GRID_SYMMETRIC, GPTQError, LIB_PATH, load,
    status_string,
)
from .gptq import (  # noqa: F401
    HessianState, QuantizedLayer, QuantResult, apply_layerwise, dequant_matmul, factor_route, gptq_quantize,
    hessian_accumulate, pack_codes, prepare_chol, quantize_layer,
)
