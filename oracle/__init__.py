"""CPU oracle of the NVFP4 block-scaled MoE layer.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference the GPU
kernels are checked against.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the library and its Python
binding never do, and there is no CPU fallback built on it.  It shares no code,
tables or constants with the HIP sources.

Modules:
  formats  E2M1 / E4M3 tables and nearest-even encoders, bfloat16 rounding
  quant    NVFP4 quantise / dequantise (per-tensor + per-16-block scales)
  moe      route, permute, grouped GEMM, SwiGLU, combine, whole layer
  mx       MXFP4 (E2M1 with an E8M0 scale per 32): quantise, dequantise,
           grouped GEMM, SwiGLU requantisation
  fp8      FP8 E4M3 with float32 block scales (1 x 128 activations,
           128 x 128 weights): quantise, dequantise, grouped GEMM

Parity status: every function is pinned by tests/test_oracle_*.py against
closed forms, library routines (torch.float8_e4m3fn and float8_e8m0fnu, numpy
sorting, scipy's expit/softmax), exact rational brute force and invariants.  The Zipf-skewed
routing recipe has no pin from the pages (it is a synthetic input recipe).
"""
from . import formats, quant, moe, mx, fp8  # noqa: F401
from .quant import quantize, dequantize, dequantize_unscaled, pack_codes, unpack_codes  # noqa: F401
from .moe import (route, permute, grouped_gemm, grouped_gemm_blockwise, swiglu,  # noqa: F401
                  swiglu_quantize, combine, moe_layer, quantize_experts)
