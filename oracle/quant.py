"""NVFP4 quantisation and dequantisation (CPU oracle; test infrastructure).

Format (the block-scaled MMA in "From Empirical Limits to Research-Driven
Optimization: The SM120 FP4 Kernel Research Campaign", section "Section 1:
CUTLASS Kernels - The Foundation"): E2M1 element codes, one unsigned E4M3 scale
per 16 consecutive elements along the reduction dimension, plus one float32
per-tensor scale.

The pages print no quantiser, so this module takes the plainest reading that
makes the block scale use the whole E4M3 range:

* per-tensor scale   g   = amax(|x|) / 2688            (2688 = 6 * 448; float32
                                                        division; g = 1 if amax = 0)
* block scale        s_b = E4M3( (absmax_b / 6) / g )  (two float32 divisions left
                                                        to right; nearest-even;
                                                        clamped to 448)
* element code       q   = E2M1( x / (f32(s_b) * g) )  (float32 product, float32
                                                        division; nearest-even on
                                                        |.|; saturate at 6; sign bit
                                                        copied from x; s_b = 0 gives
                                                        code 0)
* dequantised value  x^  = E2M1(q) * E4M3(s_b) * g

Byte layout: row-major, blocks along the last (reduction) axis; element 2i sits
in the low nibble of byte i; scales are one byte per block, row-major
[rows, cols/16].  Every decision is taken in float32, the precision the GPU
kernels use, so the codes are reproducible bit for bit.
"""
from __future__ import annotations

import numpy as np

from .formats import (e2m1_decode, e2m1_encode_magnitude, e4m3_decode,
                      e4m3_encode_satfinite)

BLOCK = 16
F32_6 = np.float32(6.0)
F32_2688 = np.float32(2688.0)


def global_scale(x32: np.ndarray) -> np.float32:
    """g = amax(|x|) / 2688 in float32; 1 when the tensor is all zeros."""
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / F32_2688)


def block_scale_codes(x32: np.ndarray, g: np.float32) -> np.ndarray:
    """E4M3 code of each 16-element block of the last axis."""
    rows, cols = x32.shape
    blocks = np.abs(x32).reshape(rows, cols // BLOCK, BLOCK)
    absmax = blocks.max(axis=2).astype(np.float32)
    t = (absmax / F32_6).astype(np.float32)
    t = (t / np.float32(g)).astype(np.float32)
    return e4m3_encode_satfinite(t)


def element_codes(x32: np.ndarray, scales: np.ndarray, g: np.float32) -> np.ndarray:
    """4-bit code of every element (unpacked, one per uint8)."""
    rows, cols = x32.shape
    s_val = e4m3_decode(scales).astype(np.float32)                 # exact
    scale_eff = (s_val * np.float32(g)).astype(np.float32)         # float32 product
    scale_eff = np.repeat(scale_eff, BLOCK, axis=1)
    ax = np.abs(x32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (ax / scale_eff).astype(np.float32)                     # float32 division
    v = np.where(scale_eff > 0, v, np.float32(0))
    v = np.minimum(v, np.float32(6.0))
    mag = e2m1_encode_magnitude(v)
    sign = np.signbit(x32).astype(np.uint8) << 3
    code = (mag | sign).astype(np.uint8)
    zero_block = np.repeat(scales == 0, BLOCK, axis=1)
    return np.where(zero_block, np.uint8(0), code).astype(np.uint8)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def quantize(x: np.ndarray, g: float | None = None):
    """x [rows, cols] (float32 values) -> (codes u8 [rows, cols/2],
    scales u8 [rows, cols/16], g float32).  ``g`` given means a caller-supplied
    per-tensor scale (static calibration); None computes it from amax."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    assert x32.ndim == 2 and x32.shape[1] % BLOCK == 0
    gg = global_scale(x32) if g is None else np.float32(g)
    scales = block_scale_codes(x32, gg)
    codes = element_codes(x32, scales, gg)
    return pack_codes(codes), scales, gg


def dequantize_unscaled(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E2M1(q) * E4M3(s_b) as float64 (exact), without the per-tensor scale."""
    q = e2m1_decode(unpack_codes(codes))
    s = np.repeat(e4m3_decode(scales), BLOCK, axis=-1)
    return q * s


def dequantize(codes: np.ndarray, scales: np.ndarray, g: float) -> np.ndarray:
    return dequantize_unscaled(codes, scales) * np.float64(np.float32(g))
