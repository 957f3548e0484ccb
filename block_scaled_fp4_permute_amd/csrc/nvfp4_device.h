// Device-side helpers of the NVFP4 path for gfx950 (CDNA4).
//
// Formats: E2M1 element codes (1 sign, 2 exponent bits with bias 1, 1 mantissa
// bit), unsigned E4M3 block scales (4 exponent bits with bias 7, 3 mantissa
// bits, subnormals, max 448), one block per 16 K-elements, FP32 accumulation -
// the operand types of the block-scaled MMA in "From Empirical Limits to
// Research-Driven Optimization: The SM120 FP4 Kernel Research Campaign",
// section "Section 1: CUTLASS Kernels - The Foundation".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ bfloat16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// nearest-even rounding of a finite float32 to bfloat16
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ------------------------------------------------------------------ E4M3
// Value of an unsigned E4M3 code (bits 6..0; the NaN code never occurs here).
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  const uint32_t e = (code >> 3) & 0xFu;
  const uint32_t m = code & 7u;
  // normal: 2^(e-7) * (1 + m/8) -> float32 exponent field e + 120, mantissa m << 20
  const float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
  const float sub = static_cast<float>(m) * 0.001953125f;  // m * 2^-9
  return e ? normal : sub;
}

// Non-negative finite float32 -> E4M3 code, nearest with ties to even; values
// at or above 448 give 448 (saturating), values at or below 2^-10 give 0.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float t) {
  if (!(t > 0.0f)) return 0u;
  if (t >= 448.0f) return 0x7Eu;
  const uint32_t u = __float_as_uint(t);
  const int ex = static_cast<int>(u >> 23) - 127;
  if (ex < -6) {
    // E4M3 subnormal range: value = m * 2^-9.  t * 512 is exact; rintf rounds
    // half to even; m = 8 is the smallest normal (code 8), which is consistent.
    return static_cast<uint32_t>(rintf(t * 512.0f));
  }
  // keep 3 mantissa bits with round-to-nearest-even at bit 20; a carry moves into
  // the exponent, which is the correct next binade
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  const uint32_t e = (r >> 23) - 120u;       // biased E4M3 exponent (>= 1 here)
  const uint32_t code = (e << 3) | ((r >> 20) & 7u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// ------------------------------------------------------------------ E2M1
// E2M1 codes from the gfx950 conversion instruction with scale 1.  For every
// float v that is not a NaN it returns the magnitude of v rounded to the grid
// 0, .5, 1, 1.5, 2, 3, 4, 6 - nearest, with ties to the code whose mantissa bit
// is 0, saturating at 6 (decision points 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5,
// the lower code winning at 0.25, 1.25, 2.5 and 5) - with the sign bit of v
// as bit 3; infinities give 7 | sign, and so do NaNs.  Checked on the device
// against that rule for every finite float of either sign, in both nibble
// positions: no difference.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, 0.0f, 1.0f, 0) & 0xFu;
}

// v[B..B+7] -> one word, element B+i in nibble i
template <int B>
__device__ __forceinline__ uint32_t e2m1_pack8(const float (&v)[16]) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[B], v[B + 1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[B + 2], v[B + 3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[B + 4], v[B + 5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[B + 6], v[B + 7], 1.0f, 3);
}

// Per-tensor scale from the absolute maximum: g = amax / 2688 (2688 = 6 * 448),
// or 1 for an all-zero tensor.
__device__ __forceinline__ float global_scale_from_amax(float amax) {
  return amax > 0.0f ? amax / 2688.0f : 1.0f;
}

// Encode one block of 16 float32 values with per-tensor scale g.  Writes the
// 8 packed code bytes (element 2i in the low nibble of byte i) as two
// 32-bit words and returns the E4M3 scale code.
__device__ __forceinline__ uint32_t encode_block16(const float (&x)[16], float g,
                                                   uint32_t& lo, uint32_t& hi) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float t = (amax / 6.0f) / g;
  const uint32_t s = f32_to_e4m3_sat(t);
  const float scale_eff = e4m3_to_f32(s) * g;
  uint32_t w[2] = {0u, 0u};
  if (s != 0u) {
    // |x| / scale_eff rounded to nearest, from the correctly rounded
    // reciprocal: q0 = a*y, r = a - q0*b (exact with an FMA), q = q0 + r*y.
    // With y = RN(1/b) this gives RN(a/b) whenever nothing underflows or
    // overflows (Markstein, IBM J. Res. Dev. 34(1), 1990).  The quotients it
    // misses come from subnormal |x| and lie below 2^-50, far under the
    // smallest E2M1 rounding boundary (0.25).  A q0 that overflows makes q a
    // NaN, which encodes like the infinity (code 7).  A reciprocal that
    // overflows (b below 2^-128) takes true divisions.  The sign bit is copied
    // from x, -0 included.
    const float y = 1.0f / scale_eff;
    const bool via_rcp = scale_eff > 0.0f && y < __builtin_huge_valf();
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float a = fabsf(x[i]);
      float q;
      if (via_rcp) {
        const float q0 = a * y;
        q = __builtin_fmaf(__builtin_fmaf(-q0, scale_eff, a), y, q0);
      } else {
        q = scale_eff > 0.0f ? a / scale_eff : 0.0f;
      }
      v[i] = __builtin_copysignf(q, x[i]);
    }
    w[0] = e2m1_pack8<0>(v);
    w[1] = e2m1_pack8<8>(v);
  }
  lo = w[0];
  hi = w[1];
  return s;
}

// ------------------------------------------------------------------ decode to FP16
// E4M3 (bias 7) and FP16 (bias 15) subnormals line up, so the E4M3 code shifted
// into the FP16 exponent/mantissa position is the FP16 bit pattern of
// scale * 2^-8 for every code (subnormal codes land on FP16 subnormals).
__device__ __forceinline__ _Float16 e4m3_to_f16_div256(uint32_t code) {
  return __builtin_bit_cast(_Float16, static_cast<uint16_t>((code & 0x7Fu) << 7));
}

// Eight E2M1 codes (one 32-bit word, element 2i in the low nibble of byte i)
// -> eight FP16 values multiplied by the block scale.  The hardware conversion
// applies the exponent of its scale operand, so 256 is exact and yields
// E2M1 * 256; one packed FP16 multiply by scale * 2^-8 then gives E2M1 * scale.
// E2M1 * E4M3 needs at most 6 significant bits and lies in [2^-10, 2688], so
// every result is an exact, normal FP16 value.
__device__ __forceinline__ half8 decode8_f16(uint32_t w, _Float16 scale_div256) {
  const half2v sc = {scale_div256, scale_div256};
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0);
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1);
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2);
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3);
  p0 *= sc;
  p1 *= sc;
  p2 *= sc;
  p3 *= sc;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// ------------------------------------------------------------------ misc
__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + expf(-x)); }

// silu with a reciprocal-based division (at most ~2 ulp from silu_f32); used
// where the result is re-quantised from values that already differ from the
// exact ones by rounding.
__device__ __forceinline__ float silu_fast(float x) { return __fdividef(x, 1.0f + expf(-x)); }

// ------------------------------------------------------------------ 16-lane rows
// DPP lane exchanges inside each row of 16 lanes (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8-lane half
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within the row

// maximum over the 16 lanes of the row, returned to every lane of the row
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v))));
  return v;
}


}  // namespace nvfp4
