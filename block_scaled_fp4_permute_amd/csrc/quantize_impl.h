// NVFP4 quantisation bodies shared by the quantiser's own kernels and the
// launches that pair it with routing: the global absolute maximum in two
// deterministic levels (one partial maximum per workgroup, no atomics; every
// encoding workgroup reduces the partials), then one thread per 16-value
// block.
#pragma once

#include "nvfp4_internal.h"

namespace nvfp4 {

// ------------------------------------------------------------------ helpers
template <int DT>
__device__ __forceinline__ void load16(const void* base, size_t elem0, float (&x)[16]) {
  if constexpr (DT == 1) {  // bf16: 32 bytes
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem0);
    const uint4 a = p[0], b = p[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {  // float32: 64 bytes
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = p[i];
      x[4 * i] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
  }
}

// Global absolute maximum in two deterministic levels: k_*_amax writes one
// partial maximum per workgroup (no atomics), and every workgroup of the
// encoder reduces the partials before it computes g.
constexpr int kAmaxBlocks = 1024;

__device__ __forceinline__ void block_max_store(float v, float* partial, int blk) {
  __shared__ float s_red[4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) partial[blk] = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
}

// per-tensor scale from the partial maxima (or the caller's scale).  All
// threads of the workgroup read the partials with independent loads (one
// round trip), then reduce through one LDS step.
__device__ __forceinline__ float reduce_scale(const float* g_in, const float* partial, int nparts) {
  if (g_in) return *g_in;
  __shared__ float s_part[4];
  float m = 0.0f;
#pragma unroll 4
  for (int i = threadIdx.x; i < nparts; i += 256) m = fmaxf(m, partial[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = m;
  __syncthreads();
  return global_scale_from_amax(fmaxf(fmaxf(s_part[0], s_part[1]), fmaxf(s_part[2], s_part[3])));
}

inline int amax_grid(int64_t nblocks) {
  const int64_t want = (nblocks + 255) / 256;
  return static_cast<int>(want < kAmaxBlocks ? (want > 0 ? want : 1) : kAmaxBlocks);
}

// ------------------------------------------------------------------ quantise
// workgroup `blk` of `nblk`: the maximum of |x| over its share of the blocks
template <int DT>
__device__ __forceinline__ void amax_body(const void* __restrict__ x, int64_t nblocks, float* __restrict__ partial,
                                          int blk, int nblk) {
  float m = 0.0f;
  for (int64_t b = blk * 256ll + threadIdx.x; b < nblocks; b += static_cast<int64_t>(nblk) * 256) {
    float v[16];
    load16<DT>(x, b * 16, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  block_max_store(m, partial, blk);
}

template <int DT>
__global__ __launch_bounds__(256) void k_amax_blocks(const void* __restrict__ x, int64_t nblocks,
                                                     float* __restrict__ partial) {
  amax_body<DT>(x, nblocks, partial, blockIdx.x, gridDim.x);
}

// workgroup `blk`: encodes blocks [256 blk, 256 blk + 256)
template <int DT>
__device__ __forceinline__ void quantize_body(const void* __restrict__ x, int64_t nblocks,
                                              const float* __restrict__ g_in, const float* __restrict__ partial,
                                              int nparts, float* __restrict__ g_out, uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ scales, int blk) {
  // the block's loads are issued before the scale reduction so that their
  // latency overlaps it
  const int64_t b = blk * 256ll + threadIdx.x;
  float v[16];
  load16<DT>(x, (b < nblocks ? b : 0) * 16, v);
  const float g = reduce_scale(g_in, partial, nparts);
  if (b == 0 && g_out) *g_out = g;
  if (b >= nblocks) return;
  uint32_t lo, hi;
  const uint32_t s = encode_block16(v, g, lo, hi);
  reinterpret_cast<uint2*>(codes)[b] = make_uint2(lo, hi);
  scales[b] = static_cast<uint8_t>(s);
}

template <int DT>
__global__ __launch_bounds__(256) void k_quantize(const void* __restrict__ x, int64_t nblocks,
                                                  const float* __restrict__ g_in,
                                                  const float* __restrict__ partial, int nparts,
                                                  float* __restrict__ g_out, uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  quantize_body<DT>(x, nblocks, g_in, partial, nparts, g_out, codes, scales, blockIdx.x);
}


}  // namespace nvfp4
