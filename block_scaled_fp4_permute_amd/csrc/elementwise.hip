// NVFP4 quantisation, the unfused SwiGLU + re-quantisation, and the unfused
// weighted combine.  All three are HBM-bound streaming kernels: one thread per
// 16-element block (quantise, SwiGLU) or per 8 output columns (combine), with
// 16-byte vector loads and stores.
#include "quantize_impl.h"

namespace nvfp4 {

hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t cols, const float* g_in, float* g_out,
                           uint8_t* codes, uint8_t* scales, void* ws, hipStream_t stream) {
  const int64_t nblocks = rows * (cols / 16);
  float* partial = static_cast<float*>(ws);
  const int nparts = g_in ? 0 : amax_grid(nblocks);
  if (!g_in) {
    if (dtype == 1)
      hipLaunchKernelGGL(k_amax_blocks<1>, dim3(nparts), dim3(256), 0, stream, x, nblocks, partial);
    else
      hipLaunchKernelGGL(k_amax_blocks<0>, dim3(nparts), dim3(256), 0, stream, x, nblocks, partial);
  }
  const dim3 grid(static_cast<unsigned>((nblocks + 255) / 256 > 0 ? (nblocks + 255) / 256 : 1));
  if (dtype == 1)
    hipLaunchKernelGGL(k_quantize<1>, grid, dim3(256), 0, stream, x, nblocks, g_in, partial, nparts, g_out, codes,
                       scales);
  else
    hipLaunchKernelGGL(k_quantize<0>, grid, dim3(256), 0, stream, x, nblocks, g_in, partial, nparts, g_out, codes,
                       scales);
  return hipGetLastError();
}

// ------------------------------------------------------------------ SwiGLU
// h block b of row r covers h columns [16c, 16c+16) with c = b % (I/16): gate
// columns are the same indices, up columns are I further.
template <int DT>
__device__ __forceinline__ void swiglu_block(const void* y, int64_t b, int I, float (&h)[16]) {
  const int bpr = I / 16;
  const int64_t r = b / bpr;
  const int c = static_cast<int>(b % bpr);
  const size_t g0 = static_cast<size_t>(r) * (2 * static_cast<size_t>(I)) + 16 * static_cast<size_t>(c);
  float gv[16], uv[16];
  load16<DT>(y, g0, gv);
  load16<DT>(y, g0 + I, uv);
#pragma unroll
  for (int i = 0; i < 16; ++i) h[i] = silu_f32(gv[i]) * uv[i];
}

template <int DT>
__global__ __launch_bounds__(256) void k_swiglu_amax(const void* __restrict__ y, int64_t nblocks, int I,
                                                     float* __restrict__ partial) {
  float m = 0.0f;
  for (int64_t b = blockIdx.x * 256ll + threadIdx.x; b < nblocks; b += static_cast<int64_t>(gridDim.x) * 256) {
    float h[16];
    swiglu_block<DT>(y, b, I, h);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(h[i]));
  }
  block_max_store(m, partial, blockIdx.x);
}

template <int DT>
__global__ __launch_bounds__(256) void k_swiglu_quant(const void* __restrict__ y, int64_t nblocks, int I,
                                                      const float* __restrict__ g_in,
                                                      const float* __restrict__ partial, int nparts,
                                                      float* __restrict__ g_out, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int64_t b = blockIdx.x * 256ll + threadIdx.x;
  float h[16];
  swiglu_block<DT>(y, b < nblocks ? b : 0, I, h);
  const float g = reduce_scale(g_in, partial, nparts);
  if (b == 0 && g_out) *g_out = g;
  if (b >= nblocks) return;
  uint32_t lo, hi;
  const uint32_t s = encode_block16(h, g, lo, hi);
  reinterpret_cast<uint2*>(codes)[b] = make_uint2(lo, hi);
  scales[b] = static_cast<uint8_t>(s);
}

hipError_t launch_swiglu(const void* y, int dtype, int64_t M, int I, const float* g_in, float* g_out,
                         uint8_t* codes, uint8_t* scales, void* ws, hipStream_t stream) {
  const int64_t nblocks = M * (I / 16);
  float* partial = static_cast<float*>(ws);
  const int nparts = g_in ? 0 : amax_grid(nblocks);
  if (!g_in) {
    if (dtype == 1)
      hipLaunchKernelGGL(k_swiglu_amax<1>, dim3(nparts), dim3(256), 0, stream, y, nblocks, I, partial);
    else
      hipLaunchKernelGGL(k_swiglu_amax<0>, dim3(nparts), dim3(256), 0, stream, y, nblocks, I, partial);
  }
  const dim3 grid(static_cast<unsigned>((nblocks + 255) / 256 > 0 ? (nblocks + 255) / 256 : 1));
  if (dtype == 1)
    hipLaunchKernelGGL(k_swiglu_quant<1>, grid, dim3(256), 0, stream, y, nblocks, I, g_in, partial, nparts, g_out,
                       codes, scales);
  else
    hipLaunchKernelGGL(k_swiglu_quant<0>, grid, dim3(256), 0, stream, y, nblocks, I, g_in, partial, nparts, g_out,
                       codes, scales);
  return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// out[t, 8c .. 8c+8) = sum_j w[t, j] * y[row(t, j), 8c .. 8c+8), summed in
// order j = 0, 1, ...  The k rows of a token are fetched in batches of 8
// independent loads (rows past k re-read the last one and are not added), so
// a thread waits for one round trip per batch instead of one per row.
// Each row is read once, so the loads are non-temporal: at T=2048 top-8 this
// cut down + combine from 152 to 149 us, and at T=16384 from 947 to 884 us.
typedef unsigned int u32x4c __attribute__((ext_vector_type(4)));
typedef float f32x4c __attribute__((ext_vector_type(4)));
template <int YT>
__device__ __forceinline__ void load_row8(const void* y, int64_t row, int H, int c, float (&v)[8]) {
  if constexpr (YT == 1) {
    const u32x4c q =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4c*>(static_cast<const uint16_t*>(y) + row * H) + c);
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v[2 * m] = __uint_as_float(u[m] << 16);
      v[2 * m + 1] = __uint_as_float(u[m] & 0xFFFF0000u);
    }
  } else {
    const f32x4c* p = reinterpret_cast<const f32x4c*>(static_cast<const float*>(y) + row * H) + 2 * c;
    const f32x4c a0 = __builtin_nontemporal_load(p), a1 = __builtin_nontemporal_load(p + 1);
    v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
    v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
  }
}

template <int YT, int OT>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y, const int* __restrict__ perm,
                                                 const float* __restrict__ w, int T, int k, int H,
                                                 void* __restrict__ out) {
  constexpr int B = 8;
  const int groups = H / 8;
  const int64_t i = blockIdx.x * 256ll + threadIdx.x;
  if (i >= static_cast<int64_t>(T) * groups) return;
  const int t = static_cast<int>(i / groups);
  const int c = static_cast<int>(i % groups);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j0 = 0; j0 < k; j0 += B) {
    int64_t rows[B];
    float wt[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int64_t a = static_cast<int64_t>(t) * k + min(j0 + u, k - 1);
      rows[u] = perm ? perm[a] : a;
      wt[u] = w ? w[a] : 1.0f;
    }
    float v[B][8];
#pragma unroll
    for (int u = 0; u < B; ++u) load_row8<YT>(y, rows[u], H, c, v[u]);
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (j0 + u < k)
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m] = fmaf(wt[u], v[u][m], acc[m]);
  }
  if constexpr (OT == 1) {
    uint4 q;
    q.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    q.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    q.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
    q.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
    reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + static_cast<int64_t>(t) * H)[c] = q;
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + static_cast<int64_t>(t) * H) + 2 * c;
    p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

hipError_t launch_combine(const void* y, int y_dtype, const int* perm, const float* w, int T, int k, int H,
                          void* out, int out_dtype, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(T) * (H / 8);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (y_dtype == 1 && out_dtype == 1)
    hipLaunchKernelGGL((k_combine<1, 1>), grid, dim3(256), 0, stream, y, perm, w, T, k, H, out);
  else if (y_dtype == 1)
    hipLaunchKernelGGL((k_combine<1, 0>), grid, dim3(256), 0, stream, y, perm, w, T, k, H, out);
  else if (out_dtype == 1)
    hipLaunchKernelGGL((k_combine<0, 1>), grid, dim3(256), 0, stream, y, perm, w, T, k, H, out);
  else
    hipLaunchKernelGGL((k_combine<0, 0>), grid, dim3(256), 0, stream, y, perm, w, T, k, H, out);
  return hipGetLastError();
}

}  // namespace nvfp4
