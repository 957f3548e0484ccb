// FP8 block-scaled variant for gfx950: E4M3 operands with float32 scales per
// 128-value block along K (one per row for activations, one per 128 x 128
// tile for weights) - the FP8 grouped GEMM the pages name next to the FP4
// ones ("From Empirical Limits to Research-Driven Optimization", section
// "Sections 2-4: Framework and Community Landscape"), with the blockwise
// scaling of the FP8 collective they search for ("The Critical Search:
// Uncovering SM120 CUTLASS Collective Implementations", section "Output
// Knowledge Created").
//
//   fp8_quantize  s = absmax_block / 448 (1 for a zero block), q = E4M3
//                 nearest-even of |x| / s (correctly rounded float32 quotient),
//                 saturating, sign copied
//   fp8 gemm      per 128-value K step, one v_mfma_scale_f32_16x16x128_f8f6f4
//                 (E4M3 operands, unit E8M0 scales) per 16 x 16 tile gives the
//                 block's partial sum, and the float32 block scales enter as
//                 acc += partial * (sa[row] * sb[tile]) (four FMAs a lane)
//
// Operand mapping: a K step is 128 values; lane l = 16 g + r holds values
// [32 g, 32 g + 32) of its row (8 dwords), the layout of the 16x16x128 FP8
// instruction.  Weights are read from packed tiles (fp8_weight_repack): tile
// (e, 16-row tile rt, step st) is 2048 bytes, lane l's first 16 bytes at
// [16 l, 16 l + 16) and the next 16 at [1024 + 16 l, +16).
#include "gemm_device.h"

namespace nvfp4 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kFp8Block = 128;
constexpr int kFp8Tile = 2048;
constexpr int kFp8FmtE4M3 = 0;         // operand format code of E4M3 in the scaled MFMA
constexpr int kE8M0One = 127;          // E8M0 code of 2^0

__device__ __forceinline__ uint32_t fp8_encode(float x, float s) {
  const float v = fabsf(x) / s;                       // correctly rounded float32 quotient
  return f32_to_e4m3_sat(v) | (__float_as_uint(x) >> 31 << 7);
}

// ------------------------------------------------------------------ quantise, 1 x 128 blocks
// 16 lanes per block, 8 values a lane (one 16-byte load of bf16, two of
// float32, and one 8-byte store of codes); 4 blocks per wave, 16 per
// workgroup.  The 16 lanes of a block are aligned in the wave, so the
// reduction's lane exchanges (xor 8, 4, 2, 1) stay inside the block and a
// block past the end leaves as a whole.
constexpr int kFp8RowLanes = 16;
constexpr int kFp8RowBlocksPerGroup = 256 / kFp8RowLanes;

template <int DT>
__global__ __launch_bounds__(256) void k_fp8_quant_rows(const void* __restrict__ x, int64_t nblocks,
                                                        uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int64_t b = blockIdx.x * static_cast<int64_t>(kFp8RowBlocksPerGroup) + (threadIdx.x / kFp8RowLanes);
  const int q = threadIdx.x % kFp8RowLanes;
  if (b >= nblocks) return;
  float v[8];
  if constexpr (DT == 1) {
    const uint4 w = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + b * kFp8Block)[q];
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + b * kFp8Block) + 2 * q;
    const float4 w0 = p[0], w1 = p[1];
    v[0] = w0.x; v[1] = w0.y; v[2] = w0.z; v[3] = w0.w;
    v[4] = w1.x; v[5] = w1.y; v[6] = w1.z; v[7] = w1.w;
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
  for (int d = kFp8RowLanes / 2; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
  const float s = m > 0.0f ? m / 448.0f : 1.0f;
  uint32_t c[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    c[h] = fp8_encode(v[4 * h], s) | (fp8_encode(v[4 * h + 1], s) << 8) | (fp8_encode(v[4 * h + 2], s) << 16) |
           (fp8_encode(v[4 * h + 3], s) << 24);
  reinterpret_cast<uint2*>(codes + b * kFp8Block)[q] = make_uint2(c[0], c[1]);
  if (q == 0) scales[b] = s;
}

// ------------------------------------------------------------------ quantise, 128 x 128 blocks
// One workgroup per block of matrix blockIdx.z: thread t takes row t / 2 of
// the block, 64 values (half t % 2); rows past the matrix count as zeros.
template <int DT>
__global__ __launch_bounds__(256) void k_fp8_quant_tiles(const void* __restrict__ x_all, int64_t rows, int64_t cols,
                                                         uint8_t* __restrict__ codes_all,
                                                         float* __restrict__ scales_all) {
  __shared__ float s_max[4];
  const int64_t rb = blockIdx.y, cb = blockIdx.x, z = blockIdx.z;
  const int64_t nrb = gridDim.y;
  const void* x = static_cast<const uint8_t*>(x_all) + z * rows * cols * (DT == 1 ? 2 : 4);
  uint8_t* codes = codes_all + z * rows * cols;
  float* scales = scales_all + z * nrb * (cols / kFp8Block);
  const int t = threadIdx.x;
  const int64_t r = rb * kFp8Block + (t >> 1);
  const int64_t c0 = cb * kFp8Block + 64 * (t & 1);
  const bool row_ok = r < rows;
  float v[64];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    if constexpr (DT == 1) {
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok) w = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + r * cols + c0)[q];
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = __uint_as_float(u[i] << 16);
        v[8 * q + 2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row_ok) w = reinterpret_cast<const float4*>(static_cast<const float*>(x) + r * cols + c0)[2 * q + h];
        v[8 * q + 4 * h] = w.x; v[8 * q + 4 * h + 1] = w.y; v[8 * q + 4 * h + 2] = w.z; v[8 * q + 4 * h + 3] = w.w;
      }
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
  if ((t & 63) == 0) s_max[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float s = m > 0.0f ? m / 448.0f : 1.0f;
  if (t == 0) scales[rb * (cols / kFp8Block) + cb] = s;
  if (!row_ok) return;
  uint4* dst = reinterpret_cast<uint4*>(codes + r * cols + c0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 16 * q + 4 * i;
      w[i] = fp8_encode(v[e], s) | (fp8_encode(v[e + 1], s) << 8) | (fp8_encode(v[e + 2], s) << 16) |
             (fp8_encode(v[e + 3], s) << 24);
    }
    dst[q] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_fp8_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols, int block_rows,
                               uint8_t* codes, float* scales, hipStream_t stream) {
  if (block_rows == 1) {
    const int64_t nb = batch * rows * (cols / kFp8Block);
    const dim3 grid(static_cast<unsigned>((nb + kFp8RowBlocksPerGroup - 1) / kFp8RowBlocksPerGroup));
    if (dtype == 1)
      hipLaunchKernelGGL(k_fp8_quant_rows<1>, grid, dim3(256), 0, stream, x, nb, codes, scales);
    else
      hipLaunchKernelGGL(k_fp8_quant_rows<0>, grid, dim3(256), 0, stream, x, nb, codes, scales);
  } else {
    const dim3 grid(static_cast<unsigned>(cols / kFp8Block), static_cast<unsigned>((rows + kFp8Block - 1) / kFp8Block),
                    static_cast<unsigned>(batch));
    if (dtype == 1)
      hipLaunchKernelGGL(k_fp8_quant_tiles<1>, grid, dim3(256), 0, stream, x, rows, cols, codes, scales);
    else
      hipLaunchKernelGGL(k_fp8_quant_tiles<0>, grid, dim3(256), 0, stream, x, rows, cols, codes, scales);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ SwiGLU + quantise
// h = silu(gate) * up of the gate_up output y [M, 2I] (gate = columns [0, I),
// up = [I, 2I)), in float32, quantised like fp8_quantize with 1 x 128 blocks:
// 16 lanes per (row, 128 columns of h), eight values a lane, as the activation
// quantiser.  y need only be 8-byte and codes 2-byte aligned, so the lane's
// loads are 8 bytes wide and its codes leave as four 2-byte stores.
template <int DT>
__global__ __launch_bounds__(256) void k_fp8_swiglu_quant(const void* __restrict__ y, int64_t M, int I,
                                                          uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int nbr = I / kFp8Block;                  // blocks per row
  const int64_t b = blockIdx.x * static_cast<int64_t>(kFp8RowBlocksPerGroup) + (threadIdx.x / kFp8RowLanes);
  const int q = threadIdx.x % kFp8RowLanes;
  if (b >= M * nbr) return;
  const int64_t row = b / nbr;
  const int c = static_cast<int>(b % nbr) * kFp8Block + 8 * q;
  float g[8], u[8];
  if constexpr (DT == 1) {
    const uint16_t* yr = static_cast<const uint16_t*>(y) + row * 2 * I;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint2 wg = *reinterpret_cast<const uint2*>(yr + c + 4 * h);
      const uint2 wu = *reinterpret_cast<const uint2*>(yr + I + c + 4 * h);
      g[4 * h + 0] = __uint_as_float(wg.x << 16); g[4 * h + 1] = __uint_as_float(wg.x & 0xFFFF0000u);
      g[4 * h + 2] = __uint_as_float(wg.y << 16); g[4 * h + 3] = __uint_as_float(wg.y & 0xFFFF0000u);
      u[4 * h + 0] = __uint_as_float(wu.x << 16); u[4 * h + 1] = __uint_as_float(wu.x & 0xFFFF0000u);
      u[4 * h + 2] = __uint_as_float(wu.y << 16); u[4 * h + 3] = __uint_as_float(wu.y & 0xFFFF0000u);
    }
  } else {
    const float* yr = static_cast<const float*>(y) + row * 2 * I;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float2 wg = *reinterpret_cast<const float2*>(yr + c + 2 * h);
      const float2 wu = *reinterpret_cast<const float2*>(yr + I + c + 2 * h);
      g[2 * h] = wg.x; g[2 * h + 1] = wg.y;
      u[2 * h] = wu.x; u[2 * h + 1] = wu.y;
    }
  }
  float hv[8];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hv[i] = silu_f32(g[i]) * u[i];
    m = fmaxf(m, fabsf(hv[i]));
  }
#pragma unroll
  for (int d = kFp8RowLanes / 2; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
  const float s = m > 0.0f ? m / 448.0f : 1.0f;
  uint16_t* dst = reinterpret_cast<uint16_t*>(codes + row * I + c);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dst[i] = static_cast<uint16_t>(fp8_encode(hv[2 * i], s) | (fp8_encode(hv[2 * i + 1], s) << 8));
  if (q == 0) scales[b] = s;
}

hipError_t launch_fp8_swiglu(const void* y, int dtype, int64_t M, int I, uint8_t* codes, float* scales,
                             hipStream_t stream) {
  const int64_t nb = M * (I / kFp8Block);
  const dim3 grid(static_cast<unsigned>((nb + kFp8RowBlocksPerGroup - 1) / kFp8RowBlocksPerGroup));
  if (dtype == 1)
    hipLaunchKernelGGL(k_fp8_swiglu_quant<1>, grid, dim3(256), 0, stream, y, M, I, codes, scales);
  else
    hipLaunchKernelGGL(k_fp8_swiglu_quant<0>, grid, dim3(256), 0, stream, y, M, I, codes, scales);
  return hipGetLastError();
}

// ------------------------------------------------------------------ packed weights
size_t fp8_packed_weight_bytes(int E, int N, int K) {
  return static_cast<size_t>(E) * ((int64_t(N) + 15) / 16) * ((int64_t(K) + kFp8Block - 1) / kFp8Block) * kFp8Tile;
}

__global__ __launch_bounds__(256) void k_fp8_repack(const uint8_t* __restrict__ codes, int E, int N, int K,
                                                    uint8_t* __restrict__ packed, int64_t total_tiles) {
  const int64_t t = blockIdx.x * 256ll + threadIdx.x;
  const int64_t tile = t >> 6;
  const int lane = static_cast<int>(t & 63);
  if (tile >= total_tiles) return;
  const int nst = (K + kFp8Block - 1) / kFp8Block;
  const int ntr = (N + 15) / 16;
  const int st = static_cast<int>(tile % nst);
  const int rt = static_cast<int>((tile / nst) % ntr);
  const int e = static_cast<int>(tile / (static_cast<int64_t>(nst) * ntr));
  const int n = 16 * rt + (lane & 15);
  const int g = lane >> 4;
  uint8_t* dst = packed + tile * kFp8Tile;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = kFp8Block * st + 32 * g + 16 * h;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < N && k < K) v = *reinterpret_cast<const u32x4*>(codes + (static_cast<size_t>(e) * N + n) * K + k);
    *reinterpret_cast<u32x4*>(dst + 1024 * h + 16 * lane) = v;
  }
}

hipError_t launch_fp8_repack(const uint8_t* codes, int E, int N, int K, uint8_t* packed, hipStream_t stream) {
  const int64_t tiles = static_cast<int64_t>(E) * ((N + 15) / 16) * ((K + kFp8Block - 1) / kFp8Block);
  hipLaunchKernelGGL(k_fp8_repack, dim3(static_cast<unsigned>((tiles * 64 + 255) / 256)), dim3(256), 0, stream, codes,
                     E, N, K, packed, tiles);
  return hipGetLastError();
}

// ------------------------------------------------------------------ GEMM

constexpr int kFp8RowLds = 144;     // A row pitch in LDS: 128 code bytes + 16 of padding

// A staging: thread t stages (row t / 4, quarter t % 4: 32 code bytes) of the
// chunk's 64 rows for one step, and threads t < 64 the row's block scale;
// rows that do not exist stage zero codes.
struct Fp8AStage {
  rsrc_t rc, rs;
  uint32_t vc, vs;
  bool row_ok;
  int q;
};

__device__ __forceinline__ void fp8a_setup(const Fp8Params& p, int row0, int m0, int rows, Fp8AStage& S) {
  const int t = threadIdx.x;
  const uint32_t krow = static_cast<uint32_t>(p.K), srow = static_cast<uint32_t>(p.K / kFp8Block);
  S.rc = make_rsrc(p.a_codes, static_cast<uint32_t>(p.a_rows_total) * krow);
  S.rs = make_rsrc(p.a_scales, static_cast<uint32_t>(p.a_rows_total) * srow * 4u);
  const int ar = t >> 2;
  S.q = t & 3;
  S.row_ok = ar < rows;
  int arow = row0 + m0 + (S.row_ok ? ar : 0);
  if (p.a_rows) arow = p.a_rows[arow];
  arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
  S.vc = static_cast<uint32_t>(arow) * krow + 32u * S.q;
  const int sr = t & 63;       // every thread stages a scale: t, t + 64, ... the same row's
  int srow_i = row0 + m0 + (sr < rows ? sr : 0);
  if (p.a_rows) srow_i = p.a_rows[srow_i];
  srow_i = (srow_i >= 0 && srow_i < p.a_rows_total) ? srow_i : 0;
  S.vs = static_cast<uint32_t>(srow_i) * srow * 4u;
}

struct Fp8ARegs {
  u32x4 c[2];
  float s;
};

__device__ __forceinline__ void fp8a_load(const Fp8AStage& S, Fp8ARegs& R, int st, int nsteps) {
  const int s = min(st, nsteps - 1);
  const uint32_t oc = static_cast<uint32_t>(s) * kFp8Block;
  R.c[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(S.rc, S.vc + oc, 0, 0));
  R.c[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(S.rc, S.vc + oc + 16u, 0, 0));
  R.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(S.rs, S.vs + 4u * s, 0, 0));
}

// rows that do not exist, and steps past the last, stage zero codes
__device__ __forceinline__ void fp8a_store(const Fp8AStage& S, const Fp8ARegs& R, bool step_ok, int rows,
                                           uint8_t* __restrict__ lds) {
  const int t = threadIdx.x;
  const u32x4 z = {0u, 0u, 0u, 0u};
  const bool ok = S.row_ok && step_ok;
  u32x4* dst = reinterpret_cast<u32x4*>(lds + (t >> 2) * kFp8RowLds + 32 * S.q);
  dst[0] = ok ? R.c[0] : z;
  dst[1] = ok ? R.c[1] : z;
  reinterpret_cast<float*>(lds + 64 * kFp8RowLds)[t & 63] = ((t & 63) < rows) ? R.s : 0.0f;
}
constexpr int kFp8ALds = 64 * kFp8RowLds + 64 * 4;

struct Fp8B {
  u32x4 c[2];
};

template <int WN, bool NT>
__device__ __forceinline__ void fp8b_load(const uint8_t* const (&tiles)[WN], Fp8B (&B)[WN], int st, int nsteps) {
  const int lane = threadIdx.x & 63;
  const size_t o = static_cast<size_t>(min(st, nsteps - 1)) * kFp8Tile;
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const u32x4* p0 = reinterpret_cast<const u32x4*>(tiles[j] + o + 16 * lane);
    const u32x4* p1 = reinterpret_cast<const u32x4*>(tiles[j] + o + 1024 + 16 * lane);
    if constexpr (NT) {
      B[j].c[0] = __builtin_nontemporal_load(p0);
      B[j].c[1] = __builtin_nontemporal_load(p1);
    } else {
      B[j].c[0] = *p0;
      B[j].c[1] = *p1;
    }
  }
}

__device__ __forceinline__ i32x8 fp8_frag(const u32x4& lo, const u32x4& hi) {
  i32x8 r = {static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
             static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
  return r;
}

// one K step: per (row tile, column tile) the block's partial sum, scaled
// into the accumulator by the row's block scale and the wave's weight block
// scale (a wave's 64 columns lie in one 128-row weight block).  SW (the
// SwiGLU arrangement): the wave's gate tiles (the first WN / 2) and its up
// tiles lie in two weight blocks, scales sb and sbu.
template <int MTA, int WN, bool SW = false>
__device__ __forceinline__ void fp8_step(const uint8_t* __restrict__ a_lds, const Fp8B (&B)[WN], float sb,
                                         float sbu, float4v (&acc)[4][WN]) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int r = 0; r < MTA; ++r) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a_lds + (16 * r + lr) * kFp8RowLds + 32 * g);
    const i32x8 af = fp8_frag(src[0], src[1]);
    const float4v sa = *reinterpret_cast<const float4v*>(a_lds + 64 * kFp8RowLds + 4 * (16 * r + 4 * g));
    float4v part[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const float4v z = {0.f, 0.f, 0.f, 0.f};
      part[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, fp8_frag(B[j].c[0], B[j].c[1]), z, kFp8FmtE4M3,
                                                                 kFp8FmtE4M3, 0, kE8M0One, 0, kE8M0One);
    }
    const float4v sab = sa * sb;
    float4v sabu = sab;
    if constexpr (SW) sabu = sa * sbu;
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[r][j][i] = __builtin_fmaf(part[j][i], (SW && j >= WN / 2) ? sabu[i] : sab[i], acc[r][j][i]);
  }
}

// Two steps per iteration, branch free: A for step s + 1 goes to the other
// LDS buffer while step s runs; steps past the last read the last step's
// weights against zero activation codes (nothing added).
template <int MTA, int WN, bool NT, bool SW = false>
__device__ __forceinline__ void fp8_loop(const Fp8AStage& AS, const uint8_t* const (&tiles)[WN],
                                         const float* __restrict__ bsc, const float* __restrict__ bscu, int nsteps,
                                         int rows, uint8_t* __restrict__ lds0, uint8_t* __restrict__ lds1,
                                         float4v (&acc)[4][WN]) {
  Fp8B B0[WN], B1[WN];
  Fp8ARegs ra;
  fp8a_load(AS, ra, 0, nsteps);
  fp8b_load<WN, NT>(tiles, B0, 0, nsteps);
  float s0 = bsc[0], u0 = SW ? bscu[0] : 0.0f;
  fp8b_load<WN, NT>(tiles, B1, 1, nsteps);
  float s1 = bsc[min(1, nsteps - 1)], u1 = SW ? bscu[min(1, nsteps - 1)] : 0.0f;
  fp8a_store(AS, ra, true, rows, lds0);
  fp8a_load(AS, ra, 1, nsteps);
  __syncthreads();
  for (int st = 0; st < nsteps; st += 2) {
    fp8_step<MTA, WN, SW>(lds0, B0, s0, u0, acc);
    fp8a_store(AS, ra, st + 1 < nsteps, rows, lds1);
    fp8a_load(AS, ra, st + 2, nsteps);
    fp8b_load<WN, NT>(tiles, B0, st + 2, nsteps);
    s0 = bsc[min(st + 2, nsteps - 1)];
    if constexpr (SW) u0 = bscu[min(st + 2, nsteps - 1)];
    __syncthreads();
    fp8_step<MTA, WN, SW>(lds1, B1, s1, u1, acc);
    fp8a_store(AS, ra, st + 2 < nsteps, rows, lds0);
    fp8a_load(AS, ra, st + 3, nsteps);
    fp8b_load<WN, NT>(tiles, B1, st + 3, nsteps);
    s1 = bsc[min(st + 3, nsteps - 1)];
    if constexpr (SW) u1 = bscu[min(st + 3, nsteps - 1)];
    __syncthreads();
  }
}

template <int EPI>
__device__ __forceinline__ void fp8_store_tile(const Fp8Params& p, const float4v& acc, int prow0, int rows_left,
                                               int col, bool col_ok) {
  const int lg = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * lg + i;
    if (m >= rows_left || !col_ok) continue;
    const size_t o = static_cast<size_t>(prow0 + m) * p.N + col;
    if constexpr (EPI == EPI_F32)
      static_cast<float*>(p.out)[o] = acc[i];
    else
      static_cast<uint16_t*>(p.out)[o] = f32_to_bf16(acc[i]);
  }
}

// SwiGLU epilogue: a task's 128 h columns are one 1 x 128 block of every row.
// Wave w holds gate tiles 0, 1 and up tiles 2, 3 of h columns [32 w, +32):
// h = silu(gate) * up in float32, the row's maximum |h| over its 32 columns
// (lanes of one 16-lane row group), then over the four waves through LDS;
// scale amax / 448 (1 for an all-zero block) and E4M3 codes of h / scale,
// as the separate SwiGLU kernel computes them from the float32 rows.
__device__ __forceinline__ void fp8_swiglu_epilogue(const Fp8Params& p, const float4v (&acc)[4][4], int mt_active,
                                                    int rows, int prow0, int nt, float* __restrict__ s_amax) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int wave = threadIdx.x >> 6;
  const int I = p.N / 2;
  const int nbr = I / kFp8Block;
  const int hc0 = nt * kFp8Block + 32 * wave;
  float h[4][2][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r >= mt_active) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[r][0][i] = silu_f32(acc[r][0][i]) * acc[r][2][i];
      h[r][1][i] = silu_f32(acc[r][1][i]) * acc[r][3][i];
      float m = fmaxf(fabsf(h[r][0][i]), fabsf(h[r][1][i]));
#pragma unroll
      for (int d = 8; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
      if (lr == 0) s_amax[64 * wave + 16 * r + 4 * lg + i] = m;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r >= mt_active) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * r + 4 * lg + i;
      const float m = fmaxf(fmaxf(s_amax[row], s_amax[64 + row]), fmaxf(s_amax[128 + row], s_amax[192 + row]));
      const float s = m > 0.0f ? m / 448.0f : 1.0f;
      if (row < rows) {
        uint8_t* crow = p.out_codes + static_cast<size_t>(prow0 + row) * I + hc0 + lr;
        crow[0] = static_cast<uint8_t>(fp8_encode(h[r][0][i], s));
        crow[16] = static_cast<uint8_t>(fp8_encode(h[r][1][i], s));
        if (wave == 0 && lr == 0) p.out_scales[static_cast<size_t>(prow0 + row) * nbr + nt] = s;
      }
    }
  }
}

// the task map's view of the FP8 problem (offsets, experts, rows, tiles)
__device__ __forceinline__ GemmParams fp8_map_params(const Fp8Params& p, int n_tiles) {
  GemmParams g{};
  g.offsets = p.offsets;
  g.E = p.E;
  g.N = p.N;
  g.K = p.K;
  g.m_total = p.m_total;
  g.n_tiles = n_tiles;
  g.slots = 1 << 30;
  return g;
}

template <int EPI, bool NT>
__global__ __launch_bounds__(256, 2) void k_fp8_gemm(const Fp8Params p, int n_tiles) {
  constexpr int WN = 4, BN = 4 * WN * 16;
  constexpr bool SW = EPI == EPI_SWIGLU;
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][kFp8ALds];
  __shared__ float s_amax[SW ? 4 * 64 : 1];
  static_assert(fits_lds(sizeof(a_lds) + sizeof(s_amax), 2), "FP8 A staging exceeds the LDS of two workgroups per CU");
  int e, m0, nt;
  bool narrow;
  const GemmParams map = fp8_map_params(p, n_tiles);
  if (!find_task<4, true, 0>(map, e, m0, nt, narrow)) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = threadIdx.x & 15;
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  const int rows = min(64, Me - m0);
  const int mt_active = (rows + 15) >> 4;
  const int N = p.N, K = p.K;
  const int nsteps = K / kFp8Block;
  const int ntr = (N + 15) / 16;
  const int nsb = (N + kFp8Block - 1) / kFp8Block;
  Fp8AStage AS;
  fp8a_setup(p, row0, m0, rows, AS);
  const uint8_t* tiles[WN];
  int col0[WN];
  bool cok[WN];
  // plain: the wave's 64 columns from wcol; SwiGLU: gate columns [wcol, +32)
  // and up columns I + [wcol, +32), wcol = 128 nt + 32 wave (I % 128 == 0)
  const int wcol = SW ? nt * kFp8Block + wave * 32 : nt * BN + wave * WN * 16;
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    col0[j] = SW ? (j < 2 ? wcol + 16 * j : N / 2 + wcol + 16 * (j - 2)) : wcol + j * 16;
    cok[j] = col0[j] + lr < N;
    const int rt = min(col0[j] / 16, ntr - 1);
    tiles[j] = p.b_packed + (static_cast<size_t>(e) * ntr + rt) * nsteps * kFp8Tile;
  }
  const float* bsc = p.b_scales + (static_cast<size_t>(e) * nsb + min(wcol, N - 1) / kFp8Block) * nsteps;
  const float* bscu = SW ? p.b_scales + (static_cast<size_t>(e) * nsb + min(N / 2 + wcol, N - 1) / kFp8Block) * nsteps
                         : bsc;
  float4v acc[4][WN];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[r][j] = float4v{0.f, 0.f, 0.f, 0.f};
  switch (mt_active) {
    case 1: fp8_loop<1, WN, NT, SW>(AS, tiles, bsc, bscu, nsteps, rows, a_lds[0], a_lds[1], acc); break;
    case 2: fp8_loop<2, WN, NT, SW>(AS, tiles, bsc, bscu, nsteps, rows, a_lds[0], a_lds[1], acc); break;
    case 3: fp8_loop<3, WN, NT, SW>(AS, tiles, bsc, bscu, nsteps, rows, a_lds[0], a_lds[1], acc); break;
    default: fp8_loop<4, WN, NT, SW>(AS, tiles, bsc, bscu, nsteps, rows, a_lds[0], a_lds[1], acc); break;
  }
  const int prow0 = row0 + m0;
  if constexpr (SW) {
    fp8_swiglu_epilogue(p, acc, mt_active, rows, prow0, nt, s_amax);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r >= mt_active) continue;
#pragma unroll
      for (int j = 0; j < WN; ++j)
        fp8_store_tile<EPI>(p, acc[r][j], prow0 + 16 * r, rows - 16 * r, col0[j] + lr, cok[j]);
    }
  }
}

// ---- stream-N (K <= 256: one or two 128-value steps; the down GEMM): the
// chunk's 64 rows (codes and block scales) are staged in LDS once, then each
// wave streams units of 64 columns (4 weight tiles per step), the next unit's
// loads in flight while one computes, and its rows leave through a per-wave
// LDS stage as whole 128-byte segments (16 bytes a lane).  A unit's 64
// columns lie in one 128-column weight block: one weight scale per unit and
// step.
constexpr int kFp8NUnit = 4;       // 16-column tiles per unit

template <int EPI>
__device__ __forceinline__ void fp8n_store(const Fp8Params& p, const float4v (&acc)[kFp8NUnit], float* __restrict__ stage,
                                           int prow0, int rows_left, int col0) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int u = 0; u < kFp8NUnit; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) stage[(4 * lg + i) * 68 + 16 * u + lr] = acc[u][i];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int r = lane >> 2;
  const int c = 16 * (lane & 3);
  if (r < rows_left && col0 + c < p.N) {
    const float* src = stage + r * 68 + c;
    const size_t base = static_cast<size_t>(prow0 + r) * p.N + col0 + c;
    if constexpr (EPI == EPI_F32) {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.out) + base);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = make_float4(src[4 * q], src[4 * q + 1], src[4 * q + 2], src[4 * q + 3]);
    } else {
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        w[q] = static_cast<uint32_t>(f32_to_bf16(src[2 * q])) | (static_cast<uint32_t>(f32_to_bf16(src[2 * q + 1])) << 16);
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + base);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The wave's work is a run of (unit, step) items, each the 4 weight tiles of
// one unit at one K step; a ring of three holds the next two items' loads in
// flight while one is multiplied.  A unit's accumulator leaves after its last
// step.
template <int MTA, int UPW, int EPI, bool NT>
__device__ __forceinline__ void fp8n_loop(const Fp8Params& p, const uint8_t* __restrict__ a_lds, float* stage,
                                          const uint8_t* tiles, const float* bsc, int u_first, int u_count, int ntr,
                                          int nsteps, int prow0, int rows) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, g = lane >> 4;
  const int n_items = u_count * nsteps;
  i32x8 R0[kFp8NUnit], R1[kFp8NUnit], R2[kFp8NUnit];
  auto load_item = [&](i32x8 (&R)[kFp8NUnit], int it) {
    const int c = min(it, n_items - 1);                  // loads past the run re-read the last item (cached)
    const int ui = u_first + c / nsteps, s = c % nsteps;
#pragma unroll
    for (int t = 0; t < kFp8NUnit; ++t) {
      const uint8_t* tp = tiles + (static_cast<size_t>(min(kFp8NUnit * ui + t, ntr - 1)) * nsteps + s) * kFp8Tile;
      const u32x4* p0 = reinterpret_cast<const u32x4*>(tp + 16 * lane);
      const u32x4* p1 = reinterpret_cast<const u32x4*>(tp + 1024 + 16 * lane);
      u32x4 lo, hi;
      if constexpr (NT) {
        lo = __builtin_nontemporal_load(p0);
        hi = __builtin_nontemporal_load(p1);
      } else {
        lo = *p0;
        hi = *p1;
      }
      R[t] = fp8_frag(lo, hi);
    }
  };
  float4v acc[MTA][kFp8NUnit];
#pragma unroll
  for (int r = 0; r < MTA; ++r)
#pragma unroll
    for (int t = 0; t < kFp8NUnit; ++t) acc[r][t] = float4v{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const i32x8 (&R)[kFp8NUnit], int it) {
    if (it >= n_items) return;                           // uniform
    const int ui = u_first + it / nsteps, s = it % nsteps;
    const float sb = bsc[(64 * ui) / kFp8Block * nsteps + s];
    const uint8_t* al = a_lds + s * kFp8ALds;
#pragma unroll
    for (int r = 0; r < MTA; ++r) {
      const u32x4* src = reinterpret_cast<const u32x4*>(al + (16 * r + lr) * kFp8RowLds + 32 * g);
      const i32x8 af = fp8_frag(src[0], src[1]);
      const float4v sa = *reinterpret_cast<const float4v*>(al + 64 * kFp8RowLds + 4 * (16 * r + 4 * g));
      const float4v sab = sa * sb;
#pragma unroll
      for (int t = 0; t < kFp8NUnit; ++t) {
        const float4v z = {0.f, 0.f, 0.f, 0.f};
        const float4v part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af, R[t], z, kFp8FmtE4M3, kFp8FmtE4M3, 0, kE8M0One, 0, kE8M0One);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[r][t][q] = __builtin_fmaf(part[q], sab[q], acc[r][t][q]);
      }
    }
    if (s == nsteps - 1) {
#pragma unroll
      for (int r = 0; r < MTA; ++r) {
        fp8n_store<EPI>(p, acc[r], stage, prow0 + 16 * r, rows - 16 * r, 64 * ui);
#pragma unroll
        for (int t = 0; t < kFp8NUnit; ++t) acc[r][t] = float4v{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  load_item(R0, 0);
  load_item(R1, 1);
  load_item(R2, 2);
  for (int it = 0; it < n_items; it += 3) {
    consume(R0, it);
    load_item(R0, it + 3);
    consume(R1, it + 1);
    load_item(R1, it + 4);
    consume(R2, it + 2);
    load_item(R2, it + 5);
  }
}

template <int UPW, int EPI, bool NT>
__global__ __launch_bounds__(256, 2) void k_fp8_gemm_n(const Fp8Params p, int n_groups) {
  constexpr int NW = 4;
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2 * kFp8ALds];
  __shared__ float stage_lds[NW * 16 * 68];
  static_assert(fits_lds(sizeof(a_lds) + sizeof(stage_lds), 2), "FP8 stream-N staging exceeds the LDS of two workgroups per CU");
  int e, m0, ng;
  bool narrow;
  const GemmParams map = fp8_map_params(p, n_groups);
  if (!find_task<4, false, 0>(map, e, m0, ng, narrow)) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  const int rows = min(64, Me - m0);
  const int mt_active = (rows + 15) >> 4;
  const int N = p.N, K = p.K;
  const int nsteps = K / kFp8Block;                    // 1 or 2
  const int ntr = (N + 15) / 16;
  const int nsb = (N + kFp8Block - 1) / kFp8Block;
  Fp8AStage AS;
  fp8a_setup(p, row0, m0, rows, AS);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    Fp8ARegs ra;
    fp8a_load(AS, ra, s, nsteps);
    fp8a_store(AS, ra, s < nsteps, rows, a_lds + s * kFp8ALds);
  }
  __syncthreads();
  const int nunits = (ntr + kFp8NUnit - 1) / kFp8NUnit;
  const int u_first = (ng * NW + wave) * UPW;
  const int u_count = min(UPW, nunits - u_first);
  if (u_count <= 0) return;
  const uint8_t* tiles = p.b_packed + static_cast<size_t>(e) * ntr * nsteps * kFp8Tile;
  const float* bsc = p.b_scales + static_cast<size_t>(e) * nsb * nsteps;
  const int prow0 = row0 + m0;
  float* stage = stage_lds + wave * (16 * 68);
  switch (mt_active) {
    case 1: fp8n_loop<1, UPW, EPI, NT>(p, a_lds, stage, tiles, bsc, u_first, u_count, ntr, nsteps, prow0, rows); break;
    case 2: fp8n_loop<2, UPW, EPI, NT>(p, a_lds, stage, tiles, bsc, u_first, u_count, ntr, nsteps, prow0, rows); break;
    case 3: fp8n_loop<3, UPW, EPI, NT>(p, a_lds, stage, tiles, bsc, u_first, u_count, ntr, nsteps, prow0, rows); break;
    default: fp8n_loop<4, UPW, EPI, NT>(p, a_lds, stage, tiles, bsc, u_first, u_count, ntr, nsteps, prow0, rows); break;
  }
}

// ---- large-M tile (from 256 rows per expert): 8 waves on 256 rows x 256
// columns, both operands of a 128-value K step staged in LDS once per
// workgroup; wave w = 4 wr + wc holds rows [128 wr, +128) and columns
// [64 wc, +64), which lie in one 128-column weight block.  One stage (65 KB,
// two double-buffered):
//   A codes   16 row tiles x 2048 bytes: half h of lane (g, r) at
//             1024 h + 256 g + 16 (r ^ (2 g + h)) (the XOR spreads the 8
//             lanes that store one row's 128 bytes over distinct banks)
//   A scales  256 floats (the rows' block scales of the step)
//   B codes   16 column tiles x 2048 bytes, as in the packed tile
// The weight block scale of a wave is one scalar per step, read from memory.
constexpr int kFp8LRows = 256;
constexpr int kFp8LThreads = 512;
constexpr int kFp8LASc = 16 * 2048;
constexpr int kFp8LB = kFp8LASc + kFp8LRows * 4;
constexpr int kFp8LStage = kFp8LB + 16 * 2048;

struct Fp8LRegs {
  u32x4 c[4];
  float s;
};

struct Fp8LSrc {
  rsrc_t ra, rs;
  uint32_t va[4];       // byte offsets of the thread's four A pieces at step 0
  uint32_t vs;          // of its row's scale at step 0 (row t % 256)
  uint32_t lda;         // LDS offset of its first A piece (the others 8 KB apart)
  const uint8_t* b;     // expert's packed tiles
  uint32_t ob[4];       // byte offsets of its four B pieces at step 0
};

__device__ __forceinline__ void fp8l_load_a(const Fp8LSrc& S, Fp8LRegs& R, int st) {
  const uint32_t oa = static_cast<uint32_t>(st) * kFp8Block;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    R.c[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(S.ra, S.va[i] + oa, 0, 0));
  R.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(S.rs, S.vs + 4u * st, 0, 0));
}

__device__ __forceinline__ void fp8l_load_b(const Fp8LSrc& S, Fp8LRegs& R, int st) {
  const uint32_t ot = static_cast<uint32_t>(st) * kFp8Tile;
#pragma unroll
  for (int i = 0; i < 4; ++i) R.c[i] = *reinterpret_cast<const u32x4*>(S.b + (S.ob[i] + ot));
}

__device__ __forceinline__ void fp8l_store_a(const Fp8LSrc& S, const Fp8LRegs& R, uint8_t* __restrict__ stage) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(stage + S.lda + 8192 * i) = R.c[i];
  if (threadIdx.x < kFp8LRows) reinterpret_cast<float*>(stage + kFp8LASc)[threadIdx.x] = R.s;
}

__device__ __forceinline__ void fp8l_store_b(const Fp8LRegs& R, uint8_t* __restrict__ stage) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<u32x4*>(stage + kFp8LB + 16 * (threadIdx.x + kFp8LThreads * i)) = R.c[i];
}

// row tiles [r0, r0 + 4) of the wave (H = r0 / 4): per 16 x 16 tile the
// block's partial sum, scaled into the accumulator by sa[row] * sb
template <int R0>
__device__ __forceinline__ void fp8l_rows(const uint8_t* __restrict__ stage, int wr, const i32x8 (&bf)[4], float sb,
                                          float4v (&acc)[8][4]) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int a0 = 256 * lg + 16 * (lr ^ (2 * lg)), a1 = 1024 + 256 * lg + 16 * (lr ^ (2 * lg + 1));
#pragma unroll
  for (int r = R0; r < R0 + 4; ++r) {
    const int rt = 8 * wr + r;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(stage + rt * 2048 + a0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(stage + rt * 2048 + a1);
    const i32x8 af = fp8_frag(lo, hi);
    const float4v sab = *reinterpret_cast<const float4v*>(stage + kFp8LASc + 4 * (16 * rt + 4 * lg)) * sb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4v z = {0.f, 0.f, 0.f, 0.f};
      const float4v part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], z, kFp8FmtE4M3, kFp8FmtE4M3,
                                                                            0, kE8M0One, 0, kE8M0One);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[r][j][i] = __builtin_fmaf(part[i], sab[i], acc[r][j][i]);
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(kFp8LThreads, 1) void k_fp8_gemm_l(const Fp8Params p, int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kFp8LStage];
  static_assert(fits_lds(sizeof(lds), 1), "FP8 large-M staging exceeds the LDS of a CU");
  int e, m0, nt;
  bool narrow;
  const GemmParams map = fp8_map_params(p, n_tiles);
  if (!find_task<16, false, 0>(map, e, m0, nt, narrow)) return;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = wave >> 2, wc = wave & 3;
  const int lr = lane & 15;
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  // inside an expert, groups of 4 row chunks run column tile by column tile
  // (the workgroups side by side on an XCD share A chunks and weight tiles)
  {
    const int nc = (Me + kFp8LRows - 1) / kFp8LRows;
    const int u = (m0 / kFp8LRows) * n_tiles + nt;
    const int grp = (m0 / kFp8LRows) / 4;
    const int gq = min(4, nc - 4 * grp);
    const int w = u - 4 * grp * n_tiles;
    m0 = (4 * grp + w % gq) * kFp8LRows;
    nt = w / gq;
  }
  const int rows = min(kFp8LRows, Me - m0);
  const int N = p.N, K = p.K;
  const int nsteps = K / kFp8Block;
  const int ntr = (N + 15) / 16;
  const int nsb = (N + kFp8Block - 1) / kFp8Block;

  Fp8LSrc S;
  {
    const uint32_t krow = static_cast<uint32_t>(K), srow = static_cast<uint32_t>(K / kFp8Block);
    S.ra = make_rsrc(p.a_codes, static_cast<uint32_t>(p.a_rows_total) * krow);
    S.rs = make_rsrc(p.a_scales, static_cast<uint32_t>(p.a_rows_total) * srow * 4u);
    const int q = t & 7;              // 16-byte piece of the row's 128 bytes: half q & 1 of lane group q >> 1
    const int g = q >> 1, h = q & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ar = (t >> 3) + 64 * i;
      int arow = row0 + m0 + (ar < rows ? ar : 0);
      if (p.a_rows) arow = p.a_rows[arow];
      arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
      S.va[i] = static_cast<uint32_t>(arow) * krow + 16u * q;
    }
    S.lda = ((t >> 3) >> 4) * 2048 + 1024 * h + 256 * g + 16 * (((t >> 3) & 15) ^ (2 * g + h));
    {
      const int ar = t & (kFp8LRows - 1);
      int arow = row0 + m0 + (ar < rows ? ar : 0);
      if (p.a_rows) arow = p.a_rows[arow];
      arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
      S.vs = static_cast<uint32_t>(arow) * srow * 4u;
    }
    S.b = p.b_packed + static_cast<size_t>(e) * ntr * nsteps * kFp8Tile;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = t + kFp8LThreads * i;    // 16-byte piece of the 16 x 2048 code bytes
      const uint32_t rt = static_cast<uint32_t>(min(nt * 16 + (pc >> 7), ntr - 1));
      S.ob[i] = rt * static_cast<uint32_t>(nsteps) * kFp8Tile + 16u * (pc & 127);
    }
  }
  const int wcol = nt * 256 + 64 * wc;
  const float* bsc = p.b_scales + (static_cast<size_t>(e) * nsb + min(wcol, N - 1) / kFp8Block) * nsteps;

  float4v acc[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[r][j] = float4v{0.f, 0.f, 0.f, 0.f};

  Fp8LRegs R;
  fp8l_load_a(S, R, 0);
  fp8l_store_a(S, R, lds);
  fp8l_load_b(S, R, 0);
  fp8l_store_b(R, lds);
  __syncthreads();
  // step st from stage st % 2; step st + 1's A pieces in flight behind the
  // first four row tiles, its B pieces behind the last four; the last step
  // re-stages itself into the idle stage (no branches)
  for (int st = 0; st < nsteps; ++st) {
    const uint8_t* cur = lds + (st & 1) * kFp8LStage;
    uint8_t* nxt = lds + ((st + 1) & 1) * kFp8LStage;
    const int sn = min(st + 1, nsteps - 1);
    const float sb = bsc[st];
    i32x8 bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* tb = cur + kFp8LB + (4 * wc + j) * 2048 + 16 * lane;
      bf[j] = fp8_frag(*reinterpret_cast<const u32x4*>(tb), *reinterpret_cast<const u32x4*>(tb + 1024));
    }
    fp8l_load_a(S, R, sn);
    fp8l_rows<0>(cur, wr, bf, sb, acc);
    fp8l_store_a(S, R, nxt);
    fp8l_load_b(S, R, sn);
    fp8l_rows<4>(cur, wr, bf, sb, acc);
    fp8l_store_b(R, nxt);
    __syncthreads();
  }

  const int prow0 = row0 + m0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int rt = 8 * wr + r;
    const int left = rows - 16 * rt;
    if (left <= 0) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wcol + 16 * j + lr;
      fp8_store_tile<EPI>(p, acc[r][j], prow0 + 16 * rt, left, col, col < N);
    }
  }
}

hipError_t launch_fp8_gemm(const Fp8Params& p, int epilogue, int64_t m_total, int hint, hipStream_t stream) {
  constexpr int BN = 256;
  const int n_tiles = (p.N + BN - 1) / BN;
  const int64_t blocks = ((((m_total + 63) / 64 + p.E) * n_tiles) + 7) / 8 * 8;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
  const int64_t rows_per_expert = hint > 0 ? hint : m_total / p.E;
  const bool nt = rows_per_expert < 64;
  if (epilogue == EPI_SWIGLU) {
    // SwiGLU + FP8 requant: the decode tile at any size, one task per 128 h
    // columns (a whole 1 x 128 block of h per row)
    const int sw_tiles = p.N / 2 / kFp8Block;
    const int64_t sblocks = ((((m_total + 63) / 64 + p.E) * sw_tiles) + 7) / 8 * 8;
    if (sblocks >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    const dim3 sgrid(static_cast<unsigned>(sblocks));
    if (nt) hipLaunchKernelGGL((k_fp8_gemm<EPI_SWIGLU, true>), sgrid, dim3(256), 0, stream, p, sw_tiles);
    else hipLaunchKernelGGL((k_fp8_gemm<EPI_SWIGLU, false>), sgrid, dim3(256), 0, stream, p, sw_tiles);
    return hipGetLastError();
  }
  if (p.K <= 2 * kFp8Block) {
    // one or two K steps (the down GEMM): the stream-N kernel at every size
    // (at 512 rows per expert, prefill down: 716 us against 754 on the large
    // tile, same output)
    constexpr int UPW = 6;
    const int nunits = ((p.N + 15) / 16 + kFp8NUnit - 1) / kFp8NUnit;
    const int n_groups = (nunits + 4 * UPW - 1) / (4 * UPW);
    const int64_t nblocks = ((((m_total + 63) / 64 + p.E) * n_groups) + 7) / 8 * 8;
    if (nblocks >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    const dim3 ngrid(static_cast<unsigned>(nblocks));
    if (epilogue == EPI_F32) {
      if (nt) hipLaunchKernelGGL((k_fp8_gemm_n<UPW, EPI_F32, true>), ngrid, dim3(256), 0, stream, p, n_groups);
      else hipLaunchKernelGGL((k_fp8_gemm_n<UPW, EPI_F32, false>), ngrid, dim3(256), 0, stream, p, n_groups);
    } else {
      if (nt) hipLaunchKernelGGL((k_fp8_gemm_n<UPW, EPI_BF16, true>), ngrid, dim3(256), 0, stream, p, n_groups);
      else hipLaunchKernelGGL((k_fp8_gemm_n<UPW, EPI_BF16, false>), ngrid, dim3(256), 0, stream, p, n_groups);
    }
    return hipGetLastError();
  }
  if (rows_per_expert >= kFp8LRows) {
    const int64_t lblocks = ((((m_total + kFp8LRows - 1) / kFp8LRows + p.E) * n_tiles) + 7) / 8 * 8;
    const dim3 lgrid(static_cast<unsigned>(lblocks));
    if (epilogue == EPI_F32)
      hipLaunchKernelGGL((k_fp8_gemm_l<EPI_F32>), lgrid, dim3(kFp8LThreads), 0, stream, p, n_tiles);
    else
      hipLaunchKernelGGL((k_fp8_gemm_l<EPI_BF16>), lgrid, dim3(kFp8LThreads), 0, stream, p, n_tiles);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(blocks));
  if (epilogue == EPI_F32) {
    if (nt) hipLaunchKernelGGL((k_fp8_gemm<EPI_F32, true>), grid, dim3(256), 0, stream, p, n_tiles);
    else hipLaunchKernelGGL((k_fp8_gemm<EPI_F32, false>), grid, dim3(256), 0, stream, p, n_tiles);
  } else {
    if (nt) hipLaunchKernelGGL((k_fp8_gemm<EPI_BF16, true>), grid, dim3(256), 0, stream, p, n_tiles);
    else hipLaunchKernelGGL((k_fp8_gemm<EPI_BF16, false>), grid, dim3(256), 0, stream, p, n_tiles);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
