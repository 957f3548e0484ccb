// MXFP4 variant for gfx950: E2M1 values with one E8M0 power-of-two scale per
// 32 values along K (the OCP MX format; the pages name an MXFP4 grouped GEMM
// with 128x128x128 tiles among the kernels they survey: "From Empirical
// Limits to Research-Driven Optimization", section "Sections 2-4: Framework
// and Community Landscape").  This format maps onto gfx950's block-scaled
// matrix instruction directly: v_mfma_scale_f32_16x16x128_f8f6f4 takes E2M1
// operands and one E8M0 scale per lane, and a lane holds exactly one 32-value
// block of one row.  So there is no decode in registers at all: codes go from
// memory to the matrix core.
//
//   mx_quantize    x (bf16/f32) -> codes + E8M0 scales: X = floor(log2 absmax)
//                  - 2 (clamped to [-127, 127]), code = E2M1 nearest-even of
//                  x * 2^-X (exact), saturating at 6; a zero block gets scale 0
//                  and codes 0
//   mx gemm        grouped GEMM over row chunks of experts, epilogues f32, bf16
//                  and SwiGLU + MXFP4 requantisation of h
//
// GEMM operand mapping (both operands row-major, K contiguous): a K step is 256
// values (128 code bytes and 8 scale bytes per row); lane l = 16 g + r reads the
// 32 code bytes [32 g, 32 g + 32) of its row (values [64 g, 64 g + 64)) and the
// 2 scale bytes of those two blocks.  MFMA h (0, 1) of the step takes the lane's
// block 2g + h, with the scale byte selected by op_sel: the step's two MFMAs
// cover the 8 blocks once.  The sum over K is order-free.  When K is not a
// multiple of 256 the last step's blocks past K are zeroed (K % 32 == 0).
// The activation rows of a step are staged in LDS once per workgroup;
// weights stream into registers from the packed tiles (mxfp4_weight_repack)
// or, slower, from row-major rows.
#include "gemm_device.h"

namespace nvfp4 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kMxFmtFp4 = 4;       // operand format code of E2M1 in the scaled MFMA

// ------------------------------------------------------------------ quantise
// One thread per 32-value block.
template <int DT>
__global__ __launch_bounds__(256) void k_mx_quantize(const void* __restrict__ x, int64_t nblocks,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t b = blockIdx.x * 256ll + threadIdx.x;
  if (b >= nblocks) return;
  float v[32];
  if constexpr (DT == 1) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + b * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w = src[q];
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = __uint_as_float(u[i] << 16);
        v[8 * q + 2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(x) + b * 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 w = src[q];
      v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // floor(log2 amax) from the exponent field; a subnormal or zero amax gives
  // an exponent of -127 or below, which the clamp turns into -127 anyway
  const int ex = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFF) - 127;
  const int X = min(max(ex - 2, -127), 127);
  // 2^-X as a float (exact; 2^-127 is a subnormal, 2^127 the largest power)
  const float inv = X == 127 ? __uint_as_float(0x00400000u) : __uint_as_float(static_cast<uint32_t>(127 - X) << 23);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (amax > 0.0f) {
    float q[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) q[i] = v[i] * inv;    // exact: a power of two, no overflow (|q| < 8)
    float h0[16], h1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { h0[i] = q[i]; h1[i] = q[16 + i]; }
    w[0] = e2m1_pack8<0>(h0);
    w[1] = e2m1_pack8<8>(h0);
    w[2] = e2m1_pack8<0>(h1);
    w[3] = e2m1_pack8<8>(h1);
  }
  reinterpret_cast<uint4*>(codes)[b] = make_uint4(w[0], w[1], w[2], w[3]);
  scales[b] = static_cast<uint8_t>(X + 127);
}

hipError_t launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream) {
  const int64_t nb = rows * (cols / 32);
  const dim3 grid(static_cast<unsigned>((nb + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(k_mx_quantize<1>, grid, dim3(256), 0, stream, x, nb, codes, scales);
  else
    hipLaunchKernelGGL(k_mx_quantize<0>, grid, dim3(256), 0, stream, x, nb, codes, scales);
  return hipGetLastError();
}

// ------------------------------------------------------------------ packed weights
// Tile (e, 16-row tile rt, 256-K step st) of 2176 bytes: lane l = 16 g + n
// (row n of the tile, lane group g) finds the code bytes of its blocks 2g and
// 2g + 1 (values [64 g, 64 g + 64) of the step) at [16 l, 16 l + 16) and
// [1024 + 16 l, +16), and their two E8M0 scale bytes at [2048 + 2 l, +2).  A
// wave then loads a tile with two fully contiguous 1 KB reads and one 128-byte
// read; zero padded past N and K (a zero code adds 0 whatever its scale).
constexpr int kMxTile = 2176;

size_t mx_packed_weight_bytes(int E, int N, int K) {
  return static_cast<size_t>(E) * ((int64_t(N) + 15) / 16) * ((int64_t(K) + 255) / 256) * kMxTile;
}

__global__ __launch_bounds__(256) void k_mx_repack(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                   int E, int N, int K, uint8_t* __restrict__ packed,
                                                   int64_t total_tiles) {
  const int64_t t = blockIdx.x * 256ll + threadIdx.x;
  const int64_t tile = t >> 6;
  const int lane = static_cast<int>(t & 63);
  if (tile >= total_tiles) return;
  const int nst = (K + 255) / 256;
  const int ntr = (N + 15) / 16;
  const int st = static_cast<int>(tile % nst);
  const int rt = static_cast<int>((tile / nst) % ntr);
  const int e = static_cast<int>(tile / (static_cast<int64_t>(nst) * ntr));
  const int n = 16 * rt + (lane & 15);
  const int g = lane >> 4;
  uint8_t* dst = packed + tile * kMxTile;
  const bool row_ok = n < N;
  const size_t row = static_cast<size_t>(e) * N + (row_ok ? n : 0);
  uint32_t sc = 0u;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = 256 * st + 64 * g + 32 * h;   // K % 32 == 0: a block is all in or all out
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row_ok && k < K) {
      v = *reinterpret_cast<const u32x4*>(codes + row * (K / 2) + k / 2);
      sc |= static_cast<uint32_t>(scales[row * (K / 32) + k / 32]) << (8 * h);
    } else {
      sc |= 127u << (8 * h);
    }
    *reinterpret_cast<u32x4*>(dst + 1024 * h + 16 * lane) = v;
  }
  *reinterpret_cast<uint16_t*>(dst + 2048 + 2 * lane) = static_cast<uint16_t>(sc);
}

hipError_t launch_mx_repack(const uint8_t* codes, const uint8_t* scales, int E, int N, int K, uint8_t* packed,
                            hipStream_t stream) {
  const int64_t tiles = static_cast<int64_t>(E) * ((N + 15) / 16) * ((K + 255) / 256);
  hipLaunchKernelGGL(k_mx_repack, dim3(static_cast<unsigned>((tiles * 64 + 255) / 256)), dim3(256), 0, stream, codes,
                     scales, E, N, K, packed, tiles);
  return hipGetLastError();
}

// ------------------------------------------------------------------ GEMM
constexpr int kMxKStep = 256;
constexpr int kMxRowLds = 144;     // LDS bytes per A row of a step: 128 code bytes + 16 of padding
                                   // (a 36-dword pitch keeps 8 consecutive rows on distinct banks)
constexpr int kMxScLds = 8;        // E8M0 bytes per A row of a step

// one lane's operand data of one K step: 8 code dwords (two 32-value blocks)
// and the two blocks' scale bytes in the low 16 bits
struct MxOp {
  u32x4 c[2];
  uint32_t s;
};

__device__ __forceinline__ i32x8 mx_frag(const MxOp& o, int h) {
  const u32x4 c = o.c[h];
  i32x8 r = {static_cast<int>(c.x), static_cast<int>(c.y), static_cast<int>(c.z), static_cast<int>(c.w), 0, 0, 0, 0};
  return r;
}

template <int H>
__device__ __forceinline__ float4v mx_mfma(const MxOp& a, const MxOp& b, float4v acc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(mx_frag(a, H), mx_frag(b, H), acc, kMxFmtFp4, kMxFmtFp4,
                                                           H, static_cast<int>(a.s), H, static_cast<int>(b.s));
}

// ---- A: the chunk's rows of one K step, staged in LDS by the whole workgroup.
// Thread t stages (row t / 4, quarter t % 4) of the 64 x 128 code bytes and
// the 8 scale bytes of row t % 64 (four threads store the same bytes).  Rows past the chunk's live rows,
// and blocks past K, are staged as zero codes with a neutral scale (2^0).
struct MxAStage {
  rsrc_t rc, rs;
  uint32_t vc, vs;      // byte offsets of the thread's piece at step 0
  bool row_ok;
  int q;                // code quarter (32 bytes) of the thread
};
struct MxARegs {
  u32x4 c[2];
  uint32_t s[2];
};

__device__ __forceinline__ void mxa_setup(const GemmParams& p, int row0, int m0, int rows, MxAStage& S) {
  const int t = threadIdx.x;
  const uint32_t krow = static_cast<uint32_t>(p.K) / 2, srow = static_cast<uint32_t>(p.K) / 32;
  S.rc = make_rsrc(p.a_codes, static_cast<uint32_t>(p.a_rows_total) * krow);
  S.rs = make_rsrc(p.a_scales, static_cast<uint32_t>(p.a_rows_total) * srow);
  const int ar = t >> 2;
  S.q = t & 3;
  S.row_ok = ar < rows;
  int arow = row0 + m0 + (S.row_ok ? ar : 0);
  if (p.a_rows) arow = p.a_rows[arow];
  arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
  S.vc = static_cast<uint32_t>(arow) * krow + 32u * S.q;
  const int sr = t & 63;  // scale row: threads t, t + 64, ... stage the same row's bytes
  int srow_i = row0 + m0 + (sr < rows ? sr : 0);
  if (p.a_rows) srow_i = p.a_rows[min(srow_i, p.m_total - 1)];
  srow_i = (srow_i >= 0 && srow_i < p.a_rows_total) ? srow_i : 0;
  S.vs = static_cast<uint32_t>(srow_i) * srow;
}

// loads of step st (clamped to the last step; blocks past K masked at the store)
__device__ __forceinline__ void mxa_load(const MxAStage& S, MxARegs& R, int st, int K) {
  const int s = min(st, (K - 1) / kMxKStep);
  const uint32_t oc = static_cast<uint32_t>(s) * (kMxKStep / 2);
  const uint32_t os = static_cast<uint32_t>(s) * (kMxKStep / 32);
  R.c[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(S.rc, S.vc + oc, 0, 0));
  R.c[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(S.rc, S.vc + oc + 16u, 0, 0));
  // the 8 scale bytes of the row, byte by byte: a row's scales start at any
  // byte when K % 128 != 0, and the range check (zeros past the buffer) is
  // exact per byte
  const uint32_t sb = S.vs + os;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t w = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      w |= static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b8(S.rs, sb + 4u * i + b, 0, 0)) << (8 * b);
    R.s[i] = w;
  }
}

// st_valid: the step exists (steps past the last one store zeros)
__device__ __forceinline__ void mxa_store(const MxAStage& S, const MxARegs& R, int st, int K, uint8_t* __restrict__ lds,
                                          int rows) {
  const int t = threadIdx.x;
  const int k0 = st * kMxKStep + 64 * S.q;          // first value of the thread's 32 code bytes
  const u32x4 z = {0u, 0u, 0u, 0u};
  const bool ok0 = S.row_ok && k0 < K;
  const bool ok1 = S.row_ok && k0 + 32 < K;
  u32x4* dst = reinterpret_cast<u32x4*>(lds + (t >> 2) * kMxRowLds + 32 * S.q);
  dst[0] = ok0 ? R.c[0] : z;
  dst[1] = ok1 ? R.c[1] : z;
  // scale byte b of the row: block b of the step; neutral (2^0) past K or
  // for rows that do not exist.  Every thread stores (threads t, t + 64, ...
  // the same bytes of row t % 64): no divergent branch inside the K loop.
  {
    const int sr = t & 63;
    uint32_t w[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t v = R.s[i];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bool ok = sr < rows && st * kMxKStep + 32 * (4 * i + b) < K;
        v = ok ? v : ((v & ~(0xFFu << (8 * b))) | (127u << (8 * b)));
      }
      w[i] = v;
    }
    *reinterpret_cast<uint2*>(lds + 64 * kMxRowLds + sr * kMxScLds) = make_uint2(w[0], w[1]);
  }
}

// A fragments of row tile r for this lane (row 16 r + lr, blocks 2g, 2g + 1)
__device__ __forceinline__ void mxa_frag(const uint8_t* __restrict__ lds, int r, MxOp& A) {
  const int lane = threadIdx.x & 63;
  const int row = 16 * r + (lane & 15);
  const int g = lane >> 4;
  const u32x4* src = reinterpret_cast<const u32x4*>(lds + row * kMxRowLds + 32 * g);
  A.c[0] = src[0];
  A.c[1] = src[1];
  A.s = *reinterpret_cast<const uint16_t*>(lds + 64 * kMxRowLds + row * kMxScLds + 2 * g);
}
constexpr int kMxALds = 64 * kMxRowLds + 64 * kMxScLds;   // bytes of one staged A step (9.7 KB)

// ---- B: packed tiles (PACKED) or row-major rows
template <int WN, bool PACKED>
struct MxBSrc {
  const uint8_t* base_c;   // expert's packed tiles, or its code rows
  const uint8_t* base_s;   // its scale rows (row-major)
  uint32_t oc[WN];         // lane offsets at step 0 (packed: of the tile, lane offset included)
  uint32_t os[WN];
  int K;
};

template <int WN, bool PACKED, bool NT>
__device__ __forceinline__ void mxb_load(const MxBSrc<WN, PACKED>& B, MxOp (&R)[WN], int st, int nsteps) {
  const int s = min(st, nsteps - 1);
  if constexpr (PACKED) {
    const uint32_t ot = static_cast<uint32_t>(s) * kMxTile;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const uint8_t* t = B.base_c + (B.oc[j] + ot);
      const u32x4* p0 = reinterpret_cast<const u32x4*>(t);
      const u32x4* p1 = reinterpret_cast<const u32x4*>(t + 1024);
      const uint16_t* ps = reinterpret_cast<const uint16_t*>(B.base_c + (B.os[j] + ot));
      if constexpr (NT) {
        R[j].c[0] = __builtin_nontemporal_load(p0);
        R[j].c[1] = __builtin_nontemporal_load(p1);
        R[j].s = __builtin_nontemporal_load(ps);
      } else {
        R[j].c[0] = *p0;
        R[j].c[1] = *p1;
        R[j].s = *ps;
      }
    }
  } else {
    // row-major: each 16-byte half (one block) clamped into its row and, past
    // K, replaced by zero codes with a neutral scale
    const int g = (threadIdx.x & 63) >> 4;
    const int K = B.K;
    const int k0 = s * kMxKStep + 64 * g;
    const bool ok0 = k0 < K, ok1 = k0 + 32 < K;
    const uint32_t pc = 32u * g, ps = 2u * g;
    const uint32_t oc0 = min(pc + static_cast<uint32_t>(s) * (kMxKStep / 2), static_cast<uint32_t>(K / 2 - 16)) - pc;
    const uint32_t oc1 = min(pc + static_cast<uint32_t>(s) * (kMxKStep / 2) + 16u, static_cast<uint32_t>(K / 2 - 16)) - pc;
    const uint32_t os0 = min(ps + static_cast<uint32_t>(s) * (kMxKStep / 32), static_cast<uint32_t>(K / 32 - 1)) - ps;
    const uint32_t os1 = min(ps + static_cast<uint32_t>(s) * (kMxKStep / 32) + 1u, static_cast<uint32_t>(K / 32 - 1)) - ps;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const u32x4 c0 = *reinterpret_cast<const u32x4*>(B.base_c + (B.oc[j] + oc0));
      const u32x4 c1 = *reinterpret_cast<const u32x4*>(B.base_c + (B.oc[j] + oc1));
      const uint32_t s0 = B.base_s[B.os[j] + os0];
      const uint32_t s1 = B.base_s[B.os[j] + os1];
      R[j].c[0] = ok0 ? c0 : z;
      R[j].c[1] = ok1 ? c1 : z;
      R[j].s = (ok0 ? s0 : 127u) | ((ok1 ? s1 : 127u) << 8);
    }
  }
}

template <int WN, bool PACKED>
__device__ __forceinline__ void mxb_setup(const GemmParams& p, int e, const int (&col)[WN], const bool (&ok)[WN],
                                          int nsteps, MxBSrc<WN, PACKED>& B) {
  const int lane = threadIdx.x & 63;
  const int N = p.N;
  B.K = p.K;
  if constexpr (PACKED) {
    const int ntr = (N + 15) / 16;
    B.base_c = p.b_packed + static_cast<size_t>(e) * ntr * nsteps * kMxTile;
    B.base_s = B.base_c;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const uint32_t rt = static_cast<uint32_t>(min(col[j] / 16, ntr - 1));
      B.oc[j] = rt * static_cast<uint32_t>(nsteps) * kMxTile + 16u * lane;
      B.os[j] = rt * static_cast<uint32_t>(nsteps) * kMxTile + 2048u + 2u * lane;
    }
  } else {
    const uint32_t krow = static_cast<uint32_t>(p.K) / 2, srow = static_cast<uint32_t>(p.K) / 32;
    const int g = lane >> 4;
    B.base_c = p.b_codes + static_cast<size_t>(e) * N * krow;
    B.base_s = p.b_scales + static_cast<size_t>(e) * N * srow;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const uint32_t brow = static_cast<uint32_t>(ok[j] ? col[j] + (lane & 15) : 0);
      B.oc[j] = brow * krow + 32u * g;
      B.os[j] = brow * srow + 2u * g;
    }
  }
}

template <int MT, int MTA, int WN>
__device__ __forceinline__ void mx_step(const uint8_t* __restrict__ a_lds, const MxOp (&B)[WN],
                                        float4v (&acc)[MT][WN]) {
#pragma unroll
  for (int r = 0; r < MTA; ++r) {
    MxOp A;
    mxa_frag(a_lds, r, A);
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[r][j] = mx_mfma<0>(A, B[j], acc[r][j]);
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[r][j] = mx_mfma<1>(A, B[j], acc[r][j]);
  }
}

// Software-pipelined K loop, branch-free like the NVFP4 one: weights one to
// two steps ahead in alternating register sets, the activation step staged in
// LDS (double-buffered) one step ahead of the MFMAs.  Steps past the last are
// computed on zero codes (A staged as zeros), which adds exactly 0.
template <int MT, int MTA, int WN, bool PACKED, bool NT>
__device__ __forceinline__ void mx_loop(const MxAStage& AS, const MxBSrc<WN, PACKED>& BS, int nsteps, int K, int rows,
                                        uint8_t* __restrict__ lds0, uint8_t* __restrict__ lds1,
                                        float4v (&acc)[MT][WN]) {
  MxOp B0[WN], B1[WN];
  MxARegs ra;
  mxa_load(AS, ra, 0, K);
  mxb_load<WN, PACKED, NT>(BS, B0, 0, nsteps);
  mxb_load<WN, PACKED, NT>(BS, B1, 1, nsteps);
  mxa_store(AS, ra, 0, K, lds0, rows);
  mxa_load(AS, ra, 1, K);
  __syncthreads();
  for (int st = 0; st < nsteps; st += 2) {
    mx_step<MT, MTA, WN>(lds0, B0, acc);
    mxa_store(AS, ra, st + 1, K, lds1, rows);
    mxa_load(AS, ra, st + 2, K);
    mxb_load<WN, PACKED, NT>(BS, B0, st + 2, nsteps);
    __syncthreads();
    mx_step<MT, MTA, WN>(lds1, B1, acc);
    mxa_store(AS, ra, st + 2, K, lds0, rows);
    mxa_load(AS, ra, st + 3, K);
    mxb_load<WN, PACKED, NT>(BS, B1, st + 3, nsteps);
    __syncthreads();
  }
}

// SwiGLU + MXFP4 requantisation of one 16-row tile: the wave's two gate tiles
// (h columns hc0 + [0, 32), one MX block) and the matching up tiles.  Lane
// (lr, lg) holds rows 4 lg + i of column lr of each tile.
__device__ __forceinline__ void mx_epilogue_swiglu(const GemmParams& p, const float4v& g0, const float4v& g1,
                                                   const float4v& u0, const float4v& u1, int prow0, int rows_left,
                                                   int hc0, bool blk_ok, float gab) {
  const int lr = threadIdx.x & 15;
  const int lg = (threadIdx.x & 63) >> 4;
  const int I = p.N / 2;
  float h0[4], h1[4], am[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h0[i] = silu_fast(g0[i] * gab) * (u0[i] * gab);
    h1[i] = silu_fast(g1[i] * gab) * (u1[i] * gab);
    am[i] = row16_max(fmaxf(fabsf(h0[i]), fabsf(h1[i])));
  }
  const int q = lr & 3;
  const float amq = q == 0 ? am[0] : q == 1 ? am[1] : q == 2 ? am[2] : am[3];
  const int exq = static_cast<int>((__float_as_uint(amq) >> 23) & 0xFF) - 127;
  const int Xq = min(max(exq - 2, -127), 127);
  if (lr < 4 && 4 * lg + lr < rows_left && blk_ok)
    p.out_scales[static_cast<size_t>(prow0 + 4 * lg + lr) * (I / 32) + hc0 / 32] = static_cast<uint8_t>(Xq + 127);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * lg + i;
    const int ex = static_cast<int>((__float_as_uint(am[i]) >> 23) & 0xFF) - 127;
    const int X = min(max(ex - 2, -127), 127);
    const float inv = X == 127 ? __uint_as_float(0x00400000u) : __uint_as_float(static_cast<uint32_t>(127 - X) << 23);
    const bool nz = am[i] > 0.0f;
    const uint32_t c0 = nz ? e2m1_code(h0[i] * inv) : 0u;
    const uint32_t c1 = nz ? e2m1_code(h1[i] * inv) : 0u;
    const uint32_t o0 = dpp_u32<kDppXor1>(c0);
    const uint32_t o1 = dpp_u32<kDppXor1>(c1);
    if (m < rows_left && blk_ok && (lr & 1) == 0) {
      uint8_t* row = p.out_codes + static_cast<size_t>(prow0 + m) * (I / 2);
      row[(hc0 + lr) / 2] = static_cast<uint8_t>(c0 | (o0 << 4));
      row[(hc0 + 16 + lr) / 2] = static_cast<uint8_t>(c1 | (o1 << 4));
    }
  }
}

// One stream-K task: rows [m0, m0 + 64) of expert e, column tile nt (256
// columns; SwiGLU: 128 gate + 128 up, a wave holding two of each).
template <int WN, int EPI, bool PACKED, bool NT>
__device__ __forceinline__ void mx_task(const GemmParams& p, int e, int m0, int nt, uint8_t* __restrict__ lds0,
                                        uint8_t* __restrict__ lds1) {
  constexpr int MT = 4, NW = 4;
  constexpr int BN = NW * WN * 16;
  static_assert(EPI != EPI_SWIGLU || WN == 4, "SwiGLU: two gate and two up tiles per wave (one MX block of h)");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  const int rows = min(16 * MT, Me - m0);
  const int mt_active = (rows + 15) >> 4;
  const int N = p.N;
  const int K = p.K;
  const int nsteps = (K + kMxKStep - 1) / kMxKStep;

  MxAStage AS;
  mxa_setup(p, row0, m0, rows, AS);
  int col0[WN];
  bool cok[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if constexpr (EPI == EPI_SWIGLU) {
      const int hc0 = nt * (BN / 2) + wave * 32 + (j & 1) * 16;
      cok[j] = hc0 + lr < N / 2;
      col0[j] = (j < 2) ? hc0 : N / 2 + hc0;
    } else {
      col0[j] = nt * BN + wave * WN * 16 + j * 16;
      cok[j] = col0[j] + lr < N;
    }
  }
  MxBSrc<WN, PACKED> BS;
  mxb_setup<WN, PACKED>(p, e, col0, cok, nsteps, BS);
  float4v acc[MT][WN];
#pragma unroll
  for (int r = 0; r < MT; ++r)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[r][j] = float4v{0.f, 0.f, 0.f, 0.f};
  switch (mt_active) {
    case 1: mx_loop<MT, 1, WN, PACKED, NT>(AS, BS, nsteps, K, rows, lds0, lds1, acc); break;
    case 2: mx_loop<MT, 2, WN, PACKED, NT>(AS, BS, nsteps, K, rows, lds0, lds1, acc); break;
    case 3: mx_loop<MT, 3, WN, PACKED, NT>(AS, BS, nsteps, K, rows, lds0, lds1, acc); break;
    default: mx_loop<MT, MT, WN, PACKED, NT>(AS, BS, nsteps, K, rows, lds0, lds1, acc); break;
  }
  const float gab = p.a_g[0] * p.b_g[e];
  const int prow0 = row0 + m0;
#pragma unroll
  for (int r = 0; r < MT; ++r) {
    if (r >= mt_active) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      mx_epilogue_swiglu(p, acc[r][0], acc[r][1], acc[r][2], acc[r][3], prow0 + 16 * r, rows - 16 * r,
                         nt * (BN / 2) + wave * 32, nt * (BN / 2) + wave * 32 < N / 2, gab);
    } else {
#pragma unroll
      for (int j = 0; j < WN; ++j)
        epilogue_tile<EPI>(p, acc[r][j], prow0 + 16 * r, rows - 16 * r, col0[j] + lr, cok[j], gab);
    }
  }
}

template <int WN, int EPI, bool PACKED, bool NT>
__global__ __launch_bounds__(256, 2) void k_mx_gemm(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][kMxALds];
  static_assert(fits_lds(sizeof(a_lds), 2), "MX A staging exceeds the LDS of two workgroups per CU");
  int e, m0, nt;
  bool narrow;
  if (!find_task<4, true, 0>(p, e, m0, nt, narrow)) return;
  mx_task<WN, EPI, PACKED, NT>(p, e, m0, nt, a_lds[0], a_lds[1]);
}

// ---- stream-N (K <= 256, packed weights): the chunk's A step staged once;
// every wave then streams its units of 64 columns (4 tiles), one unit ahead,
// and its rows leave through the per-wave LDS stage as whole 128-byte bf16
// segments (or float32).
template <int MTA, int UPW, int EPI, bool NT>
__device__ __forceinline__ void mxn_loop(const GemmParams& p, const uint8_t* __restrict__ a_lds, float* stage,
                                         const uint8_t* tiles, int u_first, int u_count, int ntr, int prow0, int rows,
                                         float gab) {
  const int lane = threadIdx.x & 63;
  MxOp R0[UNIT], R1[UNIT];
  auto load_unit = [&](MxOp (&R)[UNIT], int i) {
    const int ui = u_first + min(i, u_count - 1);
#pragma unroll
    for (int t = 0; t < UNIT; ++t) {
      const uint8_t* tp = tiles + static_cast<size_t>(min(UNIT * ui + t, ntr - 1)) * kMxTile;
      const u32x4* p0 = reinterpret_cast<const u32x4*>(tp + 16 * lane);
      const u32x4* p1 = reinterpret_cast<const u32x4*>(tp + 1024 + 16 * lane);
      const uint16_t* ps = reinterpret_cast<const uint16_t*>(tp + 2048 + 2 * lane);
      if constexpr (NT) {
        R[t].c[0] = __builtin_nontemporal_load(p0);
        R[t].c[1] = __builtin_nontemporal_load(p1);
        R[t].s = __builtin_nontemporal_load(ps);
      } else {
        R[t].c[0] = *p0;
        R[t].c[1] = *p1;
        R[t].s = *ps;
      }
    }
  };
  auto consume = [&](const MxOp (&R)[UNIT], int i) {
    float4v acc[MTA][UNIT];
#pragma unroll
    for (int r = 0; r < MTA; ++r)
#pragma unroll
      for (int t = 0; t < UNIT; ++t) acc[r][t] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < MTA; ++r) {
      MxOp A;
      mxa_frag(a_lds, r, A);
#pragma unroll
      for (int t = 0; t < UNIT; ++t) acc[r][t] = mx_mfma<0>(A, R[t], acc[r][t]);
#pragma unroll
      for (int t = 0; t < UNIT; ++t) acc[r][t] = mx_mfma<1>(A, R[t], acc[r][t]);
    }
    if (i < u_count) {
      const int col0 = 64 * (u_first + i);
#pragma unroll
      for (int r = 0; r < MTA; ++r) store_unit<EPI>(p, acc[r], stage, prow0 + 16 * r, rows - 16 * r, col0, gab);
    }
  };
  load_unit(R0, 0);
  load_unit(R1, 1);
  for (int i = 0; i < UPW; i += 2) {
    consume(R0, i);
    load_unit(R0, i + 2);
    consume(R1, i + 1);
    load_unit(R1, i + 3);
  }
}

template <int UPW, int EPI, bool NT>
__global__ __launch_bounds__(256, 2) void k_mx_gemm_n(const GemmParams p) {
  constexpr int NW = 4;
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[kMxALds];
  __shared__ float stage_lds[NW * 16 * 68];
  static_assert(fits_lds(sizeof(a_lds) + sizeof(stage_lds), 2), "MX stream-N staging exceeds the LDS of two workgroups per CU");
  int e, m0, ng;
  bool narrow;
  if (!find_task<4, false, 0>(p, e, m0, ng, narrow)) return;
  const int wave = threadIdx.x >> 6;
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  const int rows = min(64, Me - m0);
  const int mt_active = (rows + 15) >> 4;
  MxAStage AS;
  mxa_setup(p, row0, m0, rows, AS);
  MxARegs ra;
  mxa_load(AS, ra, 0, p.K);
  mxa_store(AS, ra, 0, p.K, a_lds, rows);
  __syncthreads();
  const int ntr = (p.N + 15) / 16;
  const int nunits = (ntr + UNIT - 1) / UNIT;
  const int u_first = (ng * NW + wave) * UPW;
  const int u_count = min(UPW, nunits - u_first);
  if (u_count <= 0) return;
  const uint8_t* tiles = p.b_packed + static_cast<size_t>(e) * ntr * kMxTile;
  const float gab = p.a_g[0] * p.b_g[e];
  const int prow0 = row0 + m0;
  float* stage = stage_lds + wave * (16 * 68);
  switch (mt_active) {
    case 1: mxn_loop<1, UPW, EPI, NT>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
    case 2: mxn_loop<2, UPW, EPI, NT>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
    case 3: mxn_loop<3, UPW, EPI, NT>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
    default: mxn_loop<4, UPW, EPI, NT>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
  }
}

// ---- large-M tile (K % 256 == 0, packed weights): a workgroup of 8 waves
// computes 256 rows x 256 columns (SwiGLU: 128 gate + 128 up), with both
// operands of a K step staged in LDS: each fragment read from memory once per
// workgroup feeds 8 (A) or 16 (B) waves' worth of MFMAs instead of one, which
// moves the kernel from the weight stream to the matrix core once experts
// hold hundreds of rows.  Wave w = 4 wr + wc holds rows [128 wr, +128) and
// the four 16-column tiles 4 wc.. (SwiGLU: gate tiles 2 wc, 2 wc + 1 and the
// matching up tiles).  One stage (68 KB, two of them double-buffered):
//   A codes   16 row tiles x 2048 bytes: half h of lane (g, r) at
//             1024 h + 256 g + 16 (r ^ (2 g + h)) (the XOR spreads the 8
//             lanes that store one row's 128 code bytes over distinct banks)
//   A scales  256 rows x 8 bytes (the step's 8 E8M0 bytes of the row)
//   B codes   16 column tiles x 2048 bytes, as in the packed tile
//   B scales  16 column tiles x 128 bytes, as in the packed tile
// The next step's global loads are issued before the MFMAs of the current
// one and stored into the other stage after them: one barrier per step.
constexpr int kMxLRows = 256;
constexpr int kMxLThreads = 512;
constexpr int kMxLA = 0;
constexpr int kMxLASc = 16 * 2048;
constexpr int kMxLB = kMxLASc + kMxLRows * 8;
constexpr int kMxLBSc = kMxLB + 16 * 2048;
constexpr int kMxLStage = kMxLBSc + 16 * 128;

// the thread's staging registers: its A pieces of a step, or its B pieces
struct MxLRegs {
  u32x4 c[4];
  uint32_t s;
};

struct MxLSrc {
  rsrc_t ra, rs;            // A codes and scales (range-checked)
  uint32_t va[4];           // byte offset of the thread's four A pieces at step 0
  uint32_t vs;              // of its A scale word at step 0
  uint32_t lda;             // LDS offset of its first A piece (the others follow 8 KB apart)
  const uint8_t* b;         // expert's packed tiles
  uint32_t ob[4];           // byte offset of the thread's four B code pieces at step 0
  uint32_t obs;             // of its B scale word at step 0
};

__device__ __forceinline__ void mxl_load_a(const MxLSrc& S, MxLRegs& R, int st) {
  const uint32_t oa = static_cast<uint32_t>(st) * (kMxKStep / 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    R.c[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(S.ra, S.va[i] + oa, 0, 0));
  R.s = __builtin_amdgcn_raw_buffer_load_b32(S.rs, S.vs + static_cast<uint32_t>(st) * (kMxKStep / 32), 0, 0);
}

__device__ __forceinline__ void mxl_load_b(const MxLSrc& S, MxLRegs& R, int st) {
  const uint32_t ot = static_cast<uint32_t>(st) * kMxTile;
#pragma unroll
  for (int i = 0; i < 4; ++i) R.c[i] = *reinterpret_cast<const u32x4*>(S.b + (S.ob[i] + ot));
  R.s = *reinterpret_cast<const uint32_t*>(S.b + (S.obs + ot));
}

__device__ __forceinline__ void mxl_store_a(const MxLSrc& S, const MxLRegs& R, uint8_t* __restrict__ stage) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(stage + S.lda + 8192 * i) = R.c[i];
  *reinterpret_cast<uint32_t*>(stage + kMxLASc + 4 * threadIdx.x) = R.s;
}

__device__ __forceinline__ void mxl_store_b(const MxLRegs& R, uint8_t* __restrict__ stage) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(stage + kMxLB + 16 * (t + kMxLThreads * i)) = R.c[i];
  *reinterpret_cast<uint32_t*>(stage + kMxLBSc + 4 * t) = R.s;
}

// half H of one staged step (the lane's block 2 g + H of each row): wave rows
// [128 wr, +128), B tiles jt[0..3]
template <int H>
__device__ __forceinline__ void mxl_half(const uint8_t* __restrict__ stage, int wr, const int (&jt)[4],
                                         const uint32_t (&asc)[8], const uint32_t (&bsc)[4], float4v (&acc)[8][4]) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  i32x8 bf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 c = *reinterpret_cast<const u32x4*>(stage + kMxLB + jt[j] * 2048 + 1024 * H + 16 * lane);
    bf[j] = i32x8{static_cast<int>(c.x), static_cast<int>(c.y), static_cast<int>(c.z), static_cast<int>(c.w),
                  0, 0, 0, 0};
  }
  const int aoff = kMxLA + 1024 * H + 256 * lg + 16 * (lr ^ (2 * lg + H));
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const u32x4 c = *reinterpret_cast<const u32x4*>(stage + aoff + (8 * wr + r) * 2048);
    const i32x8 af = {static_cast<int>(c.x), static_cast<int>(c.y), static_cast<int>(c.z), static_cast<int>(c.w),
                      0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[r][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[r][j], kMxFmtFp4, kMxFmtFp4, H,
                                                                    static_cast<int>(asc[r]), H,
                                                                    static_cast<int>(bsc[j]));
  }
}

// the scale bytes of one staged step for this wave's row and column tiles
__device__ __forceinline__ void mxl_scales(const uint8_t* __restrict__ stage, int wr, const int (&jt)[4],
                                           uint32_t (&asc)[8], uint32_t (&bsc)[4]) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bsc[j] = *reinterpret_cast<const uint16_t*>(stage + kMxLBSc + jt[j] * 128 + 2 * lane);
#pragma unroll
  for (int r = 0; r < 8; ++r)
    asc[r] = *reinterpret_cast<const uint16_t*>(stage + kMxLASc + (16 * (8 * wr + r) + lr) * 8 + 2 * lg);
}

template <int EPI>
__global__ __launch_bounds__(kMxLThreads, 1) void k_mx_gemm_l(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kMxLStage];
  static_assert(fits_lds(sizeof(lds), 1), "MX large-M staging exceeds the LDS of a CU");
  int e, m0, nt;
  bool narrow;
  if (!find_task<16, false, 0>(p, e, m0, nt, narrow)) return;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wr = wave >> 2, wc = wave & 3;
  const int lr = lane & 15;
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  // inside an expert, groups of 4 row chunks run column tile by column tile,
  // so that the workgroups running side by side on an XCD share 4 A chunks
  // and a few weight column tiles in its L2
  {
    const int nc = (Me + kMxLRows - 1) / kMxLRows;
    const int u = (m0 / kMxLRows) * p.n_tiles + nt;
    const int grp = (m0 / kMxLRows) / 4;
    const int gq = min(4, nc - 4 * grp);
    const int w = u - 4 * grp * p.n_tiles;
    m0 = (4 * grp + w % gq) * kMxLRows;
    nt = w / gq;
  }
  const int rows = min(kMxLRows, Me - m0);
  const int N = p.N, K = p.K;
  const int nsteps = K / kMxKStep;
  const int ntr = N / 16;

  MxLSrc S;
  {
    const uint32_t krow = static_cast<uint32_t>(K) / 2, srow = static_cast<uint32_t>(K) / 32;
    S.ra = make_rsrc(p.a_codes, static_cast<uint32_t>(p.a_rows_total) * krow);
    S.rs = make_rsrc(p.a_scales, static_cast<uint32_t>(p.a_rows_total) * srow);
    const int blk = t & 7;            // 32-value block of the step this thread stages for its A rows
    const int g = blk >> 1, h = blk & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ar = (t >> 3) + 64 * i;
      int arow = row0 + m0 + (ar < rows ? ar : 0);
      if (p.a_rows) arow = p.a_rows[arow];
      arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
      S.va[i] = static_cast<uint32_t>(arow) * krow + 16u * blk;
    }
    // rows t / 8 + 64 i: row tile 4 i further, 8 KB apart
    S.lda = kMxLA + ((t >> 3) >> 4) * 2048 + 1024 * h + 256 * g + 16 * (((t >> 3) & 15) ^ (2 * g + h));
    {
      const int ar = t >> 1;
      int arow = row0 + m0 + (ar < rows ? ar : 0);
      if (p.a_rows) arow = p.a_rows[arow];
      arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
      S.vs = static_cast<uint32_t>(arow) * srow + 4u * (t & 1);
    }
    S.b = p.b_packed + static_cast<size_t>(e) * ntr * nsteps * kMxTile;
    auto tile_of = [&](int j) {     // packed column tile of LDS tile j
      int rt;
      if constexpr (EPI == EPI_SWIGLU)
        rt = j < 8 ? nt * 8 + j : (N / 32) + nt * 8 + (j - 8);
      else
        rt = nt * 16 + j;
      return static_cast<uint32_t>(min(rt, ntr - 1));
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = t + kMxLThreads * i;     // 16-byte piece of the 16 x 2048 code bytes
      S.ob[i] = tile_of(pc >> 7) * static_cast<uint32_t>(nsteps) * kMxTile + 16u * (pc & 127);
    }
    S.obs = tile_of(t >> 5) * static_cast<uint32_t>(nsteps) * kMxTile + 2048u + 4u * (t & 31);
  }
  int jt[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (EPI == EPI_SWIGLU)
      jt[j] = (j < 2 ? 0 : 8) + 2 * wc + (j & 1);
    else
      jt[j] = 4 * wc + j;
  }

  float4v acc[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[r][j] = float4v{0.f, 0.f, 0.f, 0.f};

  // prologue: step 0 into stage 0
  MxLRegs R;
  mxl_load_a(S, R, 0);
  mxl_store_a(S, R, lds);
  mxl_load_b(S, R, 0);
  mxl_store_b(R, lds);
  __syncthreads();
  // Step st computes from stage st % 2 while the loads of step st + 1 go to
  // the other stage (its readers passed the previous barrier): the A pieces
  // in flight behind the first half of the MFMAs, the B pieces behind the
  // second half.  Scheduling barriers keep the compiler from sinking the
  // loads down to their stores, which would expose their latency (dense
  // 8192^3: 360 -> 338 us).  No branches: the last step re-stages itself into
  // the idle stage, which nothing reads afterwards.
  for (int st = 0; st < nsteps; ++st) {
    const uint8_t* cur = lds + (st & 1) * kMxLStage;
    uint8_t* nxt = lds + ((st + 1) & 1) * kMxLStage;
    const int sn = min(st + 1, nsteps - 1);
    uint32_t asc[8], bsc[4];
    mxl_scales(cur, wr, jt, asc, bsc);
    mxl_load_a(S, R, sn);
    __builtin_amdgcn_sched_barrier(0);
    mxl_half<0>(cur, wr, jt, asc, bsc, acc);
    mxl_store_a(S, R, nxt);
    mxl_load_b(S, R, sn);
    __builtin_amdgcn_sched_barrier(0);
    mxl_half<1>(cur, wr, jt, asc, bsc, acc);
    mxl_store_b(R, nxt);
    __syncthreads();
  }

  const float gab = p.a_g[0] * p.b_g[e];
  const int prow0 = row0 + m0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int rt = 8 * wr + r;
    const int left = rows - 16 * rt;
    if (left <= 0) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      const int hc0 = nt * 128 + 32 * wc;
      mx_epilogue_swiglu(p, acc[r][0], acc[r][1], acc[r][2], acc[r][3], prow0 + 16 * rt, left, hc0, hc0 < N / 2,
                         gab);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = nt * 256 + 64 * wc + 16 * j;
        epilogue_tile<EPI>(p, acc[r][j], prow0 + 16 * rt, left, col + lr, col + lr < N, gab);
      }
    }
  }
}

template <int EPI>
static hipError_t launch_mx_l(GemmParams prm, int64_t m_total, hipStream_t stream) {
  const int cols = (EPI == EPI_SWIGLU) ? prm.N / 2 : prm.N;
  const int per = (EPI == EPI_SWIGLU) ? 128 : 256;
  prm.n_tiles = (cols + per - 1) / per;
  prm.slots = 1 << 30;
  const int64_t blocks = ((((m_total + kMxLRows - 1) / kMxLRows + prm.E) * prm.n_tiles) + 7) / 8 * 8;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_mx_gemm_l<EPI>), dim3(static_cast<unsigned>(blocks)), dim3(kMxLThreads), 0, stream, prm);
  return hipGetLastError();
}

template <int EPI, bool PACKED, bool NT>
static hipError_t launch_mx_k(GemmParams prm, int64_t m_total, hipStream_t stream) {
  constexpr int WN = 4, BN = 4 * WN * 16;
  const int cols = (EPI == EPI_SWIGLU) ? prm.N / 2 : prm.N;
  const int per = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  prm.n_tiles = (cols + per - 1) / per;
  prm.slots = 1 << 30;
  const int64_t blocks = ((((m_total + 63) / 64 + prm.E) * prm.n_tiles) + 7) / 8 * 8;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_mx_gemm<WN, EPI, PACKED, NT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

template <int EPI, bool NT>
static hipError_t launch_mx_n(GemmParams prm, int64_t m_total, hipStream_t stream) {
  constexpr int UPW = 6;
  const int nunits = ((prm.N + 15) / 16 + UNIT - 1) / UNIT;
  prm.n_tiles = (nunits + 4 * UPW - 1) / (4 * UPW);
  prm.slots = 1 << 30;
  const int64_t blocks = ((((m_total + 63) / 64 + prm.E) * prm.n_tiles) + 7) / 8 * 8;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_mx_gemm_n<UPW, EPI, NT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

// Weight loads are cached once the experts average a full 64-row chunk (their
// chunks then share tiles in L2), non-temporal below.  K <= 256 with packed
// weights and a plain epilogue: the stream-N kernel.
hipError_t launch_mx_gemm(const GemmParams& prm, int epilogue, int64_t m_total, int hint, hipStream_t stream) {
  const int64_t rows_per_expert = hint > 0 ? hint : m_total / prm.E;
  const bool nt = rows_per_expert < 64;
  // one K step with a plain epilogue: the stream-N kernel, at any size (at
  // the prefill down shape it beats the 256 x 256 tile, 570 against 651 us)
  if (prm.b_packed && prm.K <= kMxKStep && (epilogue == EPI_F32 || epilogue == EPI_BF16)) {
    if (epilogue == EPI_F32)
      return nt ? launch_mx_n<EPI_F32, true>(prm, m_total, stream) : launch_mx_n<EPI_F32, false>(prm, m_total, stream);
    return nt ? launch_mx_n<EPI_BF16, true>(prm, m_total, stream) : launch_mx_n<EPI_BF16, false>(prm, m_total, stream);
  }
  if (prm.b_packed && prm.K % kMxKStep == 0 && rows_per_expert >= kMxLRows) {
    switch (epilogue) {
      case EPI_F32: return launch_mx_l<EPI_F32>(prm, m_total, stream);
      case EPI_BF16: return launch_mx_l<EPI_BF16>(prm, m_total, stream);
      case EPI_SWIGLU: return launch_mx_l<EPI_SWIGLU>(prm, m_total, stream);
      default: break;
    }
  }
#define MX_CASE(E_)                                                                                 \
  if (prm.b_packed)                                                                                 \
    return nt ? launch_mx_k<E_, true, true>(prm, m_total, stream)                                   \
              : launch_mx_k<E_, true, false>(prm, m_total, stream);                                 \
  return nt ? launch_mx_k<E_, false, true>(prm, m_total, stream) : launch_mx_k<E_, false, false>(prm, m_total, stream);
  switch (epilogue) {
    case EPI_F32: MX_CASE(EPI_F32)
    case EPI_BF16: MX_CASE(EPI_BF16)
    case EPI_SWIGLU: MX_CASE(EPI_SWIGLU)
    default: return hipErrorInvalidValue;
  }
#undef MX_CASE
}

}  // namespace nvfp4
