// Grouped NVFP4 GEMM for gfx950 with fused epilogues, and the packed weight
// layout it streams.
//
// Computes, for expert e and GEMM row p of that expert (A row r = a_rows[p]):
//   y[p, n] = g_a g_b[e] * sum_kb s_a[r,kb] s_b[e,n,kb] sum_{i<16} q_a q_b
// the block-scaled MMA of "From Empirical Limits to Research-Driven
// Optimization", section "Section 1: CUTLASS Kernels - The Foundation" (E2M1
// operands, one E4M3 scale per 16 K, FP32 accumulate), grouped per expert as in
// the MoE grouped GEMM of section "Sections 2-4: Framework and Community
// Landscape".
//
// Exactness: E2M1 x E4M3 has at most 6 significant bits in [2^-10, 2688], so
// the scaled operand is exact in FP16, and an FP16 x FP16 product is exact in
// FP32.  Codes are decoded in registers (hardware FP4->FP16 conversion, packed
// FP16 multiply by the block scale) and feed v_mfma_f32_16x16x32_f16 with FP32
// accumulation.  Narrower MFMA inputs (FP8, or the E8M0-scaled FP4 MFMA) cannot
// hold these products exactly.
//
// K permutation (both operands): a K step is 256 values; lane group g (lanes
// 16g..16g+15) owns the range [64g, 64g+64) of the step and MFMA sub-step s
// (0..7) takes its 8 values [8s, 8s+8).  The sum over K is order-free.
//
// Row chunks: rows of expert e are processed in chunks of MC = 16*MT rows; a
// workgroup prologue maps its chunk index to (expert, first row) from the
// device-side offsets, so per-expert counts never reach the host.  Experts
// with no rows read no weight byte.
//
// Two kernels:
//   stream-K  workgroup = (row chunk, BN output columns); loops over K.  The
//             chunk's A rows (gathered through a_rows) are decoded once per
//             step into LDS (double-buffered); every wave streams its own B
//             rows into registers two steps ahead of the MFMAs.
//   stream-N  for K <= 256 and packed weights: the chunk's whole A is decoded
//             into LDS once, then every wave streams a run of 16-column weight
//             tiles, two tiles ahead of the MFMAs.
//
// Weights can be read row-major or from the packed layout written by
// nvfp4_weight_repack: tile (e, row tile rt of 16 rows, K step st) is 2304
// contiguous bytes, lane l's 32 code bytes at [16l, 16l+16) and
// [1024+16l, 1024+16l+16) and its 4 scale bytes at [2048+4l, 2048+4l+4), zero
// padded past N and K.  A wave-step then reads one contiguous 4.5 KB run with
// non-temporal loads - about 1.4x the HBM rate of the best row-major pattern on
// gfx950, and no masks in the kernel.
#include "nvfp4_internal.h"

namespace nvfp4 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int KSTEP = 256;        // K values per step (and per packed tile)
constexpr int PTILE = 2304;       // bytes of a packed 16 x 256 tile

// ------------------------------------------------------------------ packed layout
size_t packed_weight_bytes(int E, int N, int K) {
  return static_cast<size_t>(E) * ((N + 15) / 16) * ((K + KSTEP - 1) / KSTEP) * PTILE;
}

__global__ __launch_bounds__(256) void k_repack(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                int E, int N, int K, uint8_t* __restrict__ packed,
                                                int64_t total_tiles) {
  const int64_t t = blockIdx.x * 256ll + threadIdx.x;
  const int64_t tile = t >> 6;
  const int lane = static_cast<int>(t & 63);
  if (tile >= total_tiles) return;
  const int nst = (K + KSTEP - 1) / KSTEP;
  const int ntr = (N + 15) / 16;
  const int st = static_cast<int>(tile % nst);
  const int rt = static_cast<int>((tile / nst) % ntr);
  const int e = static_cast<int>(tile / (static_cast<int64_t>(nst) * ntr));
  const int n = 16 * rt + (lane & 15);
  const int g = lane >> 4;
  uint8_t* dst = packed + tile * PTILE;
  const bool row_ok = n < N;
  const size_t row = static_cast<size_t>(e) * N + (row_ok ? n : 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = KSTEP * st + 64 * g + 32 * h;   // K % 32 == 0: a 32-value half is all in or all out
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row_ok && k < K) v = *reinterpret_cast<const u32x4*>(codes + row * (K / 2) + k / 2);
    *reinterpret_cast<u32x4*>(dst + 1024 * h + 16 * lane) = v;
  }
  uint32_t s = 0u;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int kb = (KSTEP * st + 64 * g) / 16 + b;
    if (row_ok && kb * 16 < K) s |= static_cast<uint32_t>(scales[row * (K / 16) + kb]) << (8 * b);
  }
  *reinterpret_cast<uint32_t*>(dst + 2048 + 4 * lane) = s;
}

hipError_t launch_repack(const uint8_t* codes, const uint8_t* scales, int E, int N, int K, uint8_t* packed,
                         hipStream_t stream) {
  const int64_t tiles = static_cast<int64_t>(E) * ((N + 15) / 16) * ((K + KSTEP - 1) / KSTEP);
  const int64_t threads = tiles * 64;
  hipLaunchKernelGGL(k_repack, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, stream, codes,
                     scales, E, N, K, packed, tiles);
  return hipGetLastError();
}

// ------------------------------------------------------------------ chunk map
// Map this workgroup's row-chunk index to (expert, first row of the chunk).
// Chunks are enumerated expert by expert: expert e owns ceil(Me/MC) chunks.
// Every thread takes part (block-wide scan of the per-expert chunk counts);
// returns false when the index lies past the last chunk.
template <int THREADS, int MC>
__device__ __forceinline__ bool find_chunk(const GemmParams& p, int chunk, int& e_out, int& m0_out,
                                           int* s_part, int* s_work) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int NWAVE = THREADS / 64;
  if (tid == 0) s_work[0] = -1;
  int base = 0;
  for (int e0 = 0; e0 < p.E; e0 += THREADS) {
    const int e = e0 + tid;
    int c = 0;
    if (e < p.E) {
      const int a = min(max(p.offsets[e], 0), p.m_total);
      const int b = min(max(p.offsets[e + 1], 0), p.m_total);
      c = b > a ? (b - a + MC - 1) / MC : 0;
    }
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    if (lane == 63) s_part[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      const int v = s_part[w];
      before += (w < wave) ? v : 0;
      total += v;
    }
    incl += before;
    const int excl = incl - c;
    if (c > 0 && chunk >= base + excl && chunk < base + incl) {
      s_work[0] = e;
      s_work[1] = (chunk - base - excl) * MC;
    }
    base += total;
    __syncthreads();
  }
  e_out = s_work[0];
  m0_out = s_work[1];
  return e_out >= 0;
}

// ------------------------------------------------------------------ A operand
// A rows (activations, row-major NVFP4) staged by this thread: pair pi ->
// (row ar = (pi & 15) + 16 (pi >> 6), K group ag = (pi >> 4) & 3); the decoded
// fragments of the pair go to LDS slot [(pi >> 6)][sub-step][pi & 63].
template <int PPT>
struct AState {
  const uint8_t* row_code[PPT];    // start of the A row (always a valid row)
  const uint8_t* row_scale[PPT];
  bool ok[PPT];
  int ag[PPT];
};

template <int PPT>
struct ARegs {
  u32x4 c[PPT][2];
  uint32_t s[PPT][2];
};

template <int THREADS, int MT, int PPT>
__device__ __forceinline__ void a_setup(const GemmParams& p, int row0, int m0, int rows, AState<PPT>& A) {
  const size_t krow = static_cast<size_t>(p.K) / 2;
  const size_t srow = static_cast<size_t>(p.K) / 16;
#pragma unroll
  for (int q = 0; q < PPT; ++q) {
    const int pi = threadIdx.x + q * THREADS;
    const int ag = (pi >> 4) & 3;
    const int ar = (pi & 15) + 16 * (pi >> 6);
    A.ok[q] = pi < MT * 64 && ar < rows;
    int arow = row0 + m0 + (A.ok[q] ? ar : 0);
    if (p.a_rows) arow = p.a_rows[arow];
    arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
    A.row_code[q] = p.a_codes + static_cast<size_t>(arow) * krow;
    A.row_scale[q] = p.a_scales + static_cast<size_t>(arow) * srow;
    A.ag[q] = ag;
  }
}

// Loads are unconditional from always-valid addresses (each 32-K half is
// clamped into its row) so the compiler can keep steps in flight; a half past
// K, or a row that does not exist, gets a zero block scale where it is used,
// which zeroes all its decoded values.  Activation rows are re-read by the
// column tiles of a chunk, so they use ordinary (L2-allocating) loads.
__device__ __forceinline__ int clamp_k(int k, int K) { return min(k, K - 32); }

template <int PPT>
__device__ __forceinline__ void a_load(const AState<PPT>& A, ARegs<PPT>& R, int k0, int K) {
#pragma unroll
  for (int q = 0; q < PPT; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = clamp_k(k0 + 64 * A.ag[q] + 32 * h, K);
      R.c[q][h] = *reinterpret_cast<const u32x4*>(A.row_code[q] + kk / 2);
      R.s[q][h] = *reinterpret_cast<const uint16_t*>(A.row_scale[q] + kk / 16);
    }
}

// decode the thread's pairs of one K step into LDS (fragment slots of row tiles < MTA)
template <int THREADS, int MT, int MTA, int PPT>
__device__ __forceinline__ void a_store(const AState<PPT>& A, const ARegs<PPT>& R, int k0, int K,
                                        half8* __restrict__ lds) {
#pragma unroll
  for (int q = 0; q < PPT; ++q) {
    const int pi = threadIdx.x + q * THREADS;
    if (pi < MT * 64 && (pi >> 6) < MTA) {
      half8* dst = lds + (pi >> 6) * 8 * 64 + (pi & 63);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // a zero block scale zeroes every decoded value of the block, so masking
        // the scale alone removes rows and K ranges that do not belong here
        const bool ok = A.ok[q] && (k0 + 64 * A.ag[q] + 32 * h) < K;
        const uint32_t as = ok ? R.s[q][h] : 0u;
        const _Float16 s0 = e4m3_to_f16_div256(as);
        const _Float16 s1 = e4m3_to_f16_div256(as >> 8);
        const u32x4 c = R.c[q][h];
        dst[(4 * h + 0) * 64] = decode8_f16(c.x, s0);
        dst[(4 * h + 1) * 64] = decode8_f16(c.y, s0);
        dst[(4 * h + 2) * 64] = decode8_f16(c.z, s1);
        dst[(4 * h + 3) * 64] = decode8_f16(c.w, s1);
      }
    }
  }
}

// ------------------------------------------------------------------ B operand
// One 16-column B tile of one K step, as held by a lane: 8 code dwords (dword
// d covers the lane's K values [8d, 8d+8)) and the 4 scale bytes of its 64 K.
struct BRegs {
  u32x4 c[2];
  uint32_t s;
};

__device__ __forceinline__ uint32_t word_of(const BRegs& b, int d) {
  const u32x4& x = b.c[d >> 2];
  const int i = d & 3;
  return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
}

__device__ __forceinline__ half8 b_frag(const BRegs& b, uint32_t scale4, int d) {
  return decode8_f16(word_of(b, d), e4m3_to_f16_div256(scale4 >> (8 * (d >> 1))));
}

// packed tile: contiguous, zero padded, streamed with non-temporal loads
__device__ __forceinline__ void b_load_packed(const uint8_t* tile, BRegs& b) {
  const int lane = threadIdx.x & 63;
  b.c[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tile + 16 * lane));
  b.c[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tile + 1024 + 16 * lane));
  b.s = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(tile + 2048 + 4 * lane));
}

// row-major B row (always a valid row): 32 code bytes and 4 scale bytes of the
// lane's K range, each 32-K half clamped into the row; the caller zeroes the
// scale bytes of halves past K
__device__ __forceinline__ void b_load_rows(const uint8_t* row_code, const uint8_t* row_scale, int lg, int k0,
                                            int K, BRegs& b) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kk = clamp_k(k0 + 64 * lg + 32 * h, K);
    b.c[h] = *reinterpret_cast<const u32x4*>(row_code + kk / 2);
  }
  const int k_lo = clamp_k(k0 + 64 * lg, K);
  const int k_hi = clamp_k(k0 + 64 * lg + 32, K);
  b.s = static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(row_scale + k_lo / 16)) |
        (static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(row_scale + k_hi / 16)) << 16);
}

// ------------------------------------------------------------------ epilogues
// Lane (lr = lane & 15, lg = lane >> 4) holds rows 4 lg + i (i < 4) of each
// 16-row tile in column lr of the 16-column tile.
template <int EPI>
__device__ __forceinline__ void epilogue_tile(const GemmParams& p, const float4v& acc, int prow0, int rows_left,
                                              int col, bool col_ok, float gab) {
  const int lg = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * lg + i;
    if (m >= rows_left || !col_ok) continue;
    const size_t prow = static_cast<size_t>(prow0 + m);
    const float y = acc[i] * gab;
    if constexpr (EPI == EPI_F32) {
      static_cast<float*>(p.out)[prow * p.N + col] = y;
    } else if constexpr (EPI == EPI_BF16) {
      static_cast<uint16_t*>(p.out)[prow * p.N + col] = f32_to_bf16(y);
    } else if constexpr (EPI == EPI_COMBINE) {
      const int tk = p.row_token[prow];
      if (tk >= 0 && tk < p.out_rows)
        unsafeAtomicAdd(static_cast<float*>(p.out) + static_cast<size_t>(tk) * p.N + col, p.row_weight[prow] * y);
    }
  }
}

// SwiGLU + NVFP4 re-quantisation of one 16-row tile: gate and up accumulators
// of the same h column; a 16-column h block lives in the 16 lanes of a group.
__device__ __forceinline__ void epilogue_swiglu(const GemmParams& p, const float4v& gate_acc,
                                                const float4v& up_acc, int prow0, int rows_left, int hc,
                                                bool hc_ok, float gab) {
  const int lr = threadIdx.x & 15;
  const int lg = (threadIdx.x & 63) >> 4;
  const int I = p.N / 2;
  const float gh = p.out_g[0];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * lg + i;
    const float h = silu_f32(gate_acc[i] * gab) * (up_acc[i] * gab);
    float amax = fabsf(h);
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    amax = fmaxf(amax, __shfl_xor(amax, 8));
    const uint32_t s = f32_to_e4m3_sat((amax / 6.0f) / gh);
    const float scale_eff = e4m3_to_f32(s) * gh;
    const uint32_t code = encode_one(h, s, scale_eff);
    const uint32_t other = __shfl_xor(code, 1);
    if (m < rows_left && hc_ok) {
      const size_t prow = static_cast<size_t>(prow0 + m);
      if ((lr & 1) == 0) p.out_codes[prow * (I / 2) + hc / 2] = static_cast<uint8_t>(code | (other << 4));
      if (lr == 0) p.out_scales[prow * (I / 16) + hc / 16] = static_cast<uint8_t>(s);
    }
  }
}

// ================================================================== stream-K
template <int WN, int PPT>
struct KCtx {
  AState<PPT> A;
  const uint8_t* b_code[WN];     // row-major: B row start; packed: first tile of the column tile
  const uint8_t* b_scale[WN];
  bool bok[WN];
  int K;
  int nsteps;
};

template <int WN, int PPT>
struct KRegs {
  ARegs<PPT> a;
  BRegs b[WN];
};

template <int WN, int PPT, bool PACKED>
__device__ __forceinline__ void k_load(const KCtx<WN, PPT>& c, KRegs<WN, PPT>& R, int st) {
  a_load(c.A, R.a, st * KSTEP, c.K);
  const int lg = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if constexpr (PACKED)
      b_load_packed(c.b_code[j] + static_cast<size_t>(min(st, c.nsteps - 1)) * PTILE, R.b[j]);
    else
      b_load_rows(c.b_code[j], c.b_scale[j], lg, st * KSTEP, c.K, R.b[j]);
  }
}

template <int NW, int WN, int MT, int MTA, int PPT, bool PACKED>
__device__ __forceinline__ void k_consume(const KCtx<WN, PPT>& c, const KRegs<WN, PPT>& R, int st,
                                          half8* __restrict__ lds, float4v (&acc)[MT][WN]) {
  const int lane = threadIdx.x & 63;
  const int lg = lane >> 4;
  const int k0 = st * KSTEP;
  a_store<NW * 64, MT, MTA, PPT>(c.A, R.a, k0, c.K, lds);
  uint32_t bs[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if constexpr (PACKED) {
      bs[j] = (st < c.nsteps) ? R.b[j].s : 0u;     // packed tiles are zero padded past N and K
    } else {
      const bool lo = c.bok[j] && (k0 + 64 * lg) < c.K;
      const bool hi = c.bok[j] && (k0 + 64 * lg + 32) < c.K;
      bs[j] = (lo ? (R.b[j].s & 0xFFFFu) : 0u) | (hi ? (R.b[j].s & 0xFFFF0000u) : 0u);
    }
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    half8 af[MTA];
#pragma unroll
    for (int r = 0; r < MTA; ++r) af[r] = lds[(r * 8 + s) * 64 + lane];
    half8 bf[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) bf[j] = b_frag(R.b[j], bs[j], s);
#pragma unroll
    for (int r = 0; r < MTA; ++r)
#pragma unroll
      for (int j = 0; j < WN; ++j)
        acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[r], bf[j], acc[r][j], 0, 0, 0);
  }
}

// Software-pipelined K loop: two register sets alternate, so the loads of
// step s+2 are in flight while step s computes (no register copies, which
// would force a wait on the outstanding loads).  The body has no branches: a
// step past K (odd step counts, and the prefetches after the last step) reads
// valid clamped addresses and its data is masked to zero, which keeps the wait
// counts exact.
template <int NW, int WN, int MT, int MTA, int PPT, bool PACKED>
__device__ __forceinline__ void k_main_loop(const KCtx<WN, PPT>& c, half8* __restrict__ lds0,
                                            half8* __restrict__ lds1, float4v (&acc)[MT][WN]) {
  KRegs<WN, PPT> R0, R1;
  k_load<WN, PPT, PACKED>(c, R0, 0);
  k_load<WN, PPT, PACKED>(c, R1, 1);
  for (int st = 0; st < c.nsteps; st += 2) {
    k_consume<NW, WN, MT, MTA, PPT, PACKED>(c, R0, st, lds0, acc);
    k_load<WN, PPT, PACKED>(c, R0, st + 2);
    k_consume<NW, WN, MT, MTA, PPT, PACKED>(c, R1, st + 1, lds1, acc);
    k_load<WN, PPT, PACKED>(c, R1, st + 3);
  }
}

template <int NW, int WN, int MT, int EPI, bool PACKED>
__global__ __launch_bounds__(NW * 64) void k_gemm_streamk(const GemmParams p) {
  constexpr int THREADS = NW * 64;
  constexpr int MC = MT * 16;
  constexpr int BN = NW * WN * 16;
  constexpr int PPT = (MT * 64 + THREADS - 1) / THREADS;   // A (row, K group) pairs per thread
  static_assert(EPI != EPI_SWIGLU || (WN % 2) == 0, "SwiGLU pairs gate and up tiles");
  static_assert(MT >= 1 && MT <= 4, "row tiles per chunk");
  __shared__ half8 a_lds[2][MT * 8 * 64];   // double-buffered [row tile][sub-step][lane] fragments
  __shared__ int s_part[NW];
  __shared__ int s_work[2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15;

  const int task = xcd_task(blockIdx.x, gridDim.x);
  const int chunk = task / p.n_tiles;
  const int nt = task - chunk * p.n_tiles;
  int e, m0;
  if (!find_chunk<THREADS, MC>(p, chunk, e, m0, s_part, s_work)) return;
  // data-dependent bounds are clamped so that inconsistent offsets can give
  // wrong rows but never an access outside the buffers
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  const int rows = min(MC, Me - m0);      // valid rows of this chunk (>= 1)
  const int mt_active = (rows + 15) >> 4;

  const int N = p.N;
  const int I = N / 2;
  KCtx<WN, PPT> c;
  c.K = p.K;
  c.nsteps = (p.K + KSTEP - 1) / KSTEP;
  int col0[WN];     // first column of each 16-column tile of this wave
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int HALF = WN / 2;
      const int hc0 = nt * (BN / 2) + wave * HALF * 16 + (j % HALF) * 16;
      c.bok[j] = hc0 + lr < I;
      col0[j] = (j < HALF) ? hc0 : I + hc0;
    } else {
      col0[j] = nt * BN + wave * WN * 16 + j * 16;
      c.bok[j] = col0[j] + lr < N;
    }
    if constexpr (PACKED) {
      const int ntr = (N + 15) / 16;
      const int rt = min(col0[j] / 16, ntr - 1);
      c.b_code[j] = p.b_packed + (static_cast<size_t>(e) * ntr + rt) * c.nsteps * PTILE;
      c.b_scale[j] = nullptr;
    } else {
      const size_t brow = static_cast<size_t>(e) * N + (c.bok[j] ? col0[j] + lr : 0);
      c.b_code[j] = p.b_codes + brow * (static_cast<size_t>(p.K) / 2);
      c.b_scale[j] = p.b_scales + brow * (static_cast<size_t>(p.K) / 16);
    }
  }
  a_setup<THREADS, MT, PPT>(p, row0, m0, rows, c.A);
  const float gab = p.a_g[0] * p.b_g[e];

  float4v acc[MT][WN];
#pragma unroll
  for (int r = 0; r < MT; ++r)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[r][j] = float4v{0.f, 0.f, 0.f, 0.f};

  switch (mt_active) {
    case 1: k_main_loop<NW, WN, MT, 1, PPT, PACKED>(c, a_lds[0], a_lds[1], acc); break;
    case 2: if constexpr (MT >= 2) k_main_loop<NW, WN, MT, 2, PPT, PACKED>(c, a_lds[0], a_lds[1], acc); break;
    case 3: if constexpr (MT >= 3) k_main_loop<NW, WN, MT, 3, PPT, PACKED>(c, a_lds[0], a_lds[1], acc); break;
    default: if constexpr (MT >= 4) k_main_loop<NW, WN, MT, MT, PPT, PACKED>(c, a_lds[0], a_lds[1], acc); break;
  }

  const int prow0 = row0 + m0;
#pragma unroll
  for (int r = 0; r < MT; ++r) {
    if (r >= mt_active) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int HALF = WN / 2;
#pragma unroll
      for (int jj = 0; jj < HALF; ++jj)
        epilogue_swiglu(p, acc[r][jj], acc[r][jj + HALF], prow0 + 16 * r, rows - 16 * r, col0[jj] + lr, c.bok[jj],
                        gab);
    } else {
#pragma unroll
      for (int j = 0; j < WN; ++j)
        epilogue_tile<EPI>(p, acc[r][j], prow0 + 16 * r, rows - 16 * r, col0[j] + lr, c.bok[j], gab);
    }
  }
}

// ================================================================== stream-N
// K <= 256 (one packed tile per 16 columns) and packed weights.  Workgroup =
// (row chunk, group of NW * UPW units of 64 columns).  The chunk's A is
// decoded into LDS once; wave w then streams its units (4 weight tiles each),
// with the next unit's loads in flight.  Float32 / bf16 results go through a
// per-wave LDS tile so that each row's 64 columns leave as whole 128- or
// 256-byte segments (16 bytes per lane) instead of 2- or 4-byte scattered
// stores.
constexpr int UNIT = 4;   // 16-column tiles per unit

template <int EPI>
__device__ __forceinline__ void store_unit(const GemmParams& p, const float4v (&acc)[UNIT], float* __restrict__ stage,
                                           int prow0, int rows_left, int col0, float gab) {
  // stage[16 rows][64 cols] float32 of this wave; lane (lr, lg) holds rows 4lg+i, cols 16u+lr
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
#pragma unroll
  for (int u = 0; u < UNIT; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) stage[(4 * lg + i) * 68 + 16 * u + lr] = acc[u][i] * gab;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // lane -> (row lane / 4, 16 columns starting at 16 * (lane % 4))
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

template <int NW, int MT, int MTA, int UPW, int EPI>
__device__ __forceinline__ void n_main_loop(const GemmParams& p, const half8* __restrict__ lds, float* stage,
                                            const uint8_t* tiles, int u_first, int u_count, int ntr, int prow0,
                                            int rows, float gab) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15;
  BRegs R0[UNIT], R1[UNIT];
  auto load_unit = [&](BRegs (&R)[UNIT], int i) {
    const int ui = u_first + min(i, u_count - 1);
#pragma unroll
    for (int t = 0; t < UNIT; ++t)
      b_load_packed(tiles + static_cast<size_t>(min(UNIT * ui + t, ntr - 1)) * PTILE, R[t]);
  };
  auto consume = [&](const BRegs (&R)[UNIT], int i) {
    float4v acc[MTA][UNIT];
#pragma unroll
    for (int r = 0; r < MTA; ++r)
#pragma unroll
      for (int t = 0; t < UNIT; ++t) acc[r][t] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8 bf[UNIT];
#pragma unroll
      for (int t = 0; t < UNIT; ++t) bf[t] = b_frag(R[t], R[t].s, s);
#pragma unroll
      for (int r = 0; r < MTA; ++r) {
        const half8 af = lds[(r * 8 + s) * 64 + lane];
#pragma unroll
        for (int t = 0; t < UNIT; ++t) acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[t], acc[r][t], 0, 0, 0);
      }
    }
    if (i < u_count) {
      const int col0 = 64 * (u_first + i);
#pragma unroll
      for (int r = 0; r < MTA; ++r) {
        if constexpr (EPI == EPI_F32 || EPI == EPI_BF16) {
          store_unit<EPI>(p, acc[r], stage, prow0 + 16 * r, rows - 16 * r, col0, gab);
        } else {
#pragma unroll
          for (int t = 0; t < UNIT; ++t)
            epilogue_tile<EPI>(p, acc[r][t], prow0 + 16 * r, rows - 16 * r, col0 + 16 * t + lr,
                               col0 + 16 * t + lr < p.N, gab);
        }
      }
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

template <int NW, int MT, int UPW, int EPI>
__global__ __launch_bounds__(NW * 64) void k_gemm_streamn(const GemmParams p) {
  constexpr int THREADS = NW * 64;
  constexpr int MC = MT * 16;
  constexpr int PPT = (MT * 64 + THREADS - 1) / THREADS;
  static_assert(UPW % 2 == 0, "units per wave come in pairs");
  __shared__ half8 a_lds[MT * 8 * 64];
  __shared__ float stage_lds[NW][16 * 68];   // per-wave output staging (row pitch 68 floats)
  __shared__ int s_part[NW];
  __shared__ int s_work[2];

  const int wave = threadIdx.x >> 6;
  const int task = xcd_task(blockIdx.x, gridDim.x);
  const int chunk = task / p.n_tiles;
  const int ng = task - chunk * p.n_tiles;
  int e, m0;
  if (!find_chunk<THREADS, MC>(p, chunk, e, m0, s_part, s_work)) return;
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  const int rows = min(MC, Me - m0);
  const int mt_active = (rows + 15) >> 4;

  // stage the whole A chunk (one K step) in LDS
  AState<PPT> A;
  a_setup<THREADS, MT, PPT>(p, row0, m0, rows, A);
  ARegs<PPT> ra;
  a_load(A, ra, 0, p.K);
  a_store<THREADS, MT, MT, PPT>(A, ra, 0, p.K, a_lds);
  __syncthreads();

  const int ntr = (p.N + 15) / 16;
  const int nunits = (ntr + UNIT - 1) / UNIT;
  const int u_first = (ng * NW + wave) * UPW;
  const int u_count = min(UPW, nunits - u_first);
  if (u_count <= 0) return;
  const uint8_t* tiles = p.b_packed + static_cast<size_t>(e) * ntr * PTILE;
  const float gab = p.a_g[0] * p.b_g[e];
  const int prow0 = row0 + m0;
  float* stage = stage_lds[wave];
  switch (mt_active) {
    case 1: n_main_loop<NW, MT, 1, UPW, EPI>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
    case 2: if constexpr (MT >= 2) n_main_loop<NW, MT, 2, UPW, EPI>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
    case 3: if constexpr (MT >= 3) n_main_loop<NW, MT, 3, UPW, EPI>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
    default: if constexpr (MT >= 4) n_main_loop<NW, MT, MT, UPW, EPI>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
  }
}

// ------------------------------------------------------------------ launchers
static hipError_t grid_check(int64_t blocks) {
  return blocks >= (int64_t(1) << 31) ? hipErrorInvalidConfiguration : hipSuccess;
}

template <int NW, int WN, int MT, int EPI, bool PACKED>
static hipError_t launch_streamk(GemmParams prm, int64_t m_total, hipStream_t stream) {
  constexpr int BN = NW * WN * 16;
  constexpr int MC = MT * 16;
  const int cols = (EPI == EPI_SWIGLU) ? prm.N / 2 : prm.N;
  const int cols_per_tile = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  prm.n_tiles = (cols + cols_per_tile - 1) / cols_per_tile;
  // sum over experts of ceil(Me / MC) <= m_total / MC + E
  const int64_t blocks = ((m_total + MC - 1) / MC + prm.E) * prm.n_tiles;
  if (grid_check(blocks) != hipSuccess) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_gemm_streamk<NW, WN, MT, EPI, PACKED>), dim3(static_cast<unsigned>(blocks)), dim3(NW * 64),
                     0, stream, prm);
  return hipGetLastError();
}

template <int NW, int MT, int UPW, int EPI>
static hipError_t launch_streamn(GemmParams prm, int64_t m_total, hipStream_t stream) {
  constexpr int MC = MT * 16;
  const int nunits = ((prm.N + 15) / 16 + UNIT - 1) / UNIT;
  prm.n_tiles = (nunits + NW * UPW - 1) / (NW * UPW);     // column-unit groups per chunk
  const int64_t blocks = ((m_total + MC - 1) / MC + prm.E) * prm.n_tiles;
  if (grid_check(blocks) != hipSuccess) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_gemm_streamn<NW, MT, UPW, EPI>), dim3(static_cast<unsigned>(blocks)), dim3(NW * 64), 0,
                     stream, prm);
  return hipGetLastError();
}

template <bool PACKED>
static hipError_t launch_k(const GemmParams& prm, int epilogue, int64_t m_total, hipStream_t stream) {
  switch (epilogue) {
    case EPI_F32: return launch_streamk<4, 2, 4, EPI_F32, PACKED>(prm, m_total, stream);
    case EPI_BF16: return launch_streamk<4, 2, 4, EPI_BF16, PACKED>(prm, m_total, stream);
    case EPI_SWIGLU: return launch_streamk<4, 2, 4, EPI_SWIGLU, PACKED>(prm, m_total, stream);
    case EPI_COMBINE: return launch_streamk<4, 2, 4, EPI_COMBINE, PACKED>(prm, m_total, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_grouped_gemm(const GemmParams& prm, int epilogue, int64_t m_total, int hint, hipStream_t stream) {
  (void)hint;
  if (prm.b_packed && prm.K <= KSTEP && epilogue != EPI_SWIGLU) {
    switch (epilogue) {
      case EPI_F32: return launch_streamn<4, 4, 6, EPI_F32>(prm, m_total, stream);
      case EPI_BF16: return launch_streamn<4, 4, 6, EPI_BF16>(prm, m_total, stream);
      case EPI_COMBINE: return launch_streamn<4, 4, 6, EPI_COMBINE>(prm, m_total, stream);
      default: return hipErrorInvalidValue;
    }
  }
  return prm.b_packed ? launch_k<true>(prm, epilogue, m_total, stream) : launch_k<false>(prm, epilogue, m_total, stream);
}

}  // namespace nvfp4
