// Large-M tile of the grouped NVFP4 GEMM (from 256 rows per expert, packed
// weights, K a multiple of 256): the regime the pages measure on very large
// matrices, where the matrix cores and not the weight stream bound the GEMM
// ("The Critical Search: Uncovering SM120 CUTLASS Collective
// Implementations", section "Context: The Optimization Journey").
//
// A workgroup of 8 waves computes 256 rows x 256 columns (SwiGLU: 128 gate +
// 128 up); wave w = 4 wr + wc holds rows [128 wr, +128) and four 16-column
// tiles (4 wc.., or gate tiles 2 wc, 2 wc + 1 and the matching up tiles).
// Both operands pass through LDS once per workgroup:
//   weights      the step's 16 packed tiles (2304 bytes each) copied verbatim;
//                every wave decodes its own four tiles' fragments from there
//                (E2M1 -> FP16 times the E4M3 block scale, exact)
//   activations  decoded once per workgroup to FP16 fragments, a quarter step
//                at a time (64 of the 256 K values: sub-steps 2q, 2q + 1 of
//                the lane layout, one 16-value block per lane group)
// A 256-K step runs as 4 quarters.  Quarter q's MFMAs read the FP16 buffer
// q % 2 while the workgroup decodes quarter q + 1 into the other; the next
// step's weight tiles are in flight during quarters 0-1 and stored into the
// idle weight stage, its activation codes during quarters 2-3.  Each FP16 A
// fragment read from LDS feeds 4 MFMAs and each decoded weight fragment 8;
// the 128-row tile (8 waves of 128 rows x 32 columns) feeds 2 MFMAs per A
// fragment, so here the activation bytes read from LDS per MFMA halve.
#include "gemm_device.h"

namespace nvfp4 {

constexpr int kLRows = 256;
constexpr int kLThreads = 512;
constexpr int kLBStage = 16 * PTILE;                  // one step's 16 packed weight tiles
constexpr int kLAQuarter = 16 * 2 * 64 * 16;          // [row tile][sub-step of the quarter][lane] of half8
constexpr int kLLds = 2 * kLBStage + 2 * kLAQuarter;

// the thread's activation codes and scales of one step: row t / 2, lane
// groups 2 (t & 1) and 2 (t & 1) + 1 (code bytes [64 (t & 1), +64) and scale
// bytes [8 (t & 1), +8) of the row's step)
struct LRawA {
  u32x4 c[4];
  uint32_t s[2];
};

// half H of the thread's share of the step's weight tiles: two 16-byte code
// pieces (pieces t + 512 i, i = 2H, 2H + 1, of the 16 x 2048 code bytes: tile
// t / 128 + 4 i, bytes 16 (t % 128)) and, with H = 0, 8 scale bytes (tile
// t / 32, bytes 2048 + 8 (t % 32))
struct LRawB {
  u32x4 c[2];
  uint2 s;
};

struct LSrc {
  rsrc_t ra, rs;          // activation codes and scales (range-checked)
  uint32_t va, vs;        // byte offsets of the thread's codes and scales at step 0
  const uint8_t* bt[4];   // step 0 of the packed tile holding piece i (uniform in a wave)
  const uint8_t* bts;     // step 0 of the tile holding the thread's scale bytes
  uint32_t lb0;           // LDS offset of piece 0 in a weight stage (piece i: + 4 i tiles)
  uint32_t lbs;           // of the scale bytes
};

__device__ __forceinline__ void l_load_a(const LSrc& S, LRawA& R, int st) {
  const uint32_t oc = S.va + static_cast<uint32_t>(st) * (KSTEP / 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    R.c[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(S.ra, oc + 16u * i, 0, 0));
  const uint32_t os = S.vs + static_cast<uint32_t>(st) * (KSTEP / 16);
  R.s[0] = __builtin_amdgcn_raw_buffer_load_b32(S.rs, os, 0, 0);
  R.s[1] = __builtin_amdgcn_raw_buffer_load_b32(S.rs, os + 4u, 0, 0);
}

template <int H>
__device__ __forceinline__ void l_load_b(const LSrc& S, LRawB& R, int st) {
  const size_t ot = static_cast<size_t>(st) * PTILE;
  const int off = 16 * (threadIdx.x & 127);
#pragma unroll
  for (int i = 0; i < 2; ++i) R.c[i] = *reinterpret_cast<const u32x4*>(S.bt[2 * H + i] + ot + off);
  if constexpr (H == 0) R.s = *reinterpret_cast<const uint2*>(S.bts + ot);
}

template <int H>
__device__ __forceinline__ void l_store_b(const LSrc& S, const LRawB& R, uint8_t* __restrict__ stage) {
#pragma unroll
  for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(stage + S.lb0 + 4 * PTILE * (2 * H + i)) = R.c[i];
  if constexpr (H == 0) *reinterpret_cast<uint2*>(stage + S.lbs) = R.s;
}

// decode quarter Q of the thread's activation codes into an FP16 buffer:
// lane group lg = 2 (t & 1) + c, dwords 2Q and 2Q + 1 of its 8 (K values
// [64 lg + 16 Q, +16): one block), to sub-steps 0 and 1 of the quarter
template <int Q>
__device__ __forceinline__ void l_decode_a(const LRawA& R, half8* __restrict__ abuf) {
  const int t = threadIdx.x;
  const int row = t >> 1;
  const int rt = row >> 4, lr = row & 15;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int lg = 2 * (t & 1) + c;
    const u32x4 w = R.c[2 * c + (Q >> 1)];
    const uint32_t w0 = (Q & 1) ? w.z : w.x;
    const uint32_t w1 = (Q & 1) ? w.w : w.y;
    const _Float16 sc = e4m3_to_f16_div256(R.s[c] >> (8 * Q));
    // lane (lg, lr) sits at slot 16 lg + (lr ^ 4 (lg >> 1)): the 8 threads of
    // a store (4 rows, lane groups c and 2 + c) then hit distinct banks
    const int slot = 16 * lg + (lr ^ ((lg & 2) << 1));
    abuf[(rt * 2 + 0) * 64 + slot] = decode8_f16(w0, sc);
    abuf[(rt * 2 + 1) * 64 + slot] = decode8_f16(w1, sc);
  }
}

// the MFMAs of quarter Q: weight dwords 2Q, 2Q + 1 of each of the wave's
// tiles (bq: the lane's dwords 0-3 for quarters 0-1, 4-7 for quarters 2-3;
// scale byte Q), activation fragments from abuf (lane l at slot
// l ^ ((l >> 3) & 4), the store swizzle)
template <int Q>
__device__ __forceinline__ void l_quarter(const half8* __restrict__ abuf, const u32x4 (&bq)[4],
                                          const uint32_t (&bsw)[4], int wr, float4v (&acc)[8][4]) {
  const int lane = threadIdx.x & 63;
  const int slot = lane ^ ((lane >> 3) & 4);
  _Float16 bsc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bsc[j] = e4m3_to_f16_div256(bsw[j] >> (8 * Q));
#pragma unroll
  for (int sp = 0; sp < 2; ++sp) {
    half8 bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = sp == 0 ? ((Q & 1) ? bq[j].z : bq[j].x) : ((Q & 1) ? bq[j].w : bq[j].y);
      bf[j] = decode8_f16(w, bsc[j]);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const half8 af = abuf[((8 * wr + r) * 2 + sp) * 64 + slot];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[r][j], 0, 0, 0);
    }
    // keep the second sub-step's weight decode behind the first one's MFMAs
    // (decoding both up front holds 16 more registers than the tile has)
    if (sp == 0) __builtin_amdgcn_sched_barrier(0);
  }
}

template <int EPI>
__global__ __launch_bounds__(kLThreads, 1) void k_gemm_l(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLLds];
  static_assert(fits_lds(sizeof(lds), 1), "large-M staging exceeds the LDS of a CU");
  int e, m0, nt;
  bool narrow;
  if (!find_task<16, false, 0>(p, e, m0, nt, narrow)) return;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = wave >> 2, wc = wave & 3;
  const int lr = lane & 15;
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  // inside an expert, groups of 4 row chunks run column tile by column tile,
  // so that the workgroups side by side on an XCD share A chunks and weight
  // tiles in its L2
  {
    const int nc = (Me + kLRows - 1) / kLRows;
    const int u = (m0 / kLRows) * p.n_tiles + nt;
    const int grp = (m0 / kLRows) / 4;
    const int gq = min(4, nc - 4 * grp);
    const int w = u - 4 * grp * p.n_tiles;
    m0 = (4 * grp + w % gq) * kLRows;
    nt = w / gq;
  }
  const int rows = min(kLRows, Me - m0);
  const int N = p.N, K = p.K;
  const int nsteps = K / KSTEP;
  const int ntr = N / 16;

  LSrc S;
  {
    const uint32_t krow = static_cast<uint32_t>(K) / 2, srow = static_cast<uint32_t>(K) / 16;
    S.ra = make_rsrc(p.a_codes, static_cast<uint32_t>(p.a_rows_total) * krow);
    S.rs = make_rsrc(p.a_scales, static_cast<uint32_t>(p.a_rows_total) * srow);
    const int ar = t >> 1;
    int arow = row0 + m0 + (ar < rows ? ar : 0);
    if (p.a_rows) arow = p.a_rows[arow];
    arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
    S.va = static_cast<uint32_t>(arow) * krow + 64u * (t & 1);
    S.vs = static_cast<uint32_t>(arow) * srow + 8u * (t & 1);
    const uint8_t* b = p.b_packed + static_cast<size_t>(e) * ntr * nsteps * PTILE;
    auto tile_of = [&](int j) {     // packed column tile held in weight-stage tile j
      int rt;
      if constexpr (EPI == EPI_SWIGLU)
        rt = j < 8 ? nt * 8 + j : (N / 32) + nt * 8 + (j - 8);
      else
        rt = nt * 16 + j;
      return static_cast<size_t>(min(rt, ntr - 1));
    };
    // piece t + 512 i lies in stage tile t / 128 + 4 i = wave / 2 + 4 i
#pragma unroll
    for (int i = 0; i < 4; ++i) S.bt[i] = b + tile_of((wave >> 1) + 4 * i) * nsteps * PTILE;
    S.bts = b + tile_of(t >> 5) * nsteps * PTILE + 2048 + 8 * (t & 31);
    S.lb0 = (wave >> 1) * PTILE + 16u * (t & 127);
    S.lbs = (t >> 5) * PTILE + 2048u + 8u * (t & 31);
  }
  int jt[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (EPI == EPI_SWIGLU)
      jt[j] = (j < 2 ? 0 : 8) + 2 * wc + (j & 1);
    else
      jt[j] = 4 * wc + j;
  }
  uint8_t* bst0 = lds;
  uint8_t* bst1 = lds + kLBStage;
  half8* abuf0 = reinterpret_cast<half8*>(lds + 2 * kLBStage);
  half8* abuf1 = reinterpret_cast<half8*>(lds + 2 * kLBStage + kLAQuarter);

  float4v acc[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[r][j] = float4v{0.f, 0.f, 0.f, 0.f};

  LRawA ra;
  LRawB rb;
  l_load_a(S, ra, 0);
  l_load_b<0>(S, rb, 0);
  l_store_b<0>(S, rb, bst0);
  l_load_b<1>(S, rb, 0);
  l_store_b<1>(S, rb, bst0);
  l_decode_a<0>(ra, abuf0);
  __syncthreads();
  // No branches: the last step re-stages itself into the idle buffers, which
  // nothing reads afterwards.
  for (int st = 0; st < nsteps; ++st) {
    const uint8_t* bcur = (st & 1) ? bst1 : bst0;
    uint8_t* bnxt = (st & 1) ? bst0 : bst1;
    const int sn = min(st + 1, nsteps - 1);
    uint32_t bsw[4];
    u32x4 bq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bsw[j] = *reinterpret_cast<const uint32_t*>(bcur + jt[j] * PTILE + 2048 + 4 * lane);
      bq[j] = *reinterpret_cast<const u32x4*>(bcur + jt[j] * PTILE + 16 * lane);
    }
    l_load_b<0>(S, rb, sn);
    l_quarter<0>(abuf0, bq, bsw, wr, acc);
    l_decode_a<1>(ra, abuf1);
    __syncthreads();
    l_quarter<1>(abuf1, bq, bsw, wr, acc);
    l_store_b<0>(S, rb, bnxt);
    l_load_b<1>(S, rb, sn);
    l_decode_a<2>(ra, abuf0);
#pragma unroll
    for (int j = 0; j < 4; ++j) bq[j] = *reinterpret_cast<const u32x4*>(bcur + jt[j] * PTILE + 1024 + 16 * lane);
    __syncthreads();
    l_quarter<2>(abuf0, bq, bsw, wr, acc);
    l_store_b<1>(S, rb, bnxt);
    l_decode_a<3>(ra, abuf1);
    l_load_a(S, ra, sn);
    __syncthreads();
    l_quarter<3>(abuf1, bq, bsw, wr, acc);
    l_decode_a<0>(ra, abuf0);
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
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int hc = nt * 128 + 32 * wc + 16 * jj + lr;
        epilogue_swiglu<false>(p, acc[r][jj], acc[r][2 + jj], prow0 + 16 * rt, left, hc, hc < N / 2, gab);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = nt * 256 + 64 * wc + 16 * j + lr;
        epilogue_tile<EPI>(p, acc[r][j], prow0 + 16 * rt, left, col, col < N, gab);
      }
    }
  }
}

template <int EPI>
static hipError_t launch_l(GemmParams prm, int64_t m_total, hipStream_t stream) {
  const int cols = (EPI == EPI_SWIGLU) ? prm.N / 2 : prm.N;
  const int per = (EPI == EPI_SWIGLU) ? 128 : 256;
  prm.n_tiles = (cols + per - 1) / per;
  prm.slots = 1 << 30;
  const int64_t blocks = ((((m_total + kLRows - 1) / kLRows + prm.E) * prm.n_tiles) + 7) / 8 * 8;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_gemm_l<EPI>), dim3(static_cast<unsigned>(blocks)), dim3(kLThreads), 0, stream, prm);
  return hipGetLastError();
}

bool gemm_large_fits(const GemmParams& prm, int64_t rows_per_expert) {
  return prm.b_packed && prm.K % KSTEP == 0 && prm.N % 16 == 0 && rows_per_expert >= kLRows;
}

hipError_t launch_gemm_large(const GemmParams& prm, int epilogue, int64_t m_total, hipStream_t stream) {
  switch (epilogue) {
    case EPI_F32: return launch_l<EPI_F32>(prm, m_total, stream);
    case EPI_BF16: return launch_l<EPI_BF16>(prm, m_total, stream);
    case EPI_SWIGLU: return launch_l<EPI_SWIGLU>(prm, m_total, stream);
    case EPI_COMBINE: return launch_l<EPI_COMBINE>(prm, m_total, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4
