// Grouped NVFP4 GEMM for gfx950 with fused epilogues.
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
// FP32.  The kernel therefore decodes codes in registers (hardware FP4->FP16
// conversion, packed FP16 multiply by the block scale) and feeds
// v_mfma_f32_16x16x32_f16 with FP32 accumulation.  Narrower MFMA inputs (FP8,
// or the E8M0-scaled FP4 MFMA) cannot hold these products exactly.
//
// Work decomposition (one workgroup = NW waves):
//   blockIdx.x -> (expert e, tile of BN = NW*WN*16 output columns), remapped so
//                each XCD gets a contiguous range of tasks (same expert -> same L2);
//   blockIdx.y -> row chunks of MC = MT*16 rows of the expert, strided by gridDim.y.
// Each wave owns WN 16-column B tiles and all MC rows of the chunk.  Per K step
// of 128: the A rows (gathered through a_rows) are decoded once into LDS in MFMA
// fragment order; every lane streams 16 bytes of codes + 2 scale bytes of each
// of its B rows straight from HBM into registers (a row's 64 bytes per step come
// from 4 consecutive lane groups), decodes them and issues MT*WN MFMAs per
// 32-K sub-step.  The sum over K is order-free, so lane group g takes the K
// range [32g, 32g+32) of the step and sub-step s its 8 values [8s, 8s+8) - the
// same permutation on both operands.
// Experts with no rows exit before reading any weight byte.
#include "nvfp4_internal.h"

namespace nvfp4 {

template <int NW, int WN, int MT, int EPI>
__global__ __launch_bounds__(NW * 64) void k_gemm_nvfp4(const GemmParams p) {
  constexpr int THREADS = NW * 64;
  constexpr int MC = MT * 16;
  constexpr int KS = 128;
  constexpr int BN = NW * WN * 16;
  static_assert(EPI != EPI_SWIGLU || (WN % 2) == 0, "SwiGLU pairs gate and up tiles");
  __shared__ half8 a_lds[MT * 4 * 64];   // [row tile][sub-step][lane] fragments, MT * 4 KiB

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 15;   // B column / A row inside a 16-wide tile
  const int lg = lane >> 4;   // K group of the lane

  const int task = xcd_task(blockIdx.x, gridDim.x);
  const int e = task / p.n_tiles;
  const int nt = task - e * p.n_tiles;
  // data-dependent bounds are clamped so that inconsistent offsets can give
  // wrong rows but never an access outside the buffers
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(p.offsets[e + 1], p.m_total) - row0;
  const int nchunks = (Me + MC - 1) / MC;
  if (static_cast<int>(blockIdx.y) >= nchunks) return;

  const int N = p.N;
  const int K = p.K;
  const int I = N / 2;
  const size_t krow = static_cast<size_t>(K) / 2;   // code bytes per row
  const size_t srow = static_cast<size_t>(K) / 16;  // scale bytes per row

  int bcol[WN];
  bool bok[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int HALF = WN / 2;
      const int jj = j % HALF;
      const int hc = nt * (BN / 2) + wave * HALF * 16 + jj * 16 + lr;
      bok[j] = hc < I;
      bcol[j] = (j < HALF) ? hc : I + hc;
    } else {
      bcol[j] = nt * BN + wave * WN * 16 + j * 16 + lr;
      bok[j] = bcol[j] < N;
    }
  }
  const uint8_t* bcode[WN];
  const uint8_t* bscale[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const size_t brow = static_cast<size_t>(e) * N + (bok[j] ? bcol[j] : 0);
    bcode[j] = p.b_codes + brow * krow + 16 * lg;
    bscale[j] = p.b_scales + brow * srow + 2 * lg;
  }
  const float gab = p.a_g[0] * p.b_g[e];

  for (int mc = blockIdx.y; mc < nchunks; mc += gridDim.y) {
    const int m0 = mc * MC;
    float4v acc[MT][WN];
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[r][j] = float4v{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < K; k0 += KS) {
      // ---- stage the A rows of this K step into LDS, decoded to FP16
      __syncthreads();
      for (int pi = tid; pi < MT * 64; pi += THREADS) {
        const int ag = (pi >> 4) & 3;
        const int ar = (pi & 15) + 16 * (pi >> 6);
        const int m = m0 + ar;
        const int kg = k0 + 32 * ag;
        uint4 c = make_uint4(0u, 0u, 0u, 0u);
        uint32_t sc = 0u;
        if (m < Me && kg < K) {
          int arow = p.a_rows ? p.a_rows[row0 + m] : row0 + m;
          arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
          c = *reinterpret_cast<const uint4*>(p.a_codes + static_cast<size_t>(arow) * krow + kg / 2);
          sc = *reinterpret_cast<const uint16_t*>(p.a_scales + static_cast<size_t>(arow) * srow + kg / 16);
        }
        const _Float16 s0 = e4m3_to_f16(sc & 0xFFu);
        const _Float16 s1 = e4m3_to_f16(sc >> 8);
        half8* dst = a_lds + (ar >> 4) * 4 * 64 + (pi & 63);
        dst[0 * 64] = decode8_f16(c.x, s0);
        dst[1 * 64] = decode8_f16(c.y, s0);
        dst[2 * 64] = decode8_f16(c.z, s1);
        dst[3 * 64] = decode8_f16(c.w, s1);
      }
      __syncthreads();

      // ---- B rows of this lane: 16 code bytes + 2 scale bytes each
      uint4 bc[WN];
      uint32_t bs[WN];
      const bool kin = (k0 + 32 * lg) < K;
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        if (bok[j] && kin) {
          bc[j] = *reinterpret_cast<const uint4*>(bcode[j] + k0 / 2);
          bs[j] = *reinterpret_cast<const uint16_t*>(bscale[j] + k0 / 16);
        } else {
          bc[j] = make_uint4(0u, 0u, 0u, 0u);
          bs[j] = 0u;
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        half8 bf[WN];
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const uint32_t w = s == 0 ? bc[j].x : s == 1 ? bc[j].y : s == 2 ? bc[j].z : bc[j].w;
          bf[j] = decode8_f16(w, e4m3_to_f16((bs[j] >> (8 * (s >> 1))) & 0xFFu));
        }
#pragma unroll
        for (int r = 0; r < MT; ++r) {
          const half8 af = a_lds[(r * 4 + s) * 64 + lane];
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[r][j], 0, 0, 0);
        }
      }
    }

    // ---- epilogue: lane holds rows 4*lg + i of each 16-row tile, column lr
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int HALF = WN / 2;
      const float gh = p.out_g[0];
#pragma unroll
      for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int jj = 0; jj < HALF; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = m0 + r * 16 + 4 * lg + i;
            const float gate = acc[r][jj][i] * gab;
            const float up = acc[r][jj + HALF][i] * gab;
            const float h = silu_f32(gate) * up;
            float amax = fabsf(h);
            amax = fmaxf(amax, __shfl_xor(amax, 1));
            amax = fmaxf(amax, __shfl_xor(amax, 2));
            amax = fmaxf(amax, __shfl_xor(amax, 4));
            amax = fmaxf(amax, __shfl_xor(amax, 8));
            const uint32_t s = f32_to_e4m3_sat((amax / 6.0f) / gh);
            const float scale_eff = e4m3_to_f32(s) * gh;
            const uint32_t code = encode_one(h, s, scale_eff);
            const uint32_t other = __shfl_xor(code, 1);
            const int hc = bcol[jj];
            if (m < Me && bok[jj]) {
              const size_t prow = static_cast<size_t>(row0 + m);
              if ((lr & 1) == 0) p.out_codes[prow * (I / 2) + hc / 2] = static_cast<uint8_t>(code | (other << 4));
              if (lr == 0) p.out_scales[prow * (I / 16) + hc / 16] = static_cast<uint8_t>(s);
            }
          }
    } else {
#pragma unroll
      for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + r * 16 + 4 * lg + i;
          if (m >= Me) continue;
          const size_t prow = static_cast<size_t>(row0 + m);
          if constexpr (EPI == EPI_COMBINE) {
            const int tk = p.row_token[prow];
            const size_t tok = static_cast<size_t>(tk);
            const float w = p.row_weight[prow];
#pragma unroll
            for (int j = 0; j < WN; ++j)
              if (bok[j] && tk >= 0 && tk < p.out_rows) unsafeAtomicAdd(static_cast<float*>(p.out) + tok * N + bcol[j], w * (acc[r][j][i] * gab));
          } else {
#pragma unroll
            for (int j = 0; j < WN; ++j) {
              if (!bok[j]) continue;
              const float y = acc[r][j][i] * gab;
              if constexpr (EPI == EPI_F32)
                static_cast<float*>(p.out)[prow * N + bcol[j]] = y;
              else
                static_cast<uint16_t*>(p.out)[prow * N + bcol[j]] = f32_to_bf16(y);
            }
          }
        }
    }
  }
}

// ------------------------------------------------------------------ launcher
template <int NW, int WN, int MT, int EPI>
static hipError_t launch_cfg(GemmParams prm, int64_t m_total, int hint, hipStream_t stream) {
  constexpr int BN = NW * WN * 16;
  constexpr int MC = MT * 16;
  const int cols = (EPI == EPI_SWIGLU) ? prm.N / 2 : prm.N;
  const int cols_per_tile = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  prm.n_tiles = (cols + cols_per_tile - 1) / cols_per_tile;
  int64_t rows_guess = hint > 0 ? hint : (m_total + prm.E - 1) / prm.E;
  int64_t slots = (rows_guess + MC - 1) / MC;
  if (slots < 1) slots = 1;
  if (slots > 64) slots = 64;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(prm.E) * prm.n_tiles), static_cast<unsigned>(slots));
  hipLaunchKernelGGL((k_gemm_nvfp4<NW, WN, MT, EPI>), grid, dim3(NW * 64), 0, stream, prm);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmParams& prm, int epilogue, int64_t m_total, int hint, hipStream_t stream) {
  switch (epilogue) {
    case EPI_F32: return launch_cfg<4, 1, 4, EPI_F32>(prm, m_total, hint, stream);
    case EPI_BF16: return launch_cfg<4, 1, 4, EPI_BF16>(prm, m_total, hint, stream);
    case EPI_SWIGLU: return launch_cfg<4, 2, 4, EPI_SWIGLU>(prm, m_total, hint, stream);
    case EPI_COMBINE: return launch_cfg<4, 1, 4, EPI_COMBINE>(prm, m_total, hint, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4
