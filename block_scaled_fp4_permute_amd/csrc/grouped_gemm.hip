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
#include "gemm_device.h"


namespace nvfp4 {

// ------------------------------------------------------------------ packed layout
size_t packed_weight_bytes(int E, int N, int K) {
  return static_cast<size_t>(E) * ((int64_t(N) + 15) / 16) * ((int64_t(K) + KSTEP - 1) / KSTEP) * PTILE;
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

// ------------------------------------------------------------------ launchers
// compute units of the current device (the runtime's cached device
// properties; 256, MI355X's count, if the query fails)
static int compute_units() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 256;
  return v;
}

static hipError_t grid_check(int64_t blocks) {
  return blocks >= (int64_t(1) << 31) ? hipErrorInvalidConfiguration : hipSuccess;
}

template <int NW, int WN, int MT, int EPI, int PACKED, int LIGHT, int MINB = 2>
static hipError_t launch_streamk(GemmParams prm, int64_t m_total, hipStream_t stream) {
  constexpr int BN = NW * WN * 16;
  constexpr int MC = MT * 16;
  const int cols = (EPI == EPI_SWIGLU) ? prm.N / 2 : prm.N;
  const int cols_per_tile = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  prm.n_tiles = (cols + cols_per_tile - 1) / cols_per_tile;
  // sum over experts of ceil(Me / MC) <= m_total / MC + E chunks, each of at
  // most n_tiles tasks (2 * n_tiles when light chunks split); a multiple of 8
  // for the XCD task map
  const int64_t per_chunk = static_cast<int64_t>(prm.n_tiles) * (LIGHT > 0 ? 2 : 1);
  prm.slots = MINB * compute_units();
  const int64_t blocks = ((((m_total + MC - 1) / MC + prm.E) * per_chunk) + 7) / 8 * 8;
  if (grid_check(blocks) != hipSuccess) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_gemm_streamk<NW, WN, MT, EPI, PACKED, MINB, LIGHT>), dim3(static_cast<unsigned>(blocks)),
                     dim3(NW * 64), 0, stream, prm);
  return hipGetLastError();
}

template <int NW, int MT, int UPW, int EPI, int PACKED>
static hipError_t launch_streamn(GemmParams prm, int64_t m_total, hipStream_t stream) {
  constexpr int MC = MT * 16;
  const int nunits = ((prm.N + 15) / 16 + UNIT - 1) / UNIT;
  prm.n_tiles = (nunits + NW * UPW - 1) / (NW * UPW);     // column-unit groups per chunk
  const int64_t blocks = ((((m_total + MC - 1) / MC + prm.E) * prm.n_tiles) + 7) / 8 * 8;
  if (grid_check(blocks) != hipSuccess) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_gemm_streamn<NW, MT, UPW, EPI, PACKED>), dim3(static_cast<unsigned>(blocks)), dim3(NW * 64), 0,
                     stream, prm);
  return hipGetLastError();
}

// Two tile shapes for the stream-K kernel:
//   decode  (few rows per expert): 4 waves, 64-row chunks; SwiGLU tiles of
//           256 columns (waves of 2 gate + 2 up tiles), other epilogues 128;
//   large-M (>= kLargeRows rows per expert): 8 waves, 128-row chunks, 256
//           columns - each weight tile then serves twice the rows, which pays
//           off once the MFMA work dominates.
constexpr int kLargeRows = 128;

#ifndef LIGHT_CLASS
#define LIGHT_CLASS 1
#endif
// decode tile, packed weights: last chunks of at most this many live row tiles split
constexpr int kLightPacked = LIGHT_CLASS;

template <int PACKED, bool LARGE>
static hipError_t launch_k(const GemmParams& prm, int epilogue, int64_t m_total, hipStream_t stream) {
  // row-major weights (not the streaming layout) keep whole-width tasks: the
  // second task shape would make them spill registers
  constexpr int kLight = PACKED == kRowB ? 0 : kLightPacked;
  switch (epilogue) {
    case EPI_F32:
      return LARGE ? launch_streamk<8, 2, 8, EPI_F32, PACKED, 0, 1>(prm, m_total, stream)
                   : launch_streamk<4, 2, 4, EPI_F32, PACKED, kLight>(prm, m_total, stream);
    case EPI_BF16:
      return LARGE ? launch_streamk<8, 2, 8, EPI_BF16, PACKED, 0, 1>(prm, m_total, stream)
                   : launch_streamk<4, 2, 4, EPI_BF16, PACKED, kLight>(prm, m_total, stream);
    case EPI_SWIGLU:
      return LARGE ? launch_streamk<8, 2, 8, EPI_SWIGLU, PACKED, 0, 1>(prm, m_total, stream)
                   : launch_streamk<4, 4, 4, EPI_SWIGLU, PACKED, kLight>(prm, m_total, stream);
    case EPI_COMBINE:
      return LARGE ? launch_streamk<8, 2, 8, EPI_COMBINE, PACKED, 0, 1>(prm, m_total, stream)
                   : launch_streamk<4, 2, 4, EPI_COMBINE, PACKED, kLight>(prm, m_total, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int UPW>
static hipError_t launch_dn(const GemmParams& prm, int epilogue, bool cached, int64_t m_total, hipStream_t stream) {
  switch (epilogue) {
    case EPI_F32:
      return cached ? launch_streamn<4, 4, UPW, EPI_F32, kPackedCached>(prm, m_total, stream)
                    : launch_streamn<4, 4, UPW, EPI_F32, kPackedNT>(prm, m_total, stream);
    case EPI_BF16:
      return cached ? launch_streamn<4, 4, UPW, EPI_BF16, kPackedCached>(prm, m_total, stream)
                    : launch_streamn<4, 4, UPW, EPI_BF16, kPackedNT>(prm, m_total, stream);
    case EPI_COMBINE:
      return cached ? launch_streamn<4, 4, UPW, EPI_COMBINE, kPackedCached>(prm, m_total, stream)
                    : launch_streamn<4, 4, UPW, EPI_COMBINE, kPackedNT>(prm, m_total, stream);
    default: return hipErrorInvalidValue;
  }
}

// Weight loads are cached (not non-temporal) once the experts average a full
// 64-row chunk: their row chunks then re-read the same tiles, side by side on
// one XCD, and share them in its L2.  Decode MoE with T=2048, top-8 of 256
// experts (64 rows per expert on average, Zipf-skewed): HBM reads of gate_up
// 673 -> 609 MB and of down 364 -> 250 MB; the combine then finds less of
// the down output in the last-level cache, but the layer is still faster.
// Experts of a few rows read their tiles once, and non-temporal loads keep
// them from evicting anything.
#ifndef CACHE_ROWS
#define CACHE_ROWS 64
#endif

hipError_t launch_grouped_gemm(const GemmParams& prm, int epilogue, int64_t m_total, int hint, hipStream_t stream) {
  // rows per expert: the caller's hint, else the average (the counts stay on
  // the device)
  const int64_t rows_per_expert = hint > 0 ? hint : m_total / prm.E;
  const bool large = rows_per_expert >= kLargeRows;
  if (prm.b_packed && prm.K <= KSTEP && epilogue != EPI_SWIGLU) {
    // units of 64 columns per wave: 8 at large M (T=16384 prefill, 512 rows
    // per expert: down 586 -> 558 µs), 6 below (T=256 decode, 8 rows per
    // expert: 57 µs against 60 with 8)
    const bool cached = rows_per_expert >= CACHE_ROWS;
    return large ? launch_dn<8>(prm, epilogue, cached, m_total, stream)
                 : launch_dn<6>(prm, epilogue, cached, m_total, stream);
  }
  // from 256 rows per expert (packed weights, K a multiple of the step): the
  // 256 x 256 tile with both operands staged in LDS
  if (gemm_large_fits(prm, rows_per_expert)) return launch_gemm_large(prm, epilogue, m_total, stream);
  const int mode = !prm.b_packed ? kRowB : rows_per_expert >= CACHE_ROWS ? kPackedCached : kPackedNT;
  switch (mode) {
    case kRowB:
      return large ? launch_k<kRowB, true>(prm, epilogue, m_total, stream)
                   : launch_k<kRowB, false>(prm, epilogue, m_total, stream);
    case kPackedNT:
      return large ? launch_k<kPackedNT, true>(prm, epilogue, m_total, stream)
                   : launch_k<kPackedNT, false>(prm, epilogue, m_total, stream);
    default:
      return large ? launch_k<kPackedCached, true>(prm, epilogue, m_total, stream)
                   : launch_k<kPackedCached, false>(prm, epilogue, m_total, stream);
  }
}

}  // namespace nvfp4
