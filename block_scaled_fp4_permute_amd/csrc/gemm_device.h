// Device code of the grouped NVFP4 GEMM for gfx950: the task map, the
// activation (A) and weight (B) operand pipelines, the epilogues and the two
// task bodies (stream-K and stream-N), shared by the grouped GEMM launchers
// and the persistent expert-FFN launch.  What the GEMM computes and how the
// operands are laid out is described at the top of grouped_gemm.hip.
#pragma once

#include "nvfp4_internal.h"

namespace nvfp4 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int KSTEP = 256;        // K values per step (and per packed tile)
constexpr int PTILE = 2304;       // bytes of a packed 16 x 256 tile

// ------------------------------------------------------------------ task map
// A task is (row chunk, column tile).  Chunks are enumerated expert by expert
// (expert e owns ceil(Me/MC) of them, all full but maybe the last) and tasks
// chunk by chunk, so the tasks of an expert are contiguous.  The class of a
// task is the number of live 16-row tiles of its chunk (1..MT); its cost grows
// with the class.
//
// The hardware hands workgroups to the 8 XCDs round-robin (workgroup i to XCD
// i % 8).  Each XCD gets an equal, contiguous range of the tasks that exist,
// so the column tiles of a chunk and the chunks of an expert share one L2.
// BY_CLASS: inside its range an XCD runs the tasks heaviest class first (task
// order within a class): longest-first list scheduling, which keeps the full
// chunks out of the last round of workgroups.  Otherwise in task order, so
// that the chunks of an expert run side by side and share its weight tiles in
// L2.
//
// Every wave computes the map on its own, from one read of the expert offsets
// (4 experts per lane) and wave shuffles only: no LDS and no barrier before a
// workgroup's first loads.  Experts beyond 256 are taken in further groups of
// 256.  Needs a grid of at least 8 * ceil(tasks / 8) workgroups.
constexpr int kExpPerLane = 4;
constexpr int kExpGroup = 64 * kExpPerLane;

// rows of expert e (0 past the last expert); data-dependent bounds are clamped
// so that inconsistent offsets give wrong rows, never an access out of bounds
__device__ __forceinline__ int expert_rows(const GemmParams& p, int e) {
  if (e >= p.E) return 0;
  const int a = min(max(p.offsets[e], 0), p.m_total);
  const int b = min(max(p.offsets[e + 1], 0), p.m_total);
  return max(b - a, 0);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// exclusive prefix sum over the 64 lanes; total: the sum of all lanes
__device__ __forceinline__ int wave_excl_scan(int v, int& total) {
  const int lane = threadIdx.x & 63;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  total = __shfl(incl, 63);
  return incl - v;
}

__device__ __forceinline__ int overlap(int a0, int a1, int b0, int b1) { return max(0, min(a1, b1) - max(a0, b0)); }

// experts g0 + 4 lane + i of one group: rows, chunks, first task, tasks
template <int MC>
struct ExpGroup {
  int Me[kExpPerLane];
  int c[kExpPerLane];
  int tb[kExpPerLane];
  int nt[kExpPerLane];
  int total;            // tasks of the whole group
};

// live 16-row tiles of the last chunk of an expert with Me rows in c chunks
template <int MC>
__device__ __forceinline__ int last_class(int Me, int c) { return (Me - (c - 1) * MC + 15) >> 4; }

// column tasks of the last chunk of an expert: twice as many (half as wide)
// when its class is at most `light`
template <int MC>
__device__ __forceinline__ int last_tasks(int Me, int c, int ntl, int light) {
  return last_class<MC>(Me, c) <= light ? 2 * ntl : ntl;
}

// rows and chunks of the group's experts
template <int MC>
__device__ __forceinline__ void load_group(const GemmParams& p, int g0, ExpGroup<MC>& G) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kExpPerLane; ++i) {
    G.Me[i] = expert_rows(p, g0 + kExpPerLane * lane + i);
    G.c[i] = (G.Me[i] + MC - 1) / MC;
  }
}

// tasks of the group's experts and their first task, from task `base` on
template <int MC>
__device__ __forceinline__ void assign_tasks(int ntl, int light, int base, ExpGroup<MC>& G) {
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kExpPerLane; ++i) {
    G.nt[i] = G.c[i] > 0 ? (G.c[i] - 1) * ntl + last_tasks<MC>(G.Me[i], G.c[i], ntl, light) : 0;
    sum += G.nt[i];
  }
  int run = base + wave_excl_scan(sum, G.total);
#pragma unroll
  for (int i = 0; i < kExpPerLane; ++i) {
    G.tb[i] = run;
    run += G.nt[i];
  }
}

// (expert, first row of the chunk, column tile, narrow) of workgroup
// blockIdx.x; false (uniformly) when it has no task.  A chunk has n_tiles
// column tasks, or 2 * n_tiles half-width ("narrow") ones when it is the last
// chunk of its expert and has at most LIGHT live row tiles (LIGHT = 0: never).
// Light chunks split only when the whole-width tasks outnumber the resident
// workgroups: the light tasks then run in a last round that would leave
// workgroup slots empty; otherwise splitting only adds work.
template <int MT, bool BY_CLASS, int LIGHT>
__device__ __forceinline__ bool find_task(const GemmParams& p, int& e_out, int& m0_out, int& nt_out,
                                          bool& narrow_out) {
  constexpr int MC = MT * 16;
  static_assert(LIGHT < MT, "full chunks are never narrow");
  const int ntl = p.n_tiles;
  const int lane = threadIdx.x & 63;
  ExpGroup<MC> G0;
  load_group<MC>(p, 0, G0);
  assign_tasks<MC>(ntl, 0, 0, G0);
  int n = G0.total;
  for (int g0 = kExpGroup; g0 < p.E; g0 += kExpGroup) {
    ExpGroup<MC> G;
    load_group<MC>(p, g0, G);
    assign_tasks<MC>(ntl, 0, n, G);
    n += G.total;
  }
  const int light = (LIGHT > 0 && n > p.slots) ? LIGHT : 0;
  if (light > 0) {
    assign_tasks<MC>(ntl, light, 0, G0);
    n = G0.total;
    for (int g0 = kExpGroup; g0 < p.E; g0 += kExpGroup) {
      ExpGroup<MC> G;
      load_group<MC>(p, g0, G);
      assign_tasks<MC>(ntl, light, n, G);
      n += G.total;
    }
  }
  const int per = (n + 7) >> 3;
  const int lo = (blockIdx.x & 7) * per;
  const int hi = min(lo + per, n);
  const int j = blockIdx.x >> 3;
  if (lo + j >= hi) return false;

  // the class k and rank r of this workgroup's task among the class-k tasks
  // of [lo, hi); the tasks of an expert's full chunks are class MT, those of
  // its last chunk [t1, t1 + nl) have the class of that chunk
  int k = MT, r = j;
  if constexpr (BY_CLASS) {
    int cnt[MT + 1];
#pragma unroll
    for (int q = 0; q <= MT; ++q) cnt[q] = 0;
    int base = 0;
    for (int g0 = 0; g0 < p.E && base < hi; g0 += kExpGroup) {
      ExpGroup<MC> G;
      if (g0 == 0) {
        G = G0;
      } else {
        load_group<MC>(p, g0, G);
        assign_tasks<MC>(ntl, light, base, G);
      }
#pragma unroll
      for (int i = 0; i < kExpPerLane; ++i) {
        if (G.c[i] > 0) {
          const int cl = last_class<MC>(G.Me[i], G.c[i]);
          const int t1 = G.tb[i] + (G.c[i] - 1) * ntl;
          cnt[MT] += overlap(G.tb[i], t1, lo, hi);
          const int nl = overlap(t1, G.tb[i] + G.nt[i], lo, hi);
#pragma unroll
          for (int q = 1; q <= MT; ++q) cnt[q] += (q == cl) ? nl : 0;
        }
      }
      base += G.total;
    }
#pragma unroll
    for (int q = 1; q <= MT; ++q) cnt[q] = wave_sum(cnt[q]);
#pragma unroll
    for (int q = MT; q >= 2; --q) {
      if (k == q && r >= cnt[q]) {
        r -= cnt[q];
        k = q - 1;
      }
    }
  }

  // find the r-th class-k task of [lo, hi) in task order (without classes:
  // task lo + j); exactly one lane holds it
  const int t_plain = lo + j;
  int f_t = -1, f_e = 0, f_m0 = 0, f_nt = 0, f_narrow = 0;
  auto take = [&](const ExpGroup<MC>& G, int i, int g0, int t) {
    const int t1 = G.tb[i] + (G.c[i] - 1) * ntl;
    f_t = t;
    f_e = g0 + kExpPerLane * lane + i;
    if (t < t1) {
      const int q = (t - G.tb[i]) / ntl;
      f_m0 = q * MC;
      f_nt = t - G.tb[i] - q * ntl;
      f_narrow = 0;
    } else {
      f_m0 = (G.c[i] - 1) * MC;
      f_nt = t - t1;
      f_narrow = (G.nt[i] - (t1 - G.tb[i])) > ntl ? 1 : 0;
    }
  };
  int base = 0, before = 0;
  for (int g0 = 0; g0 < p.E && base < hi; g0 += kExpGroup) {
    ExpGroup<MC> G;
    if (g0 == 0) {
      G = G0;
    } else {
      load_group<MC>(p, g0, G);
      assign_tasks<MC>(ntl, light, base, G);
    }
    if constexpr (BY_CLASS) {
      int v[kExpPerLane], tlo[kExpPerLane];
      int vsum = 0;
#pragma unroll
      for (int i = 0; i < kExpPerLane; ++i) {
        v[i] = 0;
        tlo[i] = 0;
        if (G.c[i] > 0) {
          // the class-k tasks of one expert form one interval
          const int cl = last_class<MC>(G.Me[i], G.c[i]);
          const int t1 = G.tb[i] + (G.c[i] - 1) * ntl;
          const int a0 = (k == MT) ? G.tb[i] : t1;
          const int a1 = (cl == k) ? G.tb[i] + G.nt[i] : t1;
          if (a1 > a0) {
            tlo[i] = max(a0, lo);
            v[i] = overlap(a0, a1, lo, hi);
          }
        }
        vsum += v[i];
      }
      int vtotal;
      int vb = before + wave_excl_scan(vsum, vtotal);
#pragma unroll
      for (int i = 0; i < kExpPerLane; ++i) {
        if (v[i] > 0 && r >= vb && r < vb + v[i]) take(G, i, g0, tlo[i] + (r - vb));
        vb += v[i];
      }
      before += vtotal;
    } else {
#pragma unroll
      for (int i = 0; i < kExpPerLane; ++i)
        if (G.nt[i] > 0 && t_plain >= G.tb[i] && t_plain < G.tb[i] + G.nt[i]) take(G, i, g0, t_plain);
    }
    base += G.total;
  }
  const uint64_t found = __ballot(f_t >= 0);
  if (found == 0) return false;
  const int src = __ffsll(static_cast<unsigned long long>(found)) - 1;
  e_out = __shfl(f_e, src);
  m0_out = __shfl(f_m0, src);
  nt_out = __shfl(f_nt, src);
  narrow_out = __shfl(f_narrow, src) != 0;
  return true;
}

// ------------------------------------------------------------------ A operand
// A rows (activations, row-major NVFP4) staged by this thread: pair pi ->
// (row ar = (pi & 15) + 16 (pi >> 6), K group ag = (pi >> 4) & 3); the decoded
// fragments of the pair go to LDS slot [(pi >> 6)][sub-step][pi & 63].
// Buffer resources: loads give zero past the resource's byte count (the
// hardware range check), so reads past the end of a row set or weight block
// need no clamping.  The per-lane offset carries the whole byte offset, which
// is what the range check sees.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRawBufferFlags = 0x00020000;   // resource dword 3 for raw (untyped) buffer access
constexpr int kLoadNT = 2;                    // cache policy: non-temporal
constexpr int kCoherent = 1 | 16;             // cache policy sc0 | sc1: coherent at agent scope
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           kRawBufferFlags);
}

template <int PPT>
struct AState {
  rsrc_t rc, rs;                   // all A codes / all A scales
  uint32_t vc[PPT], vs[PPT];       // byte offsets of the lane's K group in its A row
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
  const uint32_t krow = static_cast<uint32_t>(p.K) / 2;
  const uint32_t srow = static_cast<uint32_t>(p.K) / 16;
  A.rc = make_rsrc(p.a_codes, static_cast<uint32_t>(p.a_rows_total) * krow);
  A.rs = make_rsrc(p.a_scales, static_cast<uint32_t>(p.a_rows_total) * srow);
#pragma unroll
  for (int q = 0; q < PPT; ++q) {
    const int pi = threadIdx.x + q * THREADS;
    const int ag = (pi >> 4) & 3;
    const int ar = (pi & 15) + 16 * (pi >> 6);
    A.ok[q] = pi < MT * 64 && ar < rows;
    int arow = row0 + m0 + (A.ok[q] ? ar : 0);
    if (p.a_rows) arow = p.a_rows[arow];
    arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
    A.vc[q] = static_cast<uint32_t>(arow) * krow + 32u * ag;
    A.vs[q] = static_cast<uint32_t>(arow) * srow + 4u * ag;
    A.ag[q] = ag;
  }
}

// Loads are unconditional (no branch keeps steps in flight with exact wait
// counts); a half past K reads the next row (or zeros past the last row) and
// gets a zero block scale where it is used, which zeroes all its decoded
// values, as does a row that does not exist.  Activation rows are re-read by
// the column tiles of a chunk, so they use ordinary (L2-allocating) loads.
// AUX: cache-policy bits of the loads (0: ordinary; kCoherent: agent-scope
// coherent, for rows another workgroup wrote in the same launch)
template <int PPT, int AUX = 0>
__device__ __forceinline__ void a_load(const AState<PPT>& A, ARegs<PPT>& R, int k0, int K) {
  // steps past K re-read the last step (cached) instead of fetching new bytes
  const uint32_t kq = static_cast<uint32_t>(min(k0, ((K - 1) / KSTEP) * KSTEP));
  const uint32_t kc = kq / 2;
  const uint32_t ks = kq / 16;
#pragma unroll
  for (int q = 0; q < PPT; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      R.c[q][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(A.rc, A.vc[q] + kc + 16u * h, 0, AUX));
      R.s[q][h] = __builtin_amdgcn_raw_buffer_load_b16(A.rs, A.vs[q] + ks + 2u * h, 0, AUX);
    }
}

// decode the thread's pairs of one K step into LDS
template <int THREADS, int MT, int MTA, int PPT>
__device__ __forceinline__ void a_store(const AState<PPT>& A, const ARegs<PPT>& R, int k0, int K,
                                        half8* __restrict__ lds) {
#pragma unroll
  for (int q = 0; q < PPT; ++q) {
    const int pi = threadIdx.x + q * THREADS;
    // compile-time true in the common shapes, so the store stays branch-free;
    // pairs of row tiles >= MTA decode into slots no MFMA reads (zeros: their
    // rows do not exist) rather than branch around the store
    const bool in_chunk = (THREADS * PPT <= MT * 64) || pi < MT * 64;
    if (in_chunk) {
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

// The same decode split into 8 * PPT pieces (pair q, 32-K half h, code dword
// w), so that it can be interleaved with MFMAs: a_scales first turns the
// block scales of the step into (masked) FP16 multipliers.
template <int PPT>
struct AScales {
  _Float16 s[PPT][2][2];
};

template <int PPT>
__device__ __forceinline__ void a_scales(const AState<PPT>& A, const ARegs<PPT>& R, int k0, int K,
                                         AScales<PPT>& S) {
#pragma unroll
  for (int q = 0; q < PPT; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool ok = A.ok[q] && (k0 + 64 * A.ag[q] + 32 * h) < K;
      const uint32_t as = ok ? R.s[q][h] : 0u;
      S.s[q][h][0] = e4m3_to_f16_div256(as);
      S.s[q][h][1] = e4m3_to_f16_div256(as >> 8);
    }
}

template <int THREADS, int MT, int MTA, int PPT>
__device__ __forceinline__ void a_store_piece(const ARegs<PPT>& R, const AScales<PPT>& S, half8* __restrict__ lds,
                                              int piece) {
  const int q = piece >> 3;
  const int h = (piece >> 2) & 1;
  const int w = piece & 3;
  const int pi = threadIdx.x + q * THREADS;
  // no branch on the live row tiles (see a_store): one basic block per K step
  const bool in_chunk = (THREADS * PPT <= MT * 64) || pi < MT * 64;
  if (in_chunk) {
    const u32x4 c = R.c[q][h];
    const uint32_t word = w == 0 ? c.x : w == 1 ? c.y : w == 2 ? c.z : c.w;
    lds[(pi >> 6) * 8 * 64 + (4 * h + w) * 64 + (pi & 63)] = decode8_f16(word, S.s[q][h][w >> 1]);
  }
}

// Activation staging policies of the stream-K loop.  APairs: every thread
// stages PPT (row, K group) pairs, one row tile per wave - used when three or
// more row tiles are live.  AOneTile: only row tile 0 is live (at most 16
// rows); its 16 rows x 4 K groups x 4 word pairs are spread over 256 threads,
// 2 code words (16 values) each, so no wave decodes rows that do not exist.
// ATwoTiles (below the B operand helpers' types): row tiles 0 and 1 live.
// All write the same LDS fragments for the live row tiles.
template <int THREADS, int MT, int PPT>
struct APairs {
  using State = AState<PPT>;
  using Regs = ARegs<PPT>;
  using Scales = AScales<PPT>;
  __device__ static void setup(const GemmParams& p, int row0, int m0, int rows, State& A) {
    a_setup<THREADS, MT, PPT>(p, row0, m0, rows, A);
  }
  __device__ static void load(const State& A, Regs& R, int k0, int K) { a_load(A, R, k0, K); }
  template <int MTA>
  __device__ static void store(const State& A, const Regs& R, int k0, int K, half8* __restrict__ lds) {
    a_store<THREADS, MT, MTA, PPT>(A, R, k0, K, lds);
  }
  __device__ static void scales(const State& A, const Regs& R, int k0, int K, Scales& S) { a_scales(A, R, k0, K, S); }
  // the part of the decode that rides behind MFMA sub-step s (0..7)
  template <int MTA>
  __device__ static void piece(const State&, const Regs& R, const Scales& S, half8* __restrict__ lds, int s) {
#pragma unroll
    for (int q = 0; q < PPT; ++q) a_store_piece<THREADS, MT, MTA, PPT>(R, S, lds, 8 * q + s);
  }
};

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int THREADS, int MT>
struct AOneTile {
  static_assert(THREADS >= 256, "one live row tile needs 256 threads");
  struct State {
    rsrc_t rc, rs;
    uint32_t vc, vs;     // byte offsets of the thread's 8 code bytes / 1 scale byte in step 0
    int kq;              // K offset of its 32-value half within a step
    int slot;            // LDS slot of its first word
    bool ok;
  };
  struct Regs {
    u32x2 c;
    uint32_t s;
  };
  struct Scales {
    _Float16 s;
  };
  __device__ static bool active() { return THREADS == 256 || threadIdx.x < 256; }
  __device__ static void setup(const GemmParams& p, int row0, int m0, int rows, State& A) {
    const uint32_t krow = static_cast<uint32_t>(p.K) / 2;
    const uint32_t srow = static_cast<uint32_t>(p.K) / 16;
    A.rc = make_rsrc(p.a_codes, static_cast<uint32_t>(p.a_rows_total) * krow);
    A.rs = make_rsrc(p.a_scales, static_cast<uint32_t>(p.a_rows_total) * srow);
    const int t = threadIdx.x & 255;
    const int pair = t & 63;            // row (pair & 15), K group (pair >> 4)
    const int ar = pair & 15;
    const int ag = pair >> 4;
    const int h = (t >> 7) & 1;         // 32-value half of the K group
    const int ws = (t >> 6) & 1;        // words 2 ws, 2 ws + 1 of the half
    A.ok = active() && ar < rows;
    int arow = row0 + m0 + (A.ok ? ar : 0);
    if (p.a_rows) arow = p.a_rows[arow];
    arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
    A.vc = static_cast<uint32_t>(arow) * krow + 32u * ag + 16u * h + 8u * ws;
    A.vs = static_cast<uint32_t>(arow) * srow + 4u * ag + 2u * h + ws;
    A.kq = 64 * ag + 32 * h;
    A.slot = (4 * h + 2 * ws) * 64 + pair;
  }
  __device__ static void load(const State& A, Regs& R, int k0, int K) {
    // steps past K re-read the last step (cached) instead of fetching new bytes
    const uint32_t kq = static_cast<uint32_t>(min(k0, ((K - 1) / KSTEP) * KSTEP));
    R.c = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(A.rc, A.vc + kq / 2, 0, 0));
    R.s = __builtin_amdgcn_raw_buffer_load_b8(A.rs, A.vs + kq / 16, 0, 0);
  }
  __device__ static void scales(const State& A, const Regs& R, int k0, int K, Scales& S) {
    // a zero block scale zeroes a row that does not exist and a half past K
    const bool ok = A.ok && (k0 + A.kq) < K;
    S.s = e4m3_to_f16_div256(ok ? R.s : 0u);
  }
  template <int MTA>
  __device__ static void store(const State& A, const Regs& R, int k0, int K, half8* __restrict__ lds) {
    Scales S;
    scales(A, R, k0, K, S);
    if (active()) {
      lds[A.slot] = decode8_f16(R.c.x, S.s);
      lds[A.slot + 64] = decode8_f16(R.c.y, S.s);
    }
  }
  // the two words ride behind MFMA sub-steps 0 and 4
  template <int MTA>
  __device__ static void piece(const State& A, const Regs& R, const Scales& S, half8* __restrict__ lds, int s) {
    if ((s == 0 || s == 4) && active()) lds[A.slot + (s >> 2) * 64] = decode8_f16(s == 0 ? R.c.x : R.c.y, S.s);
  }
};

// ATwoTiles: row tiles 0 and 1 live (17 to 32 rows): their 128 (row, K
// group) pairs x 2 halves are spread over 256 threads, 4 code words each, so
// no wave decodes rows that do not exist (one row tile per wave would leave
// waves 2 and 3 decoding dead rows while waves 0 and 1 decode 8 words each).
template <int THREADS, int MT>
struct ATwoTiles {
  static_assert(THREADS >= 256, "two live row tiles need 256 threads");
  struct State {
    rsrc_t rc, rs;
    uint32_t vc, vs;
    int kq;
    int slot;
    bool ok;
  };
  struct Regs {
    u32x4 c;
    uint32_t s;
  };
  struct Scales {
    _Float16 s[2];
  };
  __device__ static bool active() { return THREADS == 256 || threadIdx.x < 256; }
  __device__ static void setup(const GemmParams& p, int row0, int m0, int rows, State& A) {
    const uint32_t krow = static_cast<uint32_t>(p.K) / 2;
    const uint32_t srow = static_cast<uint32_t>(p.K) / 16;
    A.rc = make_rsrc(p.a_codes, static_cast<uint32_t>(p.a_rows_total) * krow);
    A.rs = make_rsrc(p.a_scales, static_cast<uint32_t>(p.a_rows_total) * srow);
    const int t = threadIdx.x & 255;
    const int pi = t & 127;             // pair: row (pi & 15) + 16 (pi >> 6), K group (pi >> 4) & 3
    const int h = t >> 7;               // 32-value half of the K group
    const int ag = (pi >> 4) & 3;
    const int ar = (pi & 15) + 16 * (pi >> 6);
    A.ok = active() && ar < rows;
    int arow = row0 + m0 + (A.ok ? ar : 0);
    if (p.a_rows) arow = p.a_rows[arow];
    arow = (arow >= 0 && arow < p.a_rows_total) ? arow : 0;
    A.vc = static_cast<uint32_t>(arow) * krow + 32u * ag + 16u * h;
    A.vs = static_cast<uint32_t>(arow) * srow + 4u * ag + 2u * h;
    A.kq = 64 * ag + 32 * h;
    A.slot = (pi >> 6) * 8 * 64 + (4 * h) * 64 + (pi & 63);
  }
  __device__ static void load(const State& A, Regs& R, int k0, int K) {
    // steps past K re-read the last step (cached) instead of fetching new bytes
    const uint32_t kq = static_cast<uint32_t>(min(k0, ((K - 1) / KSTEP) * KSTEP));
    R.c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(A.rc, A.vc + kq / 2, 0, 0));
    R.s = __builtin_amdgcn_raw_buffer_load_b16(A.rs, A.vs + kq / 16, 0, 0);
  }
  __device__ static void scales(const State& A, const Regs& R, int k0, int K, Scales& S) {
    // a zero block scale zeroes a row that does not exist and a half past K
    const bool ok = A.ok && (k0 + A.kq) < K;
    const uint32_t as = ok ? R.s : 0u;
    S.s[0] = e4m3_to_f16_div256(as);
    S.s[1] = e4m3_to_f16_div256(as >> 8);
  }
  template <int MTA>
  __device__ static void store(const State& A, const Regs& R, int k0, int K, half8* __restrict__ lds) {
    Scales S;
    scales(A, R, k0, K, S);
    if (active()) {
      lds[A.slot] = decode8_f16(R.c.x, S.s[0]);
      lds[A.slot + 64] = decode8_f16(R.c.y, S.s[0]);
      lds[A.slot + 128] = decode8_f16(R.c.z, S.s[1]);
      lds[A.slot + 192] = decode8_f16(R.c.w, S.s[1]);
    }
  }
  // the four words ride behind MFMA sub-steps 0, 2, 4, 6
  template <int MTA>
  __device__ static void piece(const State& A, const Regs& R, const Scales& S, half8* __restrict__ lds, int s) {
    if ((s & 1) == 0 && active()) {
      const int w = s >> 1;
      const uint32_t word = w == 0 ? R.c.x : w == 1 ? R.c.y : w == 2 ? R.c.z : R.c.w;
      lds[A.slot + w * 64] = decode8_f16(word, S.s[w >> 1]);
    }
  }
};

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

// packed tile: contiguous, zero padded, global loads (on gfx950 they keep
// more weight bytes in flight than buffer loads of the same tiles).  NT:
// non-temporal, for weights read once; otherwise cached, so that the row
// chunks of one expert, running side by side on one XCD, share the tiles in
// its L2.
template <bool NT>
__device__ __forceinline__ void b_load_packed(const uint8_t* tile, BRegs& b) {
  const int lane = threadIdx.x & 63;
  const u32x4* c = reinterpret_cast<const u32x4*>(tile + 16 * lane);
  const u32x4* d = reinterpret_cast<const u32x4*>(tile + 1024 + 16 * lane);
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(tile + 2048 + 4 * lane);
  if constexpr (NT) {
    b.c[0] = __builtin_nontemporal_load(c);
    b.c[1] = __builtin_nontemporal_load(d);
    b.s = __builtin_nontemporal_load(sc);
  } else {
    b.c[0] = *c;
    b.c[1] = *d;
    b.s = *sc;
  }
}

// How B is laid out and loaded (the PACKED template parameter)
constexpr int kRowB = 0;          // row-major codes and scales
constexpr int kPackedNT = 1;      // packed tiles, non-temporal loads
constexpr int kPackedCached = 2;  // packed tiles, cached loads

__device__ __forceinline__ int clamp_k(int k, int K) { return min(k, K - 32); }

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
// of the same h column; a 16-column h block lives in the 16 lanes of a row,
// lane (lr, lg) holding rows 4 lg + i.  The block scales of the 4 rows a lane
// group holds are computed once: lane lr takes row 4 lg + (lr & 3), and the
// results are broadcast back inside each quad.  The block scale follows the
// quantiser exactly (two correctly rounded divisions); silu and the element
// quotient use reciprocal-based divisions, whose ~2 ulp sit far inside the
// rounding differences h already carries.
// COH: h leaves through agent-scope coherent stores (written through to the
// point of coherence), so that a workgroup of the same launch can read it
template <bool COH>
__device__ __forceinline__ void store_u8(uint8_t* p, uint32_t v) {
  if constexpr (COH)
    __hip_atomic_store(p, static_cast<uint8_t>(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = static_cast<uint8_t>(v);
}

template <bool COH = false>
__device__ __forceinline__ void epilogue_swiglu(const GemmParams& p, const float4v& gate_acc,
                                                const float4v& up_acc, int prow0, int rows_left, int hc,
                                                bool hc_ok, float gab) {
  const int lr = threadIdx.x & 15;
  const int lg = (threadIdx.x & 63) >> 4;
  const int I = p.N / 2;
  const float gh = p.out_g[0];
  float h[4], am[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = silu_fast(gate_acc[i] * gab) * (up_acc[i] * gab);
    am[i] = row16_max(fabsf(h[i]));
  }
  const int q = lr & 3;
  const float amq = q == 0 ? am[0] : q == 1 ? am[1] : q == 2 ? am[2] : am[3];
  const uint32_t sq = f32_to_e4m3_sat((amq / 6.0f) / gh);
  const float seq = e4m3_to_f32(sq) * gh;
  uint32_t s[4];
  float se[4];
  s[0] = dpp_u32<0x00>(sq); se[0] = __uint_as_float(dpp_u32<0x00>(__float_as_uint(seq)));   // quad_perm [0,0,0,0]
  s[1] = dpp_u32<0x55>(sq); se[1] = __uint_as_float(dpp_u32<0x55>(__float_as_uint(seq)));   // quad_perm [1,1,1,1]
  s[2] = dpp_u32<0xAA>(sq); se[2] = __uint_as_float(dpp_u32<0xAA>(__float_as_uint(seq)));   // quad_perm [2,2,2,2]
  s[3] = dpp_u32<0xFF>(sq); se[3] = __uint_as_float(dpp_u32<0xFF>(__float_as_uint(seq)));   // quad_perm [3,3,3,3]
  if (lr < 4 && 4 * lg + lr < rows_left && hc_ok)
    store_u8<COH>(p.out_scales + static_cast<size_t>(prow0 + 4 * lg + lr) * (I / 16) + hc / 16, sq);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * lg + i;
    const float v = (s[i] != 0u && se[i] > 0.0f) ? __fdividef(fabsf(h[i]), se[i]) : 0.0f;
    // a NaN quotient (zero times an infinite reciprocal) encodes as 0 | sign
    const uint32_t code = (s[i] != 0u) ? e2m1_code(__builtin_copysignf(v == v ? v : 0.0f, h[i])) : 0u;
    const uint32_t other = dpp_u32<kDppXor1>(code);
    if (m < rows_left && hc_ok && (lr & 1) == 0)
      store_u8<COH>(p.out_codes + static_cast<size_t>(prow0 + m) * (I / 2) + hc / 2, code | (other << 4));
  }
}

// ================================================================== stream-K
// weights part of a task's context
template <int WN>
struct BCtx {
  const uint8_t* b_code[WN];     // row-major: B row start; packed: first tile of the column tile
  const uint8_t* b_scale[WN];
  bool bok[WN];
  int K;
  int nsteps;
};

// the whole context: weights, and the activation rows as staged by policy AP
template <int WN, class AP>
struct KCtx : BCtx<WN> {
  typename AP::State A;
};

template <int WN, int PACKED>
__device__ __forceinline__ void k_load_b(const BCtx<WN>& c, BRegs (&B)[WN], int st) {
  const int lg = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if constexpr (PACKED)
      b_load_packed<PACKED == kPackedNT>(c.b_code[j] + static_cast<size_t>(min(st, c.nsteps - 1)) * PTILE, B[j]);
    else
      b_load_rows(c.b_code[j], c.b_scale[j], lg, st * KSTEP, c.K, B[j]);
  }
}

// One K step: the MFMAs of step st (A fragments from lds_cur, weights decoded
// from registers), with the decode of step st+1's activation rows into
// lds_nxt interleaved - both in one basic block, so the VALU work of the
// decodes overlaps the matrix-core work - then the step's barrier.
template <int NW, int WN, int MT, int MTA, class AP, int PACKED>
__device__ __forceinline__ void k_step(const KCtx<WN, AP>& c, const typename AP::Regs& a_nxt, const BRegs (&B)[WN],
                                       int st, const half8* __restrict__ lds_cur, half8* __restrict__ lds_nxt,
                                       float4v (&acc)[MT][WN]) {
  const int lane = threadIdx.x & 63;
  const int lg = lane >> 4;
  const int k0 = st * KSTEP;
  uint32_t bs[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if constexpr (PACKED) {
      bs[j] = (st < c.nsteps) ? B[j].s : 0u;     // packed tiles are zero padded past N and K
    } else {
      const bool lo = c.bok[j] && (k0 + 64 * lg) < c.K;
      const bool hi = c.bok[j] && (k0 + 64 * lg + 32) < c.K;
      bs[j] = (lo ? (B[j].s & 0xFFFFu) : 0u) | (hi ? (B[j].s & 0xFFFF0000u) : 0u);
    }
  }
  typename AP::Scales as;
  AP::scales(c.A, a_nxt, k0 + KSTEP, c.K, as);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    half8 af[MTA];
#pragma unroll
    for (int r = 0; r < MTA; ++r) af[r] = lds_cur[(r * 8 + s) * 64 + lane];
    half8 bf[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) bf[j] = b_frag(B[j], bs[j], s);
#pragma unroll
    for (int r = 0; r < MTA; ++r)
#pragma unroll
      for (int j = 0; j < WN; ++j)
        acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[r], bf[j], acc[r][j], 0, 0, 0);
    // a share of the next step's activation decode rides behind these MFMAs
    AP::template piece<MTA>(c.A, a_nxt, as, lds_nxt, s);
  }
  __syncthreads();
}

// Software-pipelined K loop.  Register sets alternate, so the loads of later
// steps are in flight while a step computes, with no register copies (a copy
// would force a wait on the outstanding loads): weights two steps ahead,
// activation rows one to two steps ahead of their decode, which itself runs
// one step ahead of the MFMAs (double-buffered LDS fragments).  The body has
// no branches: a step past K (an odd step count, and the prefetches after the
// last step) reads valid clamped addresses and its data is masked to zero,
// which keeps the wait counts exact.
template <int NW, int WN, int MT, int MTA, class AP, int PACKED>
__device__ __forceinline__ void k_main_loop(const KCtx<WN, AP>& c, half8* __restrict__ lds0,
                                            half8* __restrict__ lds1, float4v (&acc)[MT][WN]) {
  BRegs b0[WN], b1[WN];
  typename AP::Regs a0, a1;
  AP::load(c.A, a0, 0, c.K);
  k_load_b<WN, PACKED>(c, b0, 0);
  AP::load(c.A, a1, KSTEP, c.K);
  k_load_b<WN, PACKED>(c, b1, 1);
  AP::template store<MTA>(c.A, a0, 0, c.K, lds0);
  __syncthreads();
  AP::load(c.A, a0, 2 * KSTEP, c.K);
  for (int st = 0; st < c.nsteps; st += 2) {
    k_step<NW, WN, MT, MTA, AP, PACKED>(c, a1, b0, st, lds0, lds1, acc);
    k_load_b<WN, PACKED>(c, b0, st + 2);
    AP::load(c.A, a1, (st + 3) * KSTEP, c.K);
    k_step<NW, WN, MT, MTA, AP, PACKED>(c, a0, b1, st + 1, lds1, lds0, acc);
    k_load_b<WN, PACKED>(c, b1, st + 3);
    AP::load(c.A, a0, (st + 4) * KSTEP, c.K);
  }
}

// The K loop of one task with activation staging policy AP: the weights part
// of the context comes from cb, the activation part is set up here.
template <int NW, int WN, int MT, int MTA, class AP, int PACKED>
__device__ __forceinline__ void run_loop(const GemmParams& p, const BCtx<WN>& cb, int row0, int m0, int rows,
                                         half8* __restrict__ lds0, half8* __restrict__ lds1,
                                         float4v (&acc)[MT][WN]) {
  KCtx<WN, AP> c;
  static_cast<BCtx<WN>&>(c) = cb;
  AP::setup(p, row0, m0, rows, c.A);
  k_main_loop<NW, WN, MT, MTA, AP, PACKED>(c, lds0, lds1, acc);
}

// One task of the stream-K kernel: rows [m0, m0 + MC) of expert e, column
// tile nt of width NW * WN * 16 (SwiGLU: half of them gate, half up).
// MAXA: the most live row tiles the task can have.
template <int NW, int WN, int MT, int MAXA, int EPI, int PACKED, bool COH = false>
__device__ __forceinline__ void streamk_task(const GemmParams& p, int e, int m0, int nt, half8* __restrict__ lds0,
                                             half8* __restrict__ lds1) {
  constexpr int THREADS = NW * 64;
  constexpr int MC = MT * 16;
  constexpr int BN = NW * WN * 16;
  constexpr int PPT = (MT * 64 + THREADS - 1) / THREADS;   // A (row, K group) pairs per thread
  static_assert(EPI != EPI_SWIGLU || (WN % 2) == 0, "SwiGLU pairs gate and up tiles");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15;

  // data-dependent bounds are clamped so that inconsistent offsets can give
  // wrong rows but never an access outside the buffers
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  const int rows = min(MC, Me - m0);      // valid rows of this chunk (>= 1)
  const int mt_active = min((rows + 15) >> 4, MAXA);

  const int N = p.N;
  const int I = N / 2;
  BCtx<WN> c;      // weights part; the activation staging is set up per class below
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
  const float gab = p.a_g[0] * p.b_g[e];

  float4v acc[MT][WN];
#pragma unroll
  for (int r = 0; r < MT; ++r)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[r][j] = float4v{0.f, 0.f, 0.f, 0.f};

  switch (mt_active) {
    case 1:
      if constexpr (THREADS >= 256) {
        run_loop<NW, WN, MT, 1, AOneTile<THREADS, MT>, PACKED>(p, c, row0, m0, rows, lds0, lds1, acc);
      } else {
        run_loop<NW, WN, MT, 1, APairs<THREADS, MT, PPT>, PACKED>(p, c, row0, m0, rows, lds0, lds1, acc);
      }
      break;
    case 2:
      if constexpr (MAXA >= 2) {
        if constexpr (THREADS >= 256) {
          run_loop<NW, WN, MT, 2, ATwoTiles<THREADS, MT>, PACKED>(p, c, row0, m0, rows, lds0, lds1, acc);
        } else {
          run_loop<NW, WN, MT, 2, APairs<THREADS, MT, PPT>, PACKED>(p, c, row0, m0, rows, lds0, lds1, acc);
        }
      }
      break;
    case 3: if constexpr (MAXA >= 3) run_loop<NW, WN, MT, 3, APairs<THREADS, MT, PPT>, PACKED>(p, c, row0, m0, rows, lds0, lds1, acc); break;
    case 4: if constexpr (MAXA >= 4) run_loop<NW, WN, MT, 4, APairs<THREADS, MT, PPT>, PACKED>(p, c, row0, m0, rows, lds0, lds1, acc); break;
    case 5: case 6: if constexpr (MAXA >= 6) run_loop<NW, WN, MT, 6, APairs<THREADS, MT, PPT>, PACKED>(p, c, row0, m0, rows, lds0, lds1, acc); break;
    default: if constexpr (MAXA >= 8) run_loop<NW, WN, MT, MT, APairs<THREADS, MT, PPT>, PACKED>(p, c, row0, m0, rows, lds0, lds1, acc); break;
  }

  const int prow0 = row0 + m0;
#pragma unroll
  for (int r = 0; r < MAXA; ++r) {
    if (r >= mt_active) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int HALF = WN / 2;
#pragma unroll
      for (int jj = 0; jj < HALF; ++jj)
        epilogue_swiglu<COH>(p, acc[r][jj], acc[r][jj + HALF], prow0 + 16 * r, rows - 16 * r, col0[jj] + lr,
                             c.bok[jj], gab);
    } else {
#pragma unroll
      for (int j = 0; j < WN; ++j)
        epilogue_tile<EPI>(p, acc[r][j], prow0 + 16 * r, rows - 16 * r, col0[j] + lr, c.bok[j], gab);
    }
  }
}

// LIGHT > 0: the last chunk of an expert with at most LIGHT live row tiles
// runs as twice as many tasks of half the width (WN / 2 tiles per wave).  Such
// tasks are bound by the weight decode, which costs the same for 16 rows as
// for 64; halving each one's columns spreads the light tail of the grid over
// twice as many workgroups.  The sums are those of the wide tasks, element for
// element.
template <int NW, int WN, int MT, int EPI, int PACKED, int MINB, int LIGHT>
__global__ __launch_bounds__(NW * 64, MINB) void k_gemm_streamk(const GemmParams p) {
  static_assert(MT == 1 || MT == 2 || MT == 3 || MT == 4 || MT == 6 || MT == 8, "row tiles per chunk");
  static_assert(LIGHT == 0 || (WN % 2) == 0, "narrow tasks halve the tiles per wave");
  __shared__ half8 a_lds[2][MT * 8 * 64];   // double-buffered [row tile][sub-step][lane] fragments
  static_assert(fits_lds(sizeof(a_lds), MINB), "stream-K A staging exceeds the LDS of MINB workgroups per CU");
  int e, m0, nt;
  bool narrow;
  if (!find_task<MT, true, LIGHT>(p, e, m0, nt, narrow)) return;
  if constexpr (LIGHT > 0) {
    if (narrow) {
      streamk_task<NW, WN / 2, MT, LIGHT, EPI, PACKED>(p, e, m0, nt, a_lds[0], a_lds[1]);
      return;
    }
  }
  streamk_task<NW, WN, MT, MT, EPI, PACKED>(p, e, m0, nt, a_lds[0], a_lds[1]);
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

// OCOH: bf16 rows leave through agent-scope coherent (write-through) stores,
// so that a workgroup of the same launch on another XCD can read them (the
// output rows must then span less than 4 GiB: a buffer resource covers them)
template <int EPI, bool OCOH = false>
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
      if constexpr (OCOH) {
        const rsrc_t ro = make_rsrc(p.out, static_cast<uint32_t>(static_cast<size_t>(p.m_total) * p.N * 2));
        const uint32_t vo = static_cast<uint32_t>(base * 2);
        const u32x4 w0 = {w[0], w[1], w[2], w[3]}, w1 = {w[4], w[5], w[6], w[7]};
        __builtin_amdgcn_raw_buffer_store_b128(w0, ro, vo, 0, kCoherent);
        __builtin_amdgcn_raw_buffer_store_b128(w1, ro, vo + 16u, 0, kCoherent);
      } else {
        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + base);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int NW, int MT, int MTA, int UPW, int EPI, int PACKED, bool OCOH = false>
__device__ __forceinline__ void n_main_loop(const GemmParams& p, const half8* __restrict__ lds, float* stage,
                                            const uint8_t* tiles, int u_first, int u_count, int ntr, int prow0,
                                            int rows, float gab) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15;
  BRegs R0[UNIT], R1[UNIT];
  auto load_unit = [&](BRegs (&R)[UNIT], int i) {
    const int ui = u_first + min(i, u_count - 1);     // prefetches past the run re-read (cached)
#pragma unroll
    for (int t = 0; t < UNIT; ++t)
      b_load_packed<PACKED == kPackedNT>(tiles + static_cast<size_t>(min(UNIT * ui + t, ntr - 1)) * PTILE, R[t]);
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
          store_unit<EPI, OCOH>(p, acc[r], stage, prow0 + 16 * r, rows - 16 * r, col0, gab);
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

// One task of the stream-N kernel: rows [m0, m0 + MC) of expert e, column
// group ng (NW * UPW units of 64 columns).  a_lds: MT * 8 * 64 fragments;
// stage_lds: NW * 16 * 68 floats.  AAUX: cache policy of the A loads; OCOH:
// coherent output stores (store_unit).
template <int NW, int MT, int UPW, int EPI, int PACKED, int AAUX = 0, bool OCOH = false>
__device__ __forceinline__ void streamn_task(const GemmParams& p, int e, int m0, int ng, half8* __restrict__ a_lds,
                                             float* __restrict__ stage_lds) {
  constexpr int THREADS = NW * 64;
  constexpr int MC = MT * 16;
  constexpr int PPT = (MT * 64 + THREADS - 1) / THREADS;
  static_assert(UPW % 2 == 0, "units per wave come in pairs");
  const int wave = threadIdx.x >> 6;
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  const int rows = min(MC, Me - m0);
  const int mt_active = (rows + 15) >> 4;

  // stage the whole A chunk (one K step) in LDS
  AState<PPT> A;
  a_setup<THREADS, MT, PPT>(p, row0, m0, rows, A);
  ARegs<PPT> ra;
  a_load<PPT, AAUX>(A, ra, 0, p.K);
  a_store<THREADS, MT, MT, PPT>(A, ra, 0, p.K, a_lds);
  __syncthreads();

  const int ntr = (p.N + 15) / 16;
  const int nunits = (ntr + UNIT - 1) / UNIT;
  const int u_first = (ng * NW + wave) * UPW;
  const int u_count = min(UPW, nunits - u_first);
  if (u_count > 0) {
    const uint8_t* tiles = p.b_packed + static_cast<size_t>(e) * ntr * PTILE;
    const float gab = p.a_g[0] * p.b_g[e];
    const int prow0 = row0 + m0;
    float* stage = stage_lds + wave * (16 * 68);
    switch (mt_active) {
      case 1: n_main_loop<NW, MT, 1, UPW, EPI, PACKED, OCOH>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
      case 2: if constexpr (MT >= 2) n_main_loop<NW, MT, 2, UPW, EPI, PACKED, OCOH>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
      case 3: if constexpr (MT >= 3) n_main_loop<NW, MT, 3, UPW, EPI, PACKED, OCOH>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
      default: if constexpr (MT >= 4) n_main_loop<NW, MT, MT, UPW, EPI, PACKED, OCOH>(p, a_lds, stage, tiles, u_first, u_count, ntr, prow0, rows, gab); break;
    }
  }
}

template <int NW, int MT, int UPW, int EPI, int PACKED>
__global__ __launch_bounds__(NW * 64) void k_gemm_streamn(const GemmParams p) {
  __shared__ half8 a_lds[MT * 8 * 64];
  static_assert(fits_lds(sizeof(a_lds), 2), "stream-N A staging exceeds the LDS of two workgroups per CU");
  __shared__ float stage_lds[NW * 16 * 68];   // per-wave output staging (row pitch 68 floats)
  int e, m0, ng;
  bool narrow;
  if (!find_task<MT, false, 0>(p, e, m0, ng, narrow)) return;
  streamn_task<NW, MT, UPW, EPI, PACKED>(p, e, m0, ng, a_lds, stage_lds);
}

}  // namespace nvfp4
