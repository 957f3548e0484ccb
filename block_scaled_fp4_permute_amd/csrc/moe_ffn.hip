// The expert feed-forward part of the MoE layer in one persistent launch:
// gate_up grouped GEMM + SwiGLU + NVFP4 requantisation, then the down grouped
// GEMM, with down tasks starting while gate_up tasks are still running.
//
// The pages place the decode-time cost of the MoE layer in launch overhead and
// in small per-expert matrices ("From Empirical Limits to Research-Driven
// Optimization", section "Sections 5-6: Algorithmic Techniques": adaptive grid
// sizing, token reordering with fused reduction; section "Key Findings and
// Their Impact": fusion matters more when bandwidth is tight; "The Critical
// Search: Uncovering SM120 CUTLASS Collective Implementations", section
// "Context: The Optimization Journey": 16-64 tokens per expert).  With two
// launches, the gate_up kernel's last round of workgroups runs half empty (its
// light chunks) and the down kernel waits for all of it; here the down tasks
// of finished chunks fill those slots.
//
// Plan (k_ffn_plan, one workgroup, on the device: the per-expert counts never
// reach the host): the row chunks of all experts (64 rows each, in expert
// order) are dealt to the 8 XCDs in contiguous ranges of equal gate_up task
// counts; inside an XCD the chunks run heaviest class first (live 16-row tiles
// of the chunk: longest-first list scheduling), and the XCD's task list holds
// all its gate_up tasks, then the down tasks of the same chunks in the same
// order.  The lists go to the workspace with the counters the launch uses.
//
// Launch (k_moe_ffn, persistent: two workgroups per CU): a workgroup takes the
// next ticket of its XCD's list until the list is exhausted.  A gate_up task
// writes its h rows with agent-scope coherent stores, waits for them to
// complete, and then counts itself done on its chunk.  A down task first waits
// until every gate_up task of its chunk is done, then reads h with coherent
// loads.  No wait can block forever: a down ticket of an XCD is handed out
// only after all gate_up tickets of that XCD (which hold every gate_up task of
// its chunks) were taken by running workgroups, and gate_up tasks wait for
// nothing.  The wait is still bounded: past the spin limit the task sets the
// workspace's error word and goes on, so every workgroup ends.
#include "gemm_device.h"

namespace nvfp4 {

constexpr int kFfnMT = 4;                // row tiles per chunk (64 rows), as the decode tile
constexpr int kFfnMC = 16 * kFfnMT;
constexpr int kFfnGuBN = 256;            // gate_up columns per task (128 h columns)
constexpr int kFfnLight = 1;             // chunks with at most this many live row tiles may split in two
constexpr int kFfnHdrWords = 64;         // workspace header (int32 words)
// header word layout
constexpr int kHdrTicket = 0;            // [8] next ticket of each XCD's list
constexpr int kHdrError = 8;             // nonzero: a down task gave up waiting
constexpr int kHdrNGu = 16;              // [8] gate_up tasks of each XCD
constexpr int kHdrNDn = 24;              // [8] down tasks of each XCD
constexpr int kHdrGuBase = 32;           // [8] first gate_up task of each XCD in the gate_up list
constexpr int kHdrDnBase = 40;           // [8] first down task of each XCD in the down list
constexpr int kPlanThreads = 1024;

struct FfnLayout {
  size_t max_chunks, max_gu, max_dn, max_cnt;
  size_t off_done, off_gu, off_dn, off_cnt, bytes;   // byte offsets in the workspace
};

static inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

FfnLayout ffn_layout(int E, int64_t m_total, int ntl, int ndg) {
  FfnLayout L;
  L.max_chunks = static_cast<size_t>(m_total / kFfnMC) + static_cast<size_t>(E);
  L.max_gu = L.max_chunks * 2 * ntl;
  L.max_dn = L.max_chunks * ndg;
  L.off_done = align256(kFfnHdrWords * sizeof(int));
  L.off_gu = L.off_done + align256(L.max_chunks * sizeof(int));
  L.off_dn = L.off_gu + align256(L.max_gu * sizeof(int4));
  // combine counters: one per (token, down column group); tokens <= rows
  L.max_cnt = static_cast<size_t>(m_total) * static_cast<size_t>(ndg);
  L.off_cnt = L.off_dn + align256(L.max_dn * sizeof(int4));
  L.bytes = L.off_cnt + align256(L.max_cnt * sizeof(int));
  return L;
}

// ------------------------------------------------------------------ planner
struct PlanArgs {
  const int32_t* offsets;
  int E, m_total, ntl, ndg, slots;
  int max_chunks;       // capacity of the workspace lists (in chunks)
  int* hdr;
  int* done;
  int4* gu;
  int4* dn;
  int* cnt;             // combine counters to clear (n_cnt of them)
  int n_cnt;
};

// block-wide exclusive scan of one int per thread (kPlanThreads threads)
__device__ int plan_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    const int t = s_wave[w];
    before += (w < wave) ? t : 0;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

__global__ __launch_bounds__(kPlanThreads) void k_ffn_plan(const PlanArgs a) {
  // per expert, in LDS: rows, first chunk, first gate_up task (chunk order)
  extern __shared__ int s_dyn[];
  int* s_rows = s_dyn;                       // [E]
  int* s_chunk_base = s_dyn + a.E;           // [E + 1]
  int* s_task_base = s_dyn + 2 * a.E + 1;    // [E]
  __shared__ int s_wave[kPlanThreads / 64];
  __shared__ int s_cnt[8][kFfnMT + 1];     // chunks per (XCD, class)
  __shared__ int s_run[8][kFfnMT + 1];     // chunks per bucket placed so far
  __shared__ int s_wcnt[kPlanThreads / 64][8 * kFfnMT];
  __shared__ int s_gubase[8][kFfnMT + 1], s_dnbase[8][kFfnMT + 1];
  const int tid = threadIdx.x;
  for (int i = tid; i < a.n_cnt; i += kPlanThreads) a.cnt[i] = 0;
  if (tid < 8 * (kFfnMT + 1)) {
    (&s_cnt[0][0])[tid] = 0;
    (&s_run[0][0])[tid] = 0;
  }
  // rows and chunks per expert -> first chunk of each expert (data-dependent
  // bounds clamped: inconsistent offsets give wrong rows, never a bad access)
  int run = 0;
  for (int e0 = 0; e0 < a.E; e0 += kPlanThreads) {
    const int e = e0 + tid;
    int rows = 0;
    if (e < a.E) {
      const int lo = min(max(a.offsets[e], 0), a.m_total);
      const int hi = min(max(a.offsets[e + 1], 0), a.m_total);
      rows = max(hi - lo, 0);
      s_rows[e] = rows;
    }
    int tot;
    const int ex = plan_scan((rows + kFfnMC - 1) / kFfnMC, s_wave, tot);
    if (e < a.E) s_chunk_base[e] = run + ex;
    run += tot;
  }
  if (tid == 0) s_chunk_base[a.E] = run;
  // chunks past the lists' capacity (possible only with offsets that are not
  // non-decreasing, never with the routing calls' offsets) are dropped
  const int nc = min(run, a.max_chunks);
  // light chunks split in two only when the whole-width tasks outnumber the
  // resident workgroups (their light last round would leave slots empty)
  const int light = (static_cast<int64_t>(nc) * a.ntl > a.slots) ? kFfnLight : 0;
  auto tasks_of = [&](int q) { return q <= light ? 2 * a.ntl : a.ntl; };
  // gate_up tasks per expert -> first task of each expert, and the total
  int n_gu = 0;
  for (int e0 = 0; e0 < a.E; e0 += kPlanThreads) {
    const int e = e0 + tid;
    int t = 0;
    if (e < a.E && s_rows[e] > 0) {
      const int c = (s_rows[e] + kFfnMC - 1) / kFfnMC;
      const int q_last = min(kFfnMT, (s_rows[e] - (c - 1) * kFfnMC + 15) >> 4);
      t = (c - 1) * tasks_of(kFfnMT) + tasks_of(q_last);
    }
    int tot;
    const int ex = plan_scan(t, s_wave, tot);
    if (e < a.E) s_task_base[e] = n_gu + ex;
    n_gu += tot;
  }
  __syncthreads();
  // chunk c -> expert, first row, class (live row tiles), XCD: contiguous
  // ranges of equal gate_up task counts in chunk order
  auto chunk_info = [&](int c, int& e, int& m0, int& q, int& x) {
    // the last expert with s_chunk_base[e] <= c is the one whose chunks hold
    // c (experts without chunks share their successor's base)
    int lo = 0, hi = a.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_chunk_base[mid] <= c) lo = mid; else hi = mid;
    }
    e = lo;
    const int i = c - s_chunk_base[e];
    m0 = i * kFfnMC;
    q = min(kFfnMT, (s_rows[e] - m0 + 15) >> 4);
    const int ts = s_task_base[e] + i * tasks_of(kFfnMT);     // the chunks before it are full
    x = static_cast<int>((static_cast<int64_t>(ts) * 8) / max(n_gu, 1));
  };
  for (int c = tid; c < nc; c += kPlanThreads) {
    int e, m0, q, x;
    chunk_info(c, e, m0, q, x);
    atomicAdd(&s_cnt[x][q], 1);
  }
  __syncthreads();
  // list bases: XCD lists one after another; inside an XCD classes MT..1
  if (tid == 0) {
    int gb = 0, db = 0;
    for (int x = 0; x < 8; ++x) {
      int g = gb, d = db;
      for (int q = kFfnMT; q >= 1; --q) {
        s_gubase[x][q] = g;
        s_dnbase[x][q] = d;
        g += s_cnt[x][q] * tasks_of(q);
        d += s_cnt[x][q] * a.ndg;
      }
      a.hdr[kHdrNGu + x] = g - gb;
      a.hdr[kHdrNDn + x] = d - db;
      a.hdr[kHdrGuBase + x] = gb;
      a.hdr[kHdrDnBase + x] = db;
      a.hdr[kHdrTicket + x] = 0;
      gb = g;
      db = d;
    }
    a.hdr[kHdrError] = 0;
  }
  __syncthreads();
  // place each chunk in its bucket, keeping chunk order inside a bucket
  // (ballot ranks within a wave, wave totals within the tile, bucket totals
  // across tiles), and write its tasks
  const int lane = tid & 63, wave = tid >> 6;
  for (int c0 = 0; c0 < nc; c0 += kPlanThreads) {
    const int c = c0 + tid;
    int e = 0, m0 = 0, q = 1, x = 0;
    if (c < nc) chunk_info(c, e, m0, q, x);
    const int b = (c < nc) ? x * kFfnMT + (q - 1) : -1;
    int rank_in_wave = 0;
    for (int bb = 0; bb < 8 * kFfnMT; ++bb) {
      const uint64_t m = __ballot(b == bb);
      if (b == bb) rank_in_wave = __popcll(m & ((uint64_t(1) << lane) - 1));
      if (lane == 0) s_wcnt[wave][bb] = __popcll(m);
    }
    __syncthreads();
    if (c < nc) {
      int r = s_run[x][q] + rank_in_wave;
      for (int w = 0; w < wave; ++w) r += s_wcnt[w][b];
      const int tq = tasks_of(q);
      const bool narrow = tq != a.ntl;
      const int gpos = s_gubase[x][q] + r * tq;
      for (int k = 0; k < tq; ++k) a.gu[gpos + k] = make_int4(e, m0, k | (narrow ? 0x10000 : 0), c);
      const int dpos = s_dnbase[x][q] + r * a.ndg;
      for (int k = 0; k < a.ndg; ++k) a.dn[dpos + k] = make_int4(e, m0, k | (tq << 16), c);
      a.done[c] = 0;
    }
    __syncthreads();
    if (tid < 8 * kFfnMT) {
      int add = 0;
      for (int w = 0; w < kPlanThreads / 64; ++w) add += s_wcnt[w][tid];
      (&s_run[0][0])[(tid / kFfnMT) * (kFfnMT + 1) + (tid % kFfnMT) + 1] += add;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ persistent launch
struct FfnParams {
  GemmParams gu;          // gate_up, SwiGLU epilogue
  GemmParams dn;          // down, bf16 epilogue (A = h)
  int* hdr;
  int* done;
  const int4* gu_list;
  const int4* dn_list;
  int spin_limit;
  // fused combine: out[t] = sum_j topk_w[t, j] * y[perm_of[t, j]] (bf16)
  int* cnt;               // [T, ndg] down tasks done per (token, column group)
  const int32_t* perm_of;
  const float* topk_w;
  uint16_t* out;
  int T, k, ndg;
};

// The combine of the tokens whose last down row in column group ng this task
// wrote.  Every down task of a chunk counts, per row, one on the counter of
// (token, ng) once its coherent row stores have completed; the task that
// brings a counter to k holds the last of the token's k rows of that column
// group and combines them (rows read with coherent loads) - in the order
// j = 0, 1, ... of the unfused combine, so the output is the same bit for bit.
// No task waits for another.
template <int UPW>
__device__ __forceinline__ void ffn_finalize(const FfnParams& f, int e, int m0, int ng, int* s_list, int* s_n) {
  const GemmParams& p = f.dn;
  const int row0 = min(max(p.offsets[e], 0), p.m_total);
  const int Me = min(max(p.offsets[e + 1], 0), p.m_total) - row0;
  const int rows = min(kFfnMC, Me - m0);
  __builtin_amdgcn_s_waitcnt(0);     // this wave's row stores have completed
  __syncthreads();                   // and every wave's
  if (threadIdx.x < 64) {            // wave 0: one row per lane
    const int i = threadIdx.x;
    bool last = false;
    int tok = 0;
    if (i < rows) {
      tok = f.gu.a_rows[row0 + m0 + i];
      if (tok >= 0 && tok < f.T) {
        const int old = __hip_atomic_fetch_add(f.cnt + static_cast<size_t>(tok) * f.ndg + ng, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        last = old == f.k - 1;
      }
    }
    const uint64_t m = __ballot(last);
    if (last) s_list[__popcll(m & ((uint64_t(1) << i) - 1))] = tok;
    if (i == 0) *s_n = __popcll(m);
  }
  __syncthreads();
  const int n = *s_n;
  constexpr int kGroupCols = 4 * UPW * 64;     // columns of a down column group
  const int H = p.N;
  const int c0 = ng * kGroupCols;
  const int ncg = max(0, min(kGroupCols, H - c0)) / 8;
  const rsrc_t ry = make_rsrc(p.out, static_cast<uint32_t>(static_cast<size_t>(p.m_total) * H * 2));
  for (int it = threadIdx.x; it < n * ncg; it += blockDim.x) {
    const int tok = s_list[it / ncg];
    const int c = c0 + 8 * (it % ncg);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < f.k; j0 += 8) {
      u32x4 q[8];
      float wt[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const size_t a = static_cast<size_t>(tok) * f.k + min(j0 + u, f.k - 1);
        const int row = f.perm_of[a];
        wt[u] = f.topk_w[a];
        // rows outside [0, m_total) read zeros (the buffer range check)
        const uint32_t off = (row >= 0 && row < p.m_total) ? static_cast<uint32_t>((static_cast<size_t>(row) * H + c) * 2)
                                                           : 0xFFFFFFF0u;
        q[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, kCoherent));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u < f.k) {
          const uint32_t w4[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            acc[2 * m] = fmaf(wt[u], __uint_as_float(w4[m] << 16), acc[2 * m]);
            acc[2 * m + 1] = fmaf(wt[u], __uint_as_float(w4[m] & 0xFFFF0000u), acc[2 * m + 1]);
          }
        }
      }
    }
    uint4 o;
    o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
    o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
    *reinterpret_cast<uint4*>(f.out + static_cast<size_t>(tok) * H + c) = o;
  }
}

template <int UPW, int GU_PACKED, int DN_PACKED, bool FUSED>
__global__ __launch_bounds__(256, 2) void k_moe_ffn(const FfnParams f) {
  // gate_up: two 64-row x 256-K fragment buffers (64 KB); down: one buffer
  // (32 KB) and the per-wave output staging (17 KB) in the same space
  __shared__ half8 smem[2 * kFfnMT * 8 * 64];
  static_assert(fits_lds(sizeof(smem) + 64, 2), "expert-FFN staging exceeds the LDS of two workgroups per CU");
  __shared__ int s_ticket;
  __shared__ int s_list[kFfnMC], s_n;     // fused combine: tokens this task completes
  const int xcd = blockIdx.x & 7;
  const int n_gu = f.hdr[kHdrNGu + xcd];
  const int n_dn = f.hdr[kHdrNDn + xcd];
  const int gb = f.hdr[kHdrGuBase + xcd];
  const int db = f.hdr[kHdrDnBase + xcd];
  for (;;) {
    __syncthreads();     // the previous task's LDS reads are done
    if (threadIdx.x == 0)
      s_ticket = __hip_atomic_fetch_add(f.hdr + kHdrTicket + xcd, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int j = s_ticket;
    if (j < n_gu) {
      const int4 d = f.gu_list[gb + j];
      const int nt = d.z & 0xFFFF;
      if (d.z & 0x10000)
        streamk_task<4, 2, kFfnMT, kFfnLight, EPI_SWIGLU, GU_PACKED, true>(f.gu, d.x, d.y, nt, smem,
                                                                            smem + kFfnMT * 8 * 64);
      else
        streamk_task<4, 4, kFfnMT, kFfnMT, EPI_SWIGLU, GU_PACKED, true>(f.gu, d.x, d.y, nt, smem,
                                                                         smem + kFfnMT * 8 * 64);
      __builtin_amdgcn_s_waitcnt(0);   // this wave's h stores have completed
      __syncthreads();                 // and every wave's
      if (threadIdx.x == 0) __hip_atomic_fetch_add(f.done + d.w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (j - n_gu < n_dn) {
      const int4 d = f.dn_list[db + (j - n_gu)];
      const int need = d.z >> 16;
      if (threadIdx.x == 0) {
        int spins = 0;
        while (__hip_atomic_load(f.done + d.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
          __builtin_amdgcn_s_sleep(4);
          if (++spins > f.spin_limit) {
            __hip_atomic_store(f.hdr + kHdrError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
      }
      __syncthreads();
      streamn_task<4, kFfnMT, UPW, EPI_BF16, DN_PACKED, kCoherent, FUSED>(
          f.dn, d.x, d.y, d.z & 0xFFFF, smem, reinterpret_cast<float*>(smem + kFfnMT * 8 * 64));
      if constexpr (FUSED) ffn_finalize<UPW>(f, d.x, d.y, d.z & 0xFFFF, s_list, &s_n);
    } else {
      break;
    }
  }
}

// ------------------------------------------------------------------ host side
static int ffn_compute_units() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 256;
  return v;
}

static int ffn_ntl(int I) { return (I + kFfnGuBN / 2 - 1) / (kFfnGuBN / 2); }
static int ffn_ndg(int H, int upw) {
  const int nunits = ((H + 15) / 16 + UNIT - 1) / UNIT;
  return (nunits + 4 * upw - 1) / (4 * upw);
}
constexpr int kFfnUPW = 6;

size_t moe_ffn_ws_bytes(int E, int64_t m_total, int H, int I) {
  return ffn_layout(E, m_total, ffn_ntl(I), ffn_ndg(H, kFfnUPW)).bytes;
}

// gu: gate_up parameters (SwiGLU epilogue; A = x rows gathered by a_rows);
// dn: down parameters (bf16 epilogue; A = h).  Both with packed weights.
hipError_t launch_moe_ffn(GemmParams gu, GemmParams dn, int64_t m_total, bool cached, void* ws, int spin_limit,
                          const FfnCombine* comb, hipStream_t stream) {
  const int I = gu.N / 2;
  const int H = dn.N;
  const int ntl = ffn_ntl(I);
  const int ndg = ffn_ndg(H, kFfnUPW);
  const FfnLayout L = ffn_layout(gu.E, m_total, ntl, ndg);
  char* w = static_cast<char*>(ws);
  const int slots = 2 * ffn_compute_units();
  gu.n_tiles = ntl;
  gu.slots = slots;
  dn.n_tiles = ndg;
  dn.slots = slots;
  int* cnt = reinterpret_cast<int*>(w + L.off_cnt);
  const int n_cnt = comb ? comb->T * ndg : 0;
  PlanArgs pa{gu.offsets, gu.E, gu.m_total, ntl, ndg, slots, static_cast<int>(L.max_chunks), reinterpret_cast<int*>(w),
              reinterpret_cast<int*>(w + L.off_done), reinterpret_cast<int4*>(w + L.off_gu),
              reinterpret_cast<int4*>(w + L.off_dn), cnt, n_cnt};
  hipLaunchKernelGGL(k_ffn_plan, dim3(1), dim3(kPlanThreads), (3 * gu.E + 1) * sizeof(int), stream, pa);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  FfnParams f{gu, dn, reinterpret_cast<int*>(w), reinterpret_cast<int*>(w + L.off_done),
              reinterpret_cast<const int4*>(w + L.off_gu), reinterpret_cast<const int4*>(w + L.off_dn), spin_limit,
              cnt, comb ? comb->perm_of : nullptr, comb ? comb->topk_w : nullptr,
              comb ? static_cast<uint16_t*>(comb->out) : nullptr, comb ? comb->T : 0, comb ? comb->k : 0, ndg};
  const int grid = (slots + 7) / 8 * 8;
  if (comb) {
    if (cached)
      hipLaunchKernelGGL((k_moe_ffn<kFfnUPW, kPackedCached, kPackedCached, true>), dim3(grid), dim3(256), 0, stream, f);
    else
      hipLaunchKernelGGL((k_moe_ffn<kFfnUPW, kPackedNT, kPackedNT, true>), dim3(grid), dim3(256), 0, stream, f);
  } else {
    if (cached)
      hipLaunchKernelGGL((k_moe_ffn<kFfnUPW, kPackedCached, kPackedCached, false>), dim3(grid), dim3(256), 0, stream, f);
    else
      hipLaunchKernelGGL((k_moe_ffn<kFfnUPW, kPackedNT, kPackedNT, false>), dim3(grid), dim3(256), 0, stream, f);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
