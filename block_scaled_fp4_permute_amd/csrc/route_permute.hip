// Top-k routing and the expert-first permutation (histogram, prefix scan of
// expert offsets, stable scatter).
//
// The pages motivate both: a router picks a few of 256 experts per token
// ("Discovering SM120-Specific CUTLASS MoE Kernels", section "Input Knowledge
// Required"), and grouping rows by expert and reordering tokens is the first
// tool for raising the batch per expert ("From Empirical Limits to
// Research-Driven Optimization", section "Sections 5-6: Algorithmic
// Techniques").
//
// Kernels (all on one stream, no host round trip):
//   k_route        one wave per token: k rounds of a wave-wide argmax over the
//                  token's logits (ties to the lower id), then the renormalised
//                  softmax weights in float64.
//   k_chunk_rank   one workgroup per chunk of 1024 assignments: the stable rank
//                  of each assignment among the chunk's assignments to the same
//                  expert (wave ballots) and the chunk's expert histogram.
//   k_scan         one workgroup: counts = sum of chunk histograms, offsets =
//                  exclusive scan, and each chunk's base row per expert.
//   k_scatter      one thread per assignment: row = chunk base + rank.
// (A single-workgroup scan + scatter was slower than the two kernels even at
// 2048 assignments: one workgroup scatters with too little parallelism.)
// Atomics are used for nothing, so every output is deterministic.
#include "quantize_impl.h"

namespace nvfp4 {

static constexpr int kChunk = 1024;        // assignments per k_chunk_rank workgroup
static constexpr int kRankThreads = 256;   // 4 waves x 256 assignments

// ------------------------------------------------------------------ routing
// (v, id) is better than (bv, bid) in the order "larger logit, then lower id"
__device__ __forceinline__ bool better(float v, int id, float bv, int bid) {
  return v > bv || (v == bv && id < bid);
}

template <int CTRL>
__device__ __forceinline__ void row_argmax_step(float& bv, int& bid) {
  const float ov = __uint_as_float(dpp_u32<CTRL>(__float_as_uint(bv)));
  const int oid = static_cast<int>(dpp_u32<CTRL>(static_cast<uint32_t>(bid)));
  if (better(ov, oid, bv, bid)) {
    bv = ov;
    bid = oid;
  }
}

// Best (value, id) of the wave, returned to every lane: DPP exchanges inside
// each row of 16 lanes, then the 4 row winners read as scalars.
__device__ __forceinline__ void wave_argmax(float& bv, int& bid) {
  row_argmax_step<kDppXor1>(bv, bid);
  row_argmax_step<kDppXor2>(bv, bid);
  row_argmax_step<kDppHalfMirror>(bv, bid);
  row_argmax_step<kDppMirror>(bv, bid);
  float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
  int id = __builtin_amdgcn_readlane(bid, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * r));
    const int rid = __builtin_amdgcn_readlane(bid, 16 * r);
    if (better(rv, rid, v, id)) {
      v = rv;
      id = rid;
    }
  }
  bv = v;
  bid = id;
}

// One wave per token.  For E <= 64 * CACHE the token's logits stay in
// registers for all k rounds; larger E re-reads them (L1-resident) per round.
template <int CACHE>
__device__ __forceinline__ void route_body(const float* __restrict__ logits, int T, int E, int k,
                                           int* __restrict__ topk_ids, float* __restrict__ topk_w, int blk) {
  const int lane = threadIdx.x & 63;
  const int t = blk * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + static_cast<size_t>(t) * E;
  float cache[CACHE > 0 ? CACHE : 1];
  if constexpr (CACHE > 0) {
#pragma unroll
    for (int c = 0; c < CACHE; ++c) {
      const int i = lane + 64 * c;
      cache[c] = i < E ? row[i] : -__builtin_huge_valf();
    }
  }

  // winners so far: everything strictly better than (last_v, last_id) is taken;
  // lane j keeps the j-th winner
  float last_v = __builtin_huge_valf();
  int last_id = -1;
  float my_v = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_huge_valf();
    int bid = 0x7fffffff;
    if constexpr (CACHE > 0) {
#pragma unroll
      for (int c = 0; c < CACHE; ++c) {
        const int i = lane + 64 * c;
        const float v = cache[c];
        const bool eligible = i < E && (v < last_v || (v == last_v && i > last_id));
        if (eligible && better(v, i, bv, bid)) {
          bv = v;
          bid = i;
        }
      }
    } else {
      for (int i = lane; i < E; i += 64) {
        const float v = row[i];
        const bool eligible = v < last_v || (v == last_v && i > last_id);
        if (eligible && better(v, i, bv, bid)) {
          bv = v;
          bid = i;
        }
      }
    }
    wave_argmax(bv, bid);
    if (bid < 0 || bid >= E) bid = 0;   // only reachable with non-finite logits
    last_v = bv;
    last_id = bid;
    if (lane == j) {
      my_v = bv;
      my_id = bid;
    }
  }
  // weights: exp(l_j - l_max) / sum_i exp(l_i - l_max), in float64; l_max is the
  // first winner, held by lane 0
  const double top = static_cast<double>(__shfl(my_v, 0));
  const double mine = lane < k ? exp(static_cast<double>(my_v) - top) : 0.0;
  double sum = mine;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    topk_ids[static_cast<size_t>(t) * k + lane] = my_id;
    topk_w[static_cast<size_t>(t) * k + lane] = static_cast<float>(mine / sum);
  }
}

template <int CACHE>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E, int k,
                                               int* __restrict__ topk_ids, float* __restrict__ topk_w) {
  route_body<CACHE>(logits, T, E, k, topk_ids, topk_w, blockIdx.x);
}

// ------------------------------------------------------------------ stable ranks
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// chunk `blk`; cnt_sh: 4 E ints of LDS
__device__ __forceinline__ void chunk_rank_body(const int* __restrict__ ids, int n_asg, int E, int nbits,
                                                int* __restrict__ local_rank, int* __restrict__ chunk_hist,
                                                int* cnt_sh, int blk) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 4 * E; i += kRankThreads) cnt_sh[i] = 0;
  __syncthreads();

  int* cnt = cnt_sh + wave * E;
  const int base = blk * kChunk + wave * (kChunk / 4);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int xs[kChunk / 4 / 64];
#pragma unroll
  for (int s = 0; s < kChunk / 4 / 64; ++s) {
    const int f = base + s * 64 + lane;
    const int id = f < n_asg ? ids[f] : E;
    const bool valid = id >= 0 && id < E;
    const int x = valid ? id : E;
    xs[s] = x;
    uint64_t peers = ballot64(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (x >> b) & 1;
      const uint64_t bal = ballot64(bit);
      peers &= bit ? bal : ~bal;
    }
    if (valid) {
      const int rank_in = __popcll(peers & lt_mask);
      const int total = __popcll(peers);
      const int before = cnt[x];
      local_rank[f] = before + rank_in;
      // all lanes of the wave read cnt[] in the instruction above; the last lane
      // of each group of equal ids then advances that expert's counter
      if (rank_in == total - 1) cnt[x] = before + total;
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // per expert: exclusive prefix over the 4 waves, and the chunk's histogram
  for (int e = threadIdx.x; e < E; e += kRankThreads) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = cnt_sh[w * E + e];
      cnt_sh[w * E + e] = s;
      s += c;
    }
    chunk_hist[static_cast<size_t>(blk) * E + e] = s;
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kChunk / 4 / 64; ++s) {
    const int f = base + s * 64 + lane;
    if (f < n_asg && xs[s] < E) local_rank[f] += cnt_sh[wave * E + xs[s]];
  }
}

__global__ __launch_bounds__(kRankThreads) void k_chunk_rank(const int* __restrict__ ids, int n_asg, int E,
                                                             int nbits, int* __restrict__ local_rank,
                                                             int* __restrict__ chunk_hist) {
  extern __shared__ int cnt_sh[];  // [4][E]
  chunk_rank_body(ids, n_asg, E, nbits, local_rank, chunk_hist, cnt_sh, blockIdx.x);
}

// ------------------------------------------------------------------ routing paired with quantisation
// Routing and the activation quantisation read different inputs, and each of
// their kernels is short and leaves most of the GPU idle.  Two launches run
// them side by side, split by workgroup index (the branch is uniform per
// workgroup, so the barriers inside each body stay valid): the router's
// workgroups with the amax partials, then the chunk ranks with the encoder.
// The router's and the ranks' workgroups come first: they head the longer
// dependency chain.
template <int CACHE, int DT>
__global__ __launch_bounds__(256) void k_route_amax(const float* __restrict__ logits, int T, int E, int k,
                                                    int* __restrict__ topk_ids, float* __restrict__ topk_w,
                                                    int n_route, const void* __restrict__ x, int64_t nblocks16,
                                                    float* __restrict__ partial, int n_amax) {
  if (static_cast<int>(blockIdx.x) < n_route)
    route_body<CACHE>(logits, T, E, k, topk_ids, topk_w, blockIdx.x);
  else
    amax_body<DT>(x, nblocks16, partial, blockIdx.x - n_route, n_amax);
}

template <int DT>
__global__ __launch_bounds__(kRankThreads) void k_rank_quantize(const int* __restrict__ ids, int n_asg, int E,
                                                                int nbits, int* __restrict__ local_rank,
                                                                int* __restrict__ chunk_hist, int nchunks,
                                                                const void* __restrict__ x, int64_t nblocks16,
                                                                const float* __restrict__ g_in,
                                                                const float* __restrict__ partial, int nparts,
                                                                float* __restrict__ g_out,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales) {
  extern __shared__ int cnt_sh[];  // [4][E], used by the rank workgroups
  if (static_cast<int>(blockIdx.x) < nchunks)
    chunk_rank_body(ids, n_asg, E, nbits, local_rank, chunk_hist, cnt_sh, blockIdx.x);
  else
    quantize_body<DT>(x, nblocks16, g_in, partial, nparts, g_out, codes, scales, blockIdx.x - nchunks);
}

// ------------------------------------------------------------------ scan
// One workgroup of 1024 threads.  chunk_hist [nchunks][E] becomes the base row
// of each (chunk, expert): offsets[e] + number of earlier-chunk assignments.
// Thread t owns experts [t*per, t*per + per); a thread's chunk counts are read
// with independent loads (batches of 16), so the latency is paid once per
// batch rather than once per chunk.
static constexpr int kScanBatch = 16;
static constexpr int kMaxPer = 4;     // E <= 4096

__device__ __forceinline__ void scan_chunks(int* __restrict__ chunk_hist, int nchunks, int E,
                                            int* __restrict__ counts, int* __restrict__ offsets) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int per = (E + 1023) / 1024;
  const int e0 = tid * per;
  int cnt[kMaxPer];
  int local = 0;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int e = e0 + i;
    cnt[i] = 0;
    if (i < per && e < E) {
      for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j)
          v[j] = (c0 + j < nchunks) ? chunk_hist[static_cast<size_t>(c0 + j) * E + e] : 0;
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) cnt[i] += v[j];
      }
      counts[e] = cnt[i];
      local += cnt[i];
    }
  }
  // exclusive scan of the per-thread totals: wave scans, then the wave totals
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int wbase = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int v = wsum[w];
    wbase += (w < wave) ? v : 0;
    total += v;
  }
  int run = wbase + incl - local;
  if (tid == 0) offsets[E] = total;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int e = e0 + i;
    if (i < per && e < E) {
      offsets[e] = run;
      int s = run;
      for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j)
          v[j] = (c0 + j < nchunks) ? chunk_hist[static_cast<size_t>(c0 + j) * E + e] : 0;
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) {
          if (c0 + j < nchunks) chunk_hist[static_cast<size_t>(c0 + j) * E + e] = s;
          s += v[j];
        }
      }
      run += cnt[i];
    }
  }
}

__global__ __launch_bounds__(1024) void k_scan(int* __restrict__ chunk_hist, int nchunks, int E,
                                               int* __restrict__ counts, int* __restrict__ offsets) {
  scan_chunks(chunk_hist, nchunks, E, counts, offsets);
}

// ------------------------------------------------------------------ scatter
__global__ __launch_bounds__(256) void k_scatter(const int* __restrict__ ids, const float* __restrict__ topk_w,
                                                 const int* __restrict__ local_rank,
                                                 const int* __restrict__ chunk_base, int n_asg, int E, int k,
                                                 int* __restrict__ perm_src_token,
                                                 int* __restrict__ perm_of_assignment,
                                                 float* __restrict__ perm_weight) {
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= n_asg) return;
  const int e = min(max(ids[f], 0), E - 1);
  const int c = f / kChunk;
  int p = chunk_base[static_cast<size_t>(c) * E + e] + local_rank[f];
  p = (p >= 0 && p < n_asg) ? p : 0;   // keeps a wrong rank inside the buffers
  perm_src_token[p] = f / k;
  perm_of_assignment[f] = p;
  if (perm_weight) perm_weight[p] = topk_w[f];
}

// ------------------------------------------------------------------ host side
size_t route_permute_ws_bytes(int T, int E, int k) {
  const size_t n = static_cast<size_t>(T) * k;
  const size_t nchunks = (n + kChunk - 1) / kChunk;
  const size_t rank = (n * sizeof(int) + 255) & ~size_t(255);
  const size_t hist = (nchunks * E * sizeof(int) + 255) & ~size_t(255);
  return rank + hist;
}

hipError_t launch_route_permute(const float* logits, int T, int E, int k, int* topk_ids, float* topk_w,
                                int* counts, int* offsets, int* perm_src_token, int* perm_of_assignment,
                                float* perm_weight, void* ws, hipStream_t stream) {
  const int n = T * k;
  const int nchunks = (n + kChunk - 1) / kChunk;
  int* local_rank = static_cast<int*>(ws);
  int* chunk_hist = reinterpret_cast<int*>(static_cast<char*>(ws) +
                                           ((static_cast<size_t>(n) * sizeof(int) + 255) & ~size_t(255)));
  int nbits = 0;
  while ((1 << nbits) <= E) ++nbits;   // bits needed for ids 0..E (E is the padding sentinel)

  if (E <= 256)
    hipLaunchKernelGGL(k_route<4>, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, topk_ids, topk_w);
  else if (E <= 1024)
    hipLaunchKernelGGL(k_route<16>, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, topk_ids, topk_w);
  else
    hipLaunchKernelGGL(k_route<0>, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, topk_ids, topk_w);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_chunk_rank, dim3(nchunks), dim3(kRankThreads), 4 * E * sizeof(int), stream, topk_ids,
                     n, E, nbits, local_rank, chunk_hist);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, chunk_hist, nchunks, E, counts, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_scatter, dim3((n + 255) / 256), dim3(256), 0, stream, topk_ids, topk_w, local_rank,
                     chunk_hist, n, E, k, perm_src_token, perm_of_assignment, perm_weight);
  return hipGetLastError();
}

size_t route_quantize_ws_bytes(int T, int E, int k) {
  return route_permute_ws_bytes(T, E, k) + kAmaxBlocks * sizeof(float);
}

template <int CACHE, int DT>
static void launch_route_amax(const float* logits, int T, int E, int k, int* topk_ids, float* topk_w, int n_route,
                              const void* x, int64_t nb16, float* partial, int n_amax, hipStream_t stream) {
  hipLaunchKernelGGL((k_route_amax<CACHE, DT>), dim3(n_route + n_amax), dim3(256), 0, stream, logits, T, E, k,
                     topk_ids, topk_w, n_route, x, nb16, partial, n_amax);
}

hipError_t launch_route_quantize(const float* logits, int T, int E, int k, int* topk_ids, float* topk_w,
                                 int* counts, int* offsets, int* perm_src_token, int* perm_of_assignment,
                                 float* perm_weight, const void* x, int dtype, int64_t cols, const float* g_in,
                                 float* g_out, uint8_t* codes, uint8_t* scales, void* ws, hipStream_t stream) {
  const int n = T * k;
  const int nchunks = (n + kChunk - 1) / kChunk;
  int* local_rank = static_cast<int*>(ws);
  int* chunk_hist = reinterpret_cast<int*>(static_cast<char*>(ws) +
                                           ((static_cast<size_t>(n) * sizeof(int) + 255) & ~size_t(255)));
  float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + route_permute_ws_bytes(T, E, k));
  int nbits = 0;
  while ((1 << nbits) <= E) ++nbits;
  const int64_t nb16 = static_cast<int64_t>(T) * (cols / 16);
  const int n_route = (T + 3) / 4;
  // with a caller-given scale there is nothing to reduce: no amax workgroups
  const int n_amax = g_in ? 0 : amax_grid(nb16);
  const int nparts = n_amax;
  if (dtype == 1) {
    if (E <= 256) launch_route_amax<4, 1>(logits, T, E, k, topk_ids, topk_w, n_route, x, nb16, partial, n_amax, stream);
    else if (E <= 1024) launch_route_amax<16, 1>(logits, T, E, k, topk_ids, topk_w, n_route, x, nb16, partial, n_amax, stream);
    else launch_route_amax<0, 1>(logits, T, E, k, topk_ids, topk_w, n_route, x, nb16, partial, n_amax, stream);
  } else {
    if (E <= 256) launch_route_amax<4, 0>(logits, T, E, k, topk_ids, topk_w, n_route, x, nb16, partial, n_amax, stream);
    else if (E <= 1024) launch_route_amax<16, 0>(logits, T, E, k, topk_ids, topk_w, n_route, x, nb16, partial, n_amax, stream);
    else launch_route_amax<0, 0>(logits, T, E, k, topk_ids, topk_w, n_route, x, nb16, partial, n_amax, stream);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_quant = static_cast<int>((nb16 + 255) / 256);
  if (dtype == 1)
    hipLaunchKernelGGL(k_rank_quantize<1>, dim3(nchunks + n_quant), dim3(kRankThreads), 4 * E * sizeof(int), stream,
                       topk_ids, n, E, nbits, local_rank, chunk_hist, nchunks, x, nb16, g_in, partial, nparts, g_out,
                       codes, scales);
  else
    hipLaunchKernelGGL(k_rank_quantize<0>, dim3(nchunks + n_quant), dim3(kRankThreads), 4 * E * sizeof(int), stream,
                       topk_ids, n, E, nbits, local_rank, chunk_hist, nchunks, x, nb16, g_in, partial, nparts, g_out,
                       codes, scales);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, chunk_hist, nchunks, E, counts, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_scatter, dim3((n + 255) / 256), dim3(256), 0, stream, topk_ids, topk_w, local_rank,
                     chunk_hist, n, E, k, perm_src_token, perm_of_assignment, perm_weight);
  return hipGetLastError();
}

}  // namespace nvfp4
