// C-ABI entry points of libnvfp4moe: argument validation on the host, then
// kernel launches on the caller's stream.  Nothing is allocated here.
#include <stdio.h>
#include <stdarg.h>
#include <stdlib.h>

#include <mutex>
#include <vector>

#include "../../include/nvfp4moe.h"
#include "nvfp4_internal.h"

namespace {

thread_local char g_detail[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_detail[0] = '\0';
  return NVFP4MOE_OK;
}

int hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return ok();
  return fail(NVFP4MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a * b >= limit for non-negative a, b, without overflowing
bool prod_ge(int64_t a, int64_t b, int64_t limit) {
  int64_t r = 0;
  return __builtin_mul_overflow(a, b, &r) || r >= limit;
}
bool prod_ge(int64_t a, int64_t b, int64_t c, int64_t limit) {
  int64_t r = 0;
  return __builtin_mul_overflow(a, b, &r) || prod_ge(r, c, limit);
}

// Debug checks (NVFP4MOE_DEBUG set to anything but "" or "0", read at every
// call): before launching, a call copies the device index arrays it reads to
// the host and checks them - offsets non-decreasing from 0 to at most
// m_total, gathered rows and combine rows inside their buffers - and returns
// NVFP4MOE_ERR_INVALID naming the first bad entry.  Without the checks the
// kernels clamp such entries (wrong rows, never an access out of bounds).
// The copies synchronise the stream: for debugging, not for graph capture.
bool debug_checks() {
  const char* v = getenv("NVFP4MOE_DEBUG");
  return v && v[0] && !(v[0] == '0' && v[1] == '\0');
}

int fetch_ints(const char* fn, const int32_t* d, int64_t n, hipStream_t s, std::vector<int32_t>& h) {
  h.resize(static_cast<size_t>(n));
  hipError_t e = hipMemcpyAsync(h.data(), d, static_cast<size_t>(n) * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(NVFP4MOE_ERR_HIP, "%s: debug check copy: %s", fn, hipGetErrorString(e));
  return NVFP4MOE_OK;
}

// offsets [E+1]: 0, non-decreasing, at most m_total; rows_used: offsets[E]
int debug_check_offsets(const char* fn, const int32_t* offsets, int32_t E, int64_t m_total, hipStream_t s,
                        int64_t& rows_used) {
  std::vector<int32_t> h;
  const int st = fetch_ints(fn, offsets, int64_t(E) + 1, s, h);
  if (st != NVFP4MOE_OK) return st;
  if (h[0] != 0) return fail(NVFP4MOE_ERR_INVALID, "%s: offsets[0] = %d, expected 0", fn, h[0]);
  for (int32_t e = 0; e < E; ++e)
    if (h[e + 1] < h[e])
      return fail(NVFP4MOE_ERR_INVALID, "%s: offsets decrease at expert %d (%d -> %d)", fn, e, h[e], h[e + 1]);
  if (h[E] > m_total)
    return fail(NVFP4MOE_ERR_INVALID, "%s: offsets[E] = %d > m_total = %lld", fn, h[E],
                static_cast<long long>(m_total));
  rows_used = h[E];
  return NVFP4MOE_OK;
}

// the first n entries of an index array inside [0, hi)
int debug_check_range(const char* fn, const char* what, const int32_t* d, int64_t n, int64_t hi, hipStream_t s) {
  if (!d || n <= 0) return NVFP4MOE_OK;
  std::vector<int32_t> h;
  const int st = fetch_ints(fn, d, n, s, h);
  if (st != NVFP4MOE_OK) return st;
  for (int64_t i = 0; i < n; ++i)
    if (h[i] < 0 || h[i] >= hi)
      return fail(NVFP4MOE_ERR_INVALID, "%s: %s[%lld] = %d outside [0, %lld)", fn, what, static_cast<long long>(i),
                  h[i], static_cast<long long>(hi));
  return NVFP4MOE_OK;
}

// the checks of a grouped GEMM: offsets, gathered A rows, combine rows
int debug_check_gemm(const char* fn, const int32_t* offsets, int32_t E, int64_t m_total, const int32_t* a_rows,
                     int64_t a_rows_total, const int32_t* row_token, int64_t out_rows, hipStream_t s,
                     const char* a_rows_name = "a_rows") {
  int64_t used = 0;
  int st = debug_check_offsets(fn, offsets, E, m_total, s, used);
  if (st == NVFP4MOE_OK) st = debug_check_range(fn, a_rows_name, a_rows, used, a_rows_total, s);
  if (st == NVFP4MOE_OK) st = debug_check_range(fn, "row_token", row_token, used, out_rows, s);
  return st;
}

constexpr size_t kSmallWs = 4096;   // 1024 partial maxima of the amax reduction

// Argument checks of the route + quantise calls (everything but the workspace).
int check_route_quantize(const char* fn, const float* logits, int32_t T, int32_t E, int32_t k,
                         const int32_t* topk_ids, const float* topk_w, const int32_t* counts, const int32_t* offsets,
                         const int32_t* perm_src_token, const int32_t* perm_of_assignment, const void* x,
                         int32_t x_dtype, int64_t cols, const uint8_t* codes, const uint8_t* scales) {
  if (!logits || !topk_ids || !topk_w || !counts || !offsets || !perm_src_token || !perm_of_assignment)
    return fail(NVFP4MOE_ERR_INVALID, "%s: null routing pointer argument", fn);
  if (!x || !codes || !scales) return fail(NVFP4MOE_ERR_INVALID, "%s: null x, codes or scales", fn);
  if (T <= 0 || E <= 0 || k <= 0) return fail(NVFP4MOE_ERR_INVALID, "%s: T, E, k must be > 0", fn);
  if (k > E) return fail(NVFP4MOE_ERR_INVALID, "%s: k=%d > E=%d", fn, k, E);
  if (k > 32) return fail(NVFP4MOE_ERR_UNSUPPORTED, "%s: k=%d > 32", fn, k);
  if (E > 4096) return fail(NVFP4MOE_ERR_UNSUPPORTED, "%s: E=%d > 4096", fn, E);
  if (static_cast<int64_t>(T) * k >= (int64_t(1) << 30)) return fail(NVFP4MOE_ERR_UNSUPPORTED, "%s: T*k >= 2^30", fn);
  if (x_dtype != NVFP4MOE_F32 && x_dtype != NVFP4MOE_BF16)
    return fail(NVFP4MOE_ERR_INVALID, "%s: x_dtype %d", fn, x_dtype);
  if (cols <= 0 || cols % 32 != 0)
    return fail(NVFP4MOE_ERR_INVALID, "%s: cols=%lld must be a positive multiple of 32", fn, (long long)cols);
  if (prod_ge(T, cols / 16, int64_t(1) << 40)) return fail(NVFP4MOE_ERR_UNSUPPORTED, "%s: tensor too large", fn);
  // the encoder's workgroups are indexed after the ranks' in one grid
  if ((static_cast<int64_t>(T) * (cols / 16) + 255) / 256 + (static_cast<int64_t>(T) * k + 1023) / 1024 >=
      (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "%s: grid too large", fn);
  if (!aligned(x, 16) || !aligned(codes, 8)) return fail(NVFP4MOE_ERR_INVALID, "%s: misaligned x or codes", fn);
  return NVFP4MOE_OK;
}

// ------------------------------------------------------------------ scratch of the no-allocation entry point
// One fixed block of device memory per GPU, held until the process ends,
// shared by every call of moe_route_quantize_noalloc on that GPU.  In host
// code `scratch` names a host-side stand-in, not a device address: kernels
// get the device address that hipGetSymbolAddress returns for the current
// device, looked up once per device and kept.
constexpr size_t kScratchBytes = size_t(4) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int device_scratch(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(NVFP4MOE_ERR_HIP, "scratch: hipGetDevice: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices) return fail(NVFP4MOE_ERR_UNSUPPORTED, "scratch: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p)
      return fail(NVFP4MOE_ERR_HIP, "scratch: hipGetSymbolAddress on device %d: %s", dev, hipGetErrorString(err));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NVFP4MOE_OK;
}

}  // namespace

extern "C" {

const char* nvfp4moe_status_string(int status) {
  switch (status) {
    case NVFP4MOE_OK: return "ok";
    case NVFP4MOE_ERR_INVALID: return "invalid argument";
    case NVFP4MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case NVFP4MOE_ERR_WORKSPACE: return "workspace too small";
    case NVFP4MOE_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* nvfp4moe_last_error_detail(void) { return g_detail; }

int nvfp4moe_version(void) { return 101; }

// ------------------------------------------------------------------ route + permute
size_t moe_route_permute_workspace_size(int32_t T, int32_t E, int32_t k) {
  if (T <= 0 || E <= 0 || k <= 0 || k > 32 || E > 4096 || prod_ge(T, k, int64_t(1) << 30)) return 0;
  return nvfp4::route_permute_ws_bytes(T, E, k);
}

int moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids, float* topk_w,
                      int32_t* counts, int32_t* offsets, int32_t* perm_src_token, int32_t* perm_of_assignment,
                      float* perm_weight, void* workspace, size_t workspace_bytes, void* stream) {
  if (!logits || !topk_ids || !topk_w || !counts || !offsets || !perm_src_token || !perm_of_assignment)
    return fail(NVFP4MOE_ERR_INVALID, "moe_route_permute: null pointer argument");
  if (T <= 0 || E <= 0 || k <= 0) return fail(NVFP4MOE_ERR_INVALID, "moe_route_permute: T, E, k must be > 0");
  if (k > E) return fail(NVFP4MOE_ERR_INVALID, "moe_route_permute: k=%d > E=%d", k, E);
  if (k > 32) return fail(NVFP4MOE_ERR_UNSUPPORTED, "moe_route_permute: k=%d > 32", k);
  if (E > 4096) return fail(NVFP4MOE_ERR_UNSUPPORTED, "moe_route_permute: E=%d > 4096", E);
  if (static_cast<int64_t>(T) * k >= (int64_t(1) << 30))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "moe_route_permute: T*k >= 2^30");
  const size_t need = nvfp4::route_permute_ws_bytes(T, E, k);
  if (!workspace || workspace_bytes < need)
    return fail(NVFP4MOE_ERR_WORKSPACE, "moe_route_permute: workspace %zu < %zu bytes", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(NVFP4MOE_ERR_INVALID, "moe_route_permute: workspace not 16-byte aligned");
  return hip_status(nvfp4::launch_route_permute(logits, T, E, k, topk_ids, topk_w, counts, offsets, perm_src_token,
                                                perm_of_assignment, perm_weight, workspace,
                                                static_cast<hipStream_t>(stream)),
                    "moe_route_permute");
}

// ------------------------------------------------------------------ quantise
size_t nvfp4_quantize_workspace_size(void) { return kSmallWs; }

int nvfp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, const float* g_in, float* g_out,
                   uint8_t* codes, uint8_t* scales, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !codes || !scales) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_quantize: null pointer argument");
  if (x_dtype != NVFP4MOE_F32 && x_dtype != NVFP4MOE_BF16)
    return fail(NVFP4MOE_ERR_INVALID, "nvfp4_quantize: x_dtype %d", x_dtype);
  if (rows <= 0 || cols <= 0) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_quantize: rows, cols must be > 0");
  if (cols % 32 != 0) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_quantize: cols=%lld not a multiple of 32", (long long)cols);
  if (prod_ge(rows, cols / 16, int64_t(1) << 40))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "nvfp4_quantize: tensor too large");
  if (!aligned(x, 16) || !aligned(codes, 8)) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_quantize: misaligned x or codes");
  if (!g_in && (!workspace || workspace_bytes < kSmallWs))
    return fail(NVFP4MOE_ERR_WORKSPACE, "nvfp4_quantize: workspace of %zu bytes needed when g_in is NULL", kSmallWs);
  return hip_status(nvfp4::launch_quantize(x, x_dtype, rows, cols, g_in, g_out, codes, scales, workspace,
                                           static_cast<hipStream_t>(stream)),
                    "nvfp4_quantize");
}

// ------------------------------------------------------------------ route + quantise
size_t moe_route_quantize_workspace_size(int32_t T, int32_t E, int32_t k) {
  if (T <= 0 || E <= 0 || k <= 0 || k > 32 || E > 4096 || prod_ge(T, k, int64_t(1) << 30)) return 0;
  return nvfp4::route_quantize_ws_bytes(T, E, k);
}

int moe_route_quantize(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids, float* topk_w,
                       int32_t* counts, int32_t* offsets, int32_t* perm_src_token, int32_t* perm_of_assignment,
                       float* perm_weight, const void* x, int32_t x_dtype, int64_t cols, const float* g_in,
                       float* g_out, uint8_t* codes, uint8_t* scales, void* workspace, size_t workspace_bytes,
                       void* stream) {
  const int bad = check_route_quantize("moe_route_quantize", logits, T, E, k, topk_ids, topk_w, counts, offsets,
                                       perm_src_token, perm_of_assignment, x, x_dtype, cols, codes, scales);
  if (bad != NVFP4MOE_OK) return bad;
  const size_t need = nvfp4::route_quantize_ws_bytes(T, E, k);
  if (!workspace || workspace_bytes < need)
    return fail(NVFP4MOE_ERR_WORKSPACE, "moe_route_quantize: workspace %zu < %zu bytes", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(NVFP4MOE_ERR_INVALID, "moe_route_quantize: workspace not 16-byte aligned");
  return hip_status(nvfp4::launch_route_quantize(logits, T, E, k, topk_ids, topk_w, counts, offsets, perm_src_token,
                                                 perm_of_assignment, perm_weight, x, x_dtype, cols, g_in, g_out,
                                                 codes, scales, workspace, static_cast<hipStream_t>(stream)),
                    "moe_route_quantize");
}

size_t moe_route_quantize_noalloc_max_workspace(void) { return kScratchBytes; }

int moe_route_quantize_noalloc(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                               float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm_src_token,
                               int32_t* perm_of_assignment, float* perm_weight, const void* x, int32_t x_dtype,
                               int64_t cols, const float* g_in, float* g_out, uint8_t* codes, uint8_t* scales,
                               void* stream) {
  const int bad = check_route_quantize("moe_route_quantize_noalloc", logits, T, E, k, topk_ids, topk_w, counts,
                                       offsets, perm_src_token, perm_of_assignment, x, x_dtype, cols, codes, scales);
  if (bad != NVFP4MOE_OK) return bad;
  const size_t need = nvfp4::route_quantize_ws_bytes(T, E, k);
  if (need > kScratchBytes)
    return fail(NVFP4MOE_ERR_UNSUPPORTED,
                "moe_route_quantize_noalloc: T=%d, E=%d, k=%d need %zu bytes of scratch, more than the %zu the "
                "library holds per device (use moe_route_quantize with a workspace)",
                T, E, k, need, kScratchBytes);
  void* ws = nullptr;
  const int st = device_scratch(&ws);
  if (st != NVFP4MOE_OK) return st;
  // every scratch word the kernels read is written earlier in the same call:
  // nothing needs clearing between calls
  return hip_status(nvfp4::launch_route_quantize(logits, T, E, k, topk_ids, topk_w, counts, offsets, perm_src_token,
                                                 perm_of_assignment, perm_weight, x, x_dtype, cols, g_in, g_out,
                                                 codes, scales, ws, static_cast<hipStream_t>(stream)),
                    "moe_route_quantize_noalloc");
}

// ------------------------------------------------------------------ grouped GEMM
int nvfp4_grouped_gemm(const nvfp4moe_gemm_args* a, void* stream) {
  if (!a) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: args is NULL");
  if (!a->a_codes || !a->a_scales || !a->a_g || !a->b_g || !a->offsets)
    return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: null operand pointer");
  if (!a->b_packed && (!a->b_codes || !a->b_scales))
    return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: B needs b_codes and b_scales, or b_packed");
  if (a->E <= 0 || a->N <= 0 || a->K <= 0 || a->m_total < 0 || a->a_rows_total <= 0)
    return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: E, N, K, a_rows_total must be > 0 and m_total >= 0");
  if (a->K % 32 != 0) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: K=%d not a multiple of 32", a->K);
  if (a->N % 16 != 0) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: N=%d not a multiple of 16", a->N);
  if (!aligned(a->a_codes, 16) || !aligned(a->a_scales, 2) || !aligned(a->b_packed, 16) ||
      (!a->b_packed && (!aligned(a->b_codes, 16) || !aligned(a->b_scales, 2))))
    return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: codes and packed tiles must be 16-byte, scales 2-byte aligned");
  if (a->m_total >= (int64_t(1) << 31) || a->a_rows_total >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "nvfp4_grouped_gemm: more than 2^31 rows");
  // the kernels address A with 32-bit byte offsets
  if (a->a_rows_total * (int64_t(a->K) / 2) >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "nvfp4_grouped_gemm: A codes of 2 GiB or more (a_rows_total * K / 2)");
  if (static_cast<int64_t>(a->E) * a->N >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "nvfp4_grouped_gemm: E*N >= 2^31");
  switch (a->epilogue) {
    case NVFP4MOE_EPI_F32:
    case NVFP4MOE_EPI_BF16:
      if (!a->out && a->m_total > 0) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: out is NULL");
      // rows leave as 16-byte vector stores
      if (!aligned(a->out, 16)) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: out not 16-byte aligned");
      break;
    case NVFP4MOE_EPI_SWIGLU_NVFP4:
      if (a->N % 32 != 0) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: SwiGLU needs N = 2I with I %% 16 == 0");
      if (!a->out_codes || !a->out_scales || !a->out_g)
        return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: SwiGLU needs out_codes, out_scales, out_g");
      break;
    case NVFP4MOE_EPI_COMBINE_F32:
      if (!a->out || !a->row_token || !a->row_weight || a->out_rows <= 0)
        return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: combine needs out, row_token, row_weight, out_rows");
      if (!aligned(a->out, 4)) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: out misaligned");
      break;
    default:
      return fail(NVFP4MOE_ERR_INVALID, "nvfp4_grouped_gemm: unknown epilogue %d", a->epilogue);
  }
  if (a->m_total == 0) return ok();
  if (debug_checks()) {
    const bool comb = a->epilogue == NVFP4MOE_EPI_COMBINE_F32;
    const int st = debug_check_gemm("nvfp4_grouped_gemm", a->offsets, a->E, a->m_total, a->a_rows, a->a_rows_total,
                                    comb ? a->row_token : nullptr, a->out_rows, static_cast<hipStream_t>(stream));
    if (st != NVFP4MOE_OK) return st;
  }
  nvfp4::GemmParams prm{};
  prm.a_codes = a->a_codes;
  prm.a_scales = a->a_scales;
  prm.a_g = a->a_g;
  prm.a_rows = a->a_rows;
  prm.b_codes = a->b_codes;
  prm.b_scales = a->b_scales;
  prm.b_packed = a->b_packed;
  prm.b_g = a->b_g;
  prm.offsets = a->offsets;
  prm.E = a->E;
  prm.N = a->N;
  prm.K = a->K;
  prm.m_total = static_cast<int>(a->m_total);
  prm.a_rows_total = static_cast<int>(a->a_rows_total);
  prm.out_rows = static_cast<int>(a->out_rows < (int64_t(1) << 31) ? a->out_rows : 0);
  prm.out = a->out;
  prm.out_codes = a->out_codes;
  prm.out_scales = a->out_scales;
  prm.out_g = a->out_g;
  prm.row_token = a->row_token;
  prm.row_weight = a->row_weight;
  return hip_status(nvfp4::launch_grouped_gemm(prm, a->epilogue, a->m_total, a->max_rows_per_expert_hint,
                                               static_cast<hipStream_t>(stream)),
                    "nvfp4_grouped_gemm");
}

// ------------------------------------------------------------------ expert FFN
// The tile table of moe_expert_ffn by rows per expert (measured on MI355X,
// T tokens x top-8 of 256 experts, H = 6144, I = 256):
//   < 48    two launches, decode tile: while every expert fits one 64-row
//           chunk gate_up fills the workgroup slots in one round, so there
//           is no tail for down tasks to fill (8 rows per expert: one launch
//           157 us, two launches 140 us; uniform 32 and 40 rows: 196 / 182 us
//           and 206 / 196 us)
//   >= 48   one persistent launch, decode tile: once experts spill into a
//           second chunk, down tasks fill gate_up's light last round (uniform
//           48 rows: 222 against 255 us; Zipf T = 2048, 64 on average: 266
//           against 283 us).  In the MFMA-bound regime the launch still beats
//           the two launches with the large-M tile, since down overlaps
//           gate_up's tail and h stays in L2 (whole layer, uniform routing:
//           128 rows 599 -> 575 us, 256 rows 1058 -> 981 us, 512 rows
//           1996 -> 1885 us; same bytes out)
static constexpr int kFfnMinRows = 48;
static constexpr int kFfnSpinLimit = 1 << 20; // about a second of waiting for one chunk's h rows

size_t moe_expert_ffn_workspace_size(int32_t E, int64_t m_total, int32_t H, int32_t I) {
  if (E <= 0 || m_total < 0 || H <= 0 || I <= 0 || E > 4096 || m_total >= (int64_t(1) << 31)) return 0;
  return nvfp4::moe_ffn_ws_bytes(E, m_total, H, I);
}

int moe_expert_ffn(const nvfp4moe_ffn_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  if (!a) return fail(NVFP4MOE_ERR_INVALID, "moe_expert_ffn: args is NULL");
  if (!a->x_codes || !a->x_scales || !a->x_g || !a->perm_src_token || !a->offsets || !a->w_gu_packed ||
      !a->g_gu || !a->w_dn_packed || !a->g_dn || !a->g_h || !a->h_codes || !a->h_scales || !a->y)
    return fail(NVFP4MOE_ERR_INVALID, "moe_expert_ffn: null pointer argument");
  if (a->E <= 0 || a->H <= 0 || a->I <= 0 || a->m_total < 0 || a->x_rows <= 0)
    return fail(NVFP4MOE_ERR_INVALID, "moe_expert_ffn: E, H, I, x_rows must be > 0 and m_total >= 0");
  if (a->H % 32 != 0 || a->I % 16 != 0)
    return fail(NVFP4MOE_ERR_INVALID, "moe_expert_ffn: H=%d must be a multiple of 32 and I=%d of 16", a->H, a->I);
  if (a->I % 32 != 0 || a->I > 256)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "moe_expert_ffn: I=%d: the down GEMM runs one K step (I <= 256, I %% 32 == 0)",
                a->I);
  if (!aligned(a->x_codes, 16) || !aligned(a->x_scales, 2) || !aligned(a->w_gu_packed, 16) ||
      !aligned(a->w_dn_packed, 16) || !aligned(a->h_codes, 16) || !aligned(a->h_scales, 2) || !aligned(a->y, 16))
    return fail(NVFP4MOE_ERR_INVALID, "moe_expert_ffn: misaligned pointer");
  if (a->m_total >= (int64_t(1) << 31) || a->x_rows >= (int64_t(1) << 31) ||
      a->x_rows * (int64_t(a->H) / 2) >= (int64_t(1) << 31) || a->m_total * (int64_t(a->I) / 2) >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "moe_expert_ffn: operands of 2 GiB or more");
  if (static_cast<int64_t>(a->E) * a->H >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "moe_expert_ffn: E*H >= 2^31");
  if (a->E > 4096) return fail(NVFP4MOE_ERR_UNSUPPORTED, "moe_expert_ffn: E=%d > 4096", a->E);
  if (a->out) {
    if (!a->perm_of_assignment || !a->topk_w)
      return fail(NVFP4MOE_ERR_INVALID, "moe_expert_ffn: out needs perm_of_assignment and topk_w");
    if (a->T <= 0 || a->k <= 0 || static_cast<int64_t>(a->T) * a->k != a->m_total)
      return fail(NVFP4MOE_ERR_INVALID, "moe_expert_ffn: combine needs T, k > 0 with T * k == m_total");
    if (!aligned(a->out, 16) || !aligned(a->perm_of_assignment, 4) || !aligned(a->topk_w, 4))
      return fail(NVFP4MOE_ERR_INVALID, "moe_expert_ffn: misaligned combine pointer");
    if (prod_ge(a->m_total, int64_t(a->H) * 2, int64_t(1) << 31))
      return fail(NVFP4MOE_ERR_UNSUPPORTED, "moe_expert_ffn: the fused combine needs m_total * H * 2 < 2^31");
  }
  const size_t need = nvfp4::moe_ffn_ws_bytes(a->E, a->m_total, a->H, a->I);
  if (!workspace || workspace_bytes < need)
    return fail(NVFP4MOE_ERR_WORKSPACE, "moe_expert_ffn: workspace %zu < %zu bytes", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(NVFP4MOE_ERR_INVALID, "moe_expert_ffn: workspace not 256-byte aligned");
  if (a->m_total == 0) return ok();
  if (debug_checks()) {
    const hipStream_t ds = static_cast<hipStream_t>(stream);
    int st = debug_check_gemm("moe_expert_ffn", a->offsets, a->E, a->m_total, a->perm_src_token, a->x_rows, nullptr, 0,
                              ds, "perm_src_token");
    if (st == NVFP4MOE_OK && a->out)
      st = debug_check_range("moe_expert_ffn", "perm_of_assignment", a->perm_of_assignment, a->m_total, a->m_total, ds);
    if (st != NVFP4MOE_OK) return st;
  }
  nvfp4::GemmParams gu{};
  gu.a_codes = a->x_codes;
  gu.a_scales = a->x_scales;
  gu.a_g = a->x_g;
  gu.a_rows = a->perm_src_token;
  gu.b_packed = a->w_gu_packed;
  gu.b_g = a->g_gu;
  gu.offsets = a->offsets;
  gu.E = a->E;
  gu.N = 2 * a->I;
  gu.K = a->H;
  gu.m_total = static_cast<int>(a->m_total);
  gu.a_rows_total = static_cast<int>(a->x_rows);
  gu.out_codes = a->h_codes;
  gu.out_scales = a->h_scales;
  gu.out_g = a->g_h;
  nvfp4::GemmParams dn{};
  dn.a_codes = a->h_codes;
  dn.a_scales = a->h_scales;
  dn.a_g = a->g_h;
  dn.b_packed = a->w_dn_packed;
  dn.b_g = a->g_dn;
  dn.offsets = a->offsets;
  dn.E = a->E;
  dn.N = a->H;
  dn.K = a->I;
  dn.m_total = static_cast<int>(a->m_total);
  dn.a_rows_total = static_cast<int>(a->m_total);
  dn.out = a->y;
  const int64_t rows_per_expert = a->max_rows_per_expert_hint > 0 ? a->max_rows_per_expert_hint : a->m_total / a->E;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (rows_per_expert < kFfnMinRows) {
    hipError_t err = nvfp4::launch_grouped_gemm(gu, nvfp4::EPI_SWIGLU, a->m_total, a->max_rows_per_expert_hint, s);
    if (err != hipSuccess) return hip_status(err, "moe_expert_ffn (gate_up)");
    err = nvfp4::launch_grouped_gemm(dn, nvfp4::EPI_BF16, a->m_total, a->max_rows_per_expert_hint, s);
    if (err != hipSuccess || !a->out) return hip_status(err, "moe_expert_ffn (down)");
    return hip_status(nvfp4::launch_combine(a->y, 1, a->perm_of_assignment, a->topk_w, a->T, a->k, a->H, a->out, 1, s),
                      "moe_expert_ffn (combine)");
  }
  const nvfp4::FfnCombine comb{a->perm_of_assignment, a->topk_w, a->T, a->k, a->out};
  return hip_status(nvfp4::launch_moe_ffn(gu, dn, a->m_total, rows_per_expert >= 64, workspace, kFfnSpinLimit,
                                          a->out ? &comb : nullptr, s),
                    "moe_expert_ffn");
}

// ------------------------------------------------------------------ MXFP4
int mxfp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                   void* stream) {
  if (!x || !codes || !scales) return fail(NVFP4MOE_ERR_INVALID, "mxfp4_quantize: null pointer argument");
  if (x_dtype != NVFP4MOE_F32 && x_dtype != NVFP4MOE_BF16)
    return fail(NVFP4MOE_ERR_INVALID, "mxfp4_quantize: x_dtype %d", x_dtype);
  if (rows <= 0 || cols <= 0 || cols % 32 != 0)
    return fail(NVFP4MOE_ERR_INVALID, "mxfp4_quantize: rows > 0 and cols a positive multiple of 32 needed");
  if (prod_ge(rows, cols / 32, int64_t(1) << 38))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "mxfp4_quantize: tensor too large");
  if (!aligned(x, 16) || !aligned(codes, 16))
    return fail(NVFP4MOE_ERR_INVALID, "mxfp4_quantize: x and codes must be 16-byte aligned");
  return hip_status(nvfp4::launch_mx_quantize(x, x_dtype, rows, cols, codes, scales, static_cast<hipStream_t>(stream)),
                    "mxfp4_quantize");
}

int mxfp4_grouped_gemm(const nvfp4moe_gemm_args* a, void* stream) {
  if (!a) return fail(NVFP4MOE_ERR_INVALID, "mxfp4_grouped_gemm: args is NULL");
  if (!a->a_codes || !a->a_scales || !a->a_g || !a->b_g || !a->offsets)
    return fail(NVFP4MOE_ERR_INVALID, "mxfp4_grouped_gemm: null operand pointer");
  if (!a->b_packed && (!a->b_codes || !a->b_scales))
    return fail(NVFP4MOE_ERR_INVALID, "mxfp4_grouped_gemm: B needs b_codes and b_scales, or b_packed");
  if (a->E <= 0 || a->N <= 0 || a->K <= 0 || a->m_total < 0 || a->a_rows_total <= 0)
    return fail(NVFP4MOE_ERR_INVALID, "mxfp4_grouped_gemm: E, N, K, a_rows_total must be > 0 and m_total >= 0");
  if (a->K % 32 != 0) return fail(NVFP4MOE_ERR_INVALID, "mxfp4_grouped_gemm: K=%d not a multiple of 32", a->K);
  if (a->N % 16 != 0) return fail(NVFP4MOE_ERR_INVALID, "mxfp4_grouped_gemm: N=%d not a multiple of 16", a->N);
  if (!aligned(a->a_codes, 16) || !aligned(a->a_scales, 2) || !aligned(a->b_packed, 16) ||
      (!a->b_packed && (!aligned(a->b_codes, 16) || !aligned(a->b_scales, 2))))
    return fail(NVFP4MOE_ERR_INVALID, "mxfp4_grouped_gemm: codes and packed tiles must be 16-byte, scales 2-byte aligned");
  if (nvfp4::mx_packed_weight_bytes(1, a->N, a->K) >= (size_t(1) << 31))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "mxfp4_grouped_gemm: one expert's weights of 2 GiB or more");
  if (a->m_total >= (int64_t(1) << 31) || prod_ge(a->a_rows_total, a->K / 2, int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "mxfp4_grouped_gemm: A codes of 2 GiB or more");
  if (static_cast<int64_t>(a->E) * a->N >= (int64_t(1) << 31) ||
      static_cast<int64_t>(a->N) * (a->K / 2) >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "mxfp4_grouped_gemm: E*N or one expert's B codes (N*K/2) >= 2^31");
  switch (a->epilogue) {
    case NVFP4MOE_EPI_F32:
    case NVFP4MOE_EPI_BF16:
      if (!a->out && a->m_total > 0) return fail(NVFP4MOE_ERR_INVALID, "mxfp4_grouped_gemm: out is NULL");
      if (!aligned(a->out, 16)) return fail(NVFP4MOE_ERR_INVALID, "mxfp4_grouped_gemm: out not 16-byte aligned");
      break;
    case NVFP4MOE_EPI_SWIGLU_NVFP4:
      if (a->N % 64 != 0) return fail(NVFP4MOE_ERR_INVALID, "mxfp4_grouped_gemm: SwiGLU needs N = 2I with I %% 32 == 0");
      if (!a->out_codes || !a->out_scales)
        return fail(NVFP4MOE_ERR_INVALID, "mxfp4_grouped_gemm: SwiGLU needs out_codes, out_scales");
      break;
    default:
      return fail(NVFP4MOE_ERR_UNSUPPORTED, "mxfp4_grouped_gemm: epilogue %d (F32, BF16 or SwiGLU)", a->epilogue);
  }
  if (a->m_total == 0) return ok();
  if (debug_checks()) {
    const int st = debug_check_gemm("mxfp4_grouped_gemm", a->offsets, a->E, a->m_total, a->a_rows, a->a_rows_total,
                                    nullptr, 0, static_cast<hipStream_t>(stream));
    if (st != NVFP4MOE_OK) return st;
  }
  nvfp4::GemmParams prm{};
  prm.a_codes = a->a_codes;
  prm.a_scales = a->a_scales;
  prm.a_g = a->a_g;
  prm.a_rows = a->a_rows;
  prm.b_codes = a->b_codes;
  prm.b_scales = a->b_scales;
  prm.b_packed = a->b_packed;
  prm.b_g = a->b_g;
  prm.offsets = a->offsets;
  prm.E = a->E;
  prm.N = a->N;
  prm.K = a->K;
  prm.m_total = static_cast<int>(a->m_total);
  prm.a_rows_total = static_cast<int>(a->a_rows_total);
  prm.out = a->out;
  prm.out_codes = a->out_codes;
  prm.out_scales = a->out_scales;
  return hip_status(nvfp4::launch_mx_gemm(prm, a->epilogue, a->m_total, a->max_rows_per_expert_hint,
                                          static_cast<hipStream_t>(stream)),
                    "mxfp4_grouped_gemm");
}

size_t mxfp4_weight_packed_size(int32_t E, int32_t N, int32_t K) {
  if (E <= 0 || N <= 0 || K <= 0 || K % 32 != 0 || prod_ge(E, N, int64_t(1) << 31)) return 0;
  return nvfp4::mx_packed_weight_bytes(E, N, K);
}

int mxfp4_weight_repack(const uint8_t* codes, const uint8_t* scales, int32_t E, int32_t N, int32_t K,
                        uint8_t* packed, size_t packed_bytes, void* stream) {
  if (!codes || !scales || !packed) return fail(NVFP4MOE_ERR_INVALID, "mxfp4_weight_repack: null pointer argument");
  if (E <= 0 || N <= 0 || K <= 0) return fail(NVFP4MOE_ERR_INVALID, "mxfp4_weight_repack: E, N, K must be > 0");
  if (K % 32 != 0) return fail(NVFP4MOE_ERR_INVALID, "mxfp4_weight_repack: K=%d not a multiple of 32", K);
  if (!aligned(codes, 16) || !aligned(packed, 16))
    return fail(NVFP4MOE_ERR_INVALID, "mxfp4_weight_repack: codes and packed must be 16-byte aligned");
  if (static_cast<int64_t>(E) * N >= (int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "mxfp4_weight_repack: E*N >= 2^31");
  const size_t need = nvfp4::mx_packed_weight_bytes(E, N, K);
  if (packed_bytes < need)
    return fail(NVFP4MOE_ERR_WORKSPACE, "mxfp4_weight_repack: packed buffer %zu < %zu bytes", packed_bytes, need);
  return hip_status(nvfp4::launch_mx_repack(codes, scales, E, N, K, packed, static_cast<hipStream_t>(stream)),
                    "mxfp4_weight_repack");
}

// ------------------------------------------------------------------ FP8 block-scaled
int fp8_quantize(const void* x, int32_t x_dtype, int64_t batch, int64_t rows, int64_t cols, int32_t block_rows,
                 uint8_t* codes, float* scales, void* stream) {
  if (!x || !codes || !scales) return fail(NVFP4MOE_ERR_INVALID, "fp8_quantize: null pointer argument");
  if (x_dtype != NVFP4MOE_F32 && x_dtype != NVFP4MOE_BF16)
    return fail(NVFP4MOE_ERR_INVALID, "fp8_quantize: x_dtype %d", x_dtype);
  if (batch <= 0 || rows <= 0 || cols <= 0 || cols % 128 != 0)
    return fail(NVFP4MOE_ERR_INVALID, "fp8_quantize: batch, rows > 0 and cols a positive multiple of 128 needed");
  if (block_rows != 1 && block_rows != 128)
    return fail(NVFP4MOE_ERR_INVALID, "fp8_quantize: block_rows %d (1 or 128)", block_rows);
  // grid limits: 2^32 work-items per dimension, 65535 workgroups in y and z
  if (block_rows == 128 && (batch > 65535 || rows > 65535ll * 128 || cols / 128 >= (int64_t(1) << 24)))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "fp8_quantize: batch > 65535, rows > 8388480 or cols >= 2^31");
  if (block_rows == 1 && prod_ge(batch, rows, cols / 128, int64_t(1) << 26))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "fp8_quantize: 2^26 or more blocks of 128 values");
  if (prod_ge(batch, rows, cols / 128, int64_t(1) << 38))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "fp8_quantize: tensor too large");
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return fail(NVFP4MOE_ERR_INVALID, "fp8_quantize: x and codes must be 16-byte, scales 4-byte aligned");
  return hip_status(nvfp4::launch_fp8_quantize(x, x_dtype, batch, rows, cols, block_rows, codes, scales,
                                               static_cast<hipStream_t>(stream)),
                    "fp8_quantize");
}

int fp8_swiglu_quantize(const void* gate_up, int32_t dtype, int64_t M, int32_t I, uint8_t* codes, float* scales,
                        void* stream) {
  if (!gate_up || !codes || !scales) return fail(NVFP4MOE_ERR_INVALID, "fp8_swiglu_quantize: null pointer argument");
  if (dtype != NVFP4MOE_F32 && dtype != NVFP4MOE_BF16)
    return fail(NVFP4MOE_ERR_INVALID, "fp8_swiglu_quantize: dtype %d", dtype);
  if (M <= 0 || I <= 0 || I % 128 != 0)
    return fail(NVFP4MOE_ERR_INVALID, "fp8_swiglu_quantize: M > 0 and I a positive multiple of 128 needed");
  if (prod_ge(M, I / 128, int64_t(1) << 33))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "fp8_swiglu_quantize: 2^33 or more blocks of 128 values");
  if (!aligned(gate_up, 8) || !aligned(codes, 2) || !aligned(scales, 4))
    return fail(NVFP4MOE_ERR_INVALID, "fp8_swiglu_quantize: misaligned pointer");
  return hip_status(nvfp4::launch_fp8_swiglu(gate_up, dtype, M, I, codes, scales, static_cast<hipStream_t>(stream)),
                    "fp8_swiglu_quantize");
}

size_t fp8_weight_packed_size(int32_t E, int32_t N, int32_t K) {
  if (E <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || N % 16 != 0 ||
      prod_ge(E, N / 16, int64_t(K / 128) * 64, int64_t(1) << 40))
    return 0;
  return nvfp4::fp8_packed_weight_bytes(E, N, K);
}

int fp8_weight_repack(const uint8_t* codes, int32_t E, int32_t N, int32_t K, uint8_t* packed, size_t packed_bytes,
                      void* stream) {
  if (!codes || !packed) return fail(NVFP4MOE_ERR_INVALID, "fp8_weight_repack: null pointer argument");
  if (E <= 0 || N <= 0 || K <= 0) return fail(NVFP4MOE_ERR_INVALID, "fp8_weight_repack: E, N, K must be > 0");
  if (K % 128 != 0 || N % 16 != 0)
    return fail(NVFP4MOE_ERR_INVALID, "fp8_weight_repack: K=%d must be a multiple of 128, N=%d of 16", K, N);
  if (!aligned(codes, 16) || !aligned(packed, 16))
    return fail(NVFP4MOE_ERR_INVALID, "fp8_weight_repack: codes and packed must be 16-byte aligned");
  if (prod_ge(E, N / 16, int64_t(K / 128) * 64, int64_t(1) << 40))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "fp8_weight_repack: weights too large");
  const size_t need = nvfp4::fp8_packed_weight_bytes(E, N, K);
  if (packed_bytes < need)
    return fail(NVFP4MOE_ERR_WORKSPACE, "fp8_weight_repack: packed buffer %zu < %zu bytes", packed_bytes, need);
  return hip_status(nvfp4::launch_fp8_repack(codes, E, N, K, packed, static_cast<hipStream_t>(stream)),
                    "fp8_weight_repack");
}

int fp8_grouped_gemm(const nvfp4moe_fp8_gemm_args* a, void* stream) {
  if (!a) return fail(NVFP4MOE_ERR_INVALID, "fp8_grouped_gemm: args is NULL");
  if (!a->a_codes || !a->a_scales || !a->b_packed || !a->b_scales || !a->offsets)
    return fail(NVFP4MOE_ERR_INVALID, "fp8_grouped_gemm: null operand pointer");
  if (a->E <= 0 || a->N <= 0 || a->K <= 0 || a->m_total < 0 || a->a_rows_total <= 0)
    return fail(NVFP4MOE_ERR_INVALID, "fp8_grouped_gemm: E, N, K, a_rows_total must be > 0 and m_total >= 0");
  if (a->K % 128 != 0) return fail(NVFP4MOE_ERR_INVALID, "fp8_grouped_gemm: K=%d not a multiple of 128", a->K);
  if (a->N % 16 != 0) return fail(NVFP4MOE_ERR_INVALID, "fp8_grouped_gemm: N=%d not a multiple of 16", a->N);
  if (!aligned(a->a_codes, 16) || !aligned(a->a_scales, 4) || !aligned(a->b_packed, 16) || !aligned(a->b_scales, 4))
    return fail(NVFP4MOE_ERR_INVALID, "fp8_grouped_gemm: codes and packed tiles must be 16-byte, scales 4-byte aligned");
  if (a->E > 4096) return fail(NVFP4MOE_ERR_UNSUPPORTED, "fp8_grouped_gemm: E > 4096");
  if (a->m_total >= (int64_t(1) << 31) || prod_ge(a->a_rows_total, a->K, int64_t(1) << 31))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "fp8_grouped_gemm: A codes of 2 GiB or more");
  if (a->epilogue == NVFP4MOE_EPI_SWIGLU_NVFP4) {
    if (a->N % (2 * 128) != 0)
      return fail(NVFP4MOE_ERR_INVALID, "fp8_grouped_gemm: SwiGLU needs N = 2I with I %% 128 == 0 (N=%d)", a->N);
    if ((!a->out_codes || !a->out_scales) && a->m_total > 0)
      return fail(NVFP4MOE_ERR_INVALID, "fp8_grouped_gemm: SwiGLU needs out_codes and out_scales");
    if (!aligned(a->out_scales, 4)) return fail(NVFP4MOE_ERR_INVALID, "fp8_grouped_gemm: out_scales misaligned");
  } else {
    if (a->epilogue != NVFP4MOE_EPI_F32 && a->epilogue != NVFP4MOE_EPI_BF16)
      return fail(NVFP4MOE_ERR_UNSUPPORTED, "fp8_grouped_gemm: epilogue %d (F32, BF16 or SwiGLU)", a->epilogue);
    if (!a->out && a->m_total > 0) return fail(NVFP4MOE_ERR_INVALID, "fp8_grouped_gemm: out is NULL");
    if (!aligned(a->out, 16)) return fail(NVFP4MOE_ERR_INVALID, "fp8_grouped_gemm: out not 16-byte aligned");
  }
  if (a->m_total == 0) return ok();
  if (debug_checks()) {
    const int st = debug_check_gemm("fp8_grouped_gemm", a->offsets, a->E, a->m_total, a->a_rows, a->a_rows_total,
                                    nullptr, 0, static_cast<hipStream_t>(stream));
    if (st != NVFP4MOE_OK) return st;
  }
  nvfp4::Fp8Params prm{};
  prm.a_codes = a->a_codes;
  prm.a_scales = a->a_scales;
  prm.a_rows = a->a_rows;
  prm.b_packed = a->b_packed;
  prm.b_scales = a->b_scales;
  prm.offsets = a->offsets;
  prm.E = a->E;
  prm.N = a->N;
  prm.K = a->K;
  prm.m_total = static_cast<int>(a->m_total);
  prm.a_rows_total = static_cast<int>(a->a_rows_total);
  prm.out = a->out;
  prm.out_codes = a->out_codes;
  prm.out_scales = a->out_scales;
  return hip_status(nvfp4::launch_fp8_gemm(prm, a->epilogue, a->m_total, a->max_rows_per_expert_hint,
                                           static_cast<hipStream_t>(stream)),
                    "fp8_grouped_gemm");
}

// ------------------------------------------------------------------ packed weights
size_t nvfp4_weight_packed_size(int32_t E, int32_t N, int32_t K) {
  if (E <= 0 || N <= 0 || K <= 0 || K % 32 != 0 || prod_ge(E, N, int64_t(1) << 31)) return 0;
  return nvfp4::packed_weight_bytes(E, N, K);
}

int nvfp4_weight_repack(const uint8_t* codes, const uint8_t* scales, int32_t E, int32_t N, int32_t K,
                        uint8_t* packed, size_t packed_bytes, void* stream) {
  if (!codes || !scales || !packed) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_weight_repack: null pointer argument");
  if (E <= 0 || N <= 0 || K <= 0) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_weight_repack: E, N, K must be > 0");
  if (K % 32 != 0) return fail(NVFP4MOE_ERR_INVALID, "nvfp4_weight_repack: K=%d not a multiple of 32", K);
  if (!aligned(codes, 16) || !aligned(packed, 16))
    return fail(NVFP4MOE_ERR_INVALID, "nvfp4_weight_repack: codes and packed must be 16-byte aligned");
  if (static_cast<int64_t>(E) * N >= (int64_t(1) << 31)) return fail(NVFP4MOE_ERR_UNSUPPORTED, "nvfp4_weight_repack: E*N >= 2^31");
  const size_t need = nvfp4::packed_weight_bytes(E, N, K);
  if (packed_bytes < need)
    return fail(NVFP4MOE_ERR_WORKSPACE, "nvfp4_weight_repack: packed buffer %zu < %zu bytes", packed_bytes, need);
  return hip_status(nvfp4::launch_repack(codes, scales, E, N, K, packed, static_cast<hipStream_t>(stream)),
                    "nvfp4_weight_repack");
}

// ------------------------------------------------------------------ SwiGLU
size_t moe_swiglu_workspace_size(void) { return kSmallWs; }

int moe_swiglu(const void* gate_up, int32_t dtype, int64_t M, int32_t I, const float* g_in, float* g_out,
               uint8_t* codes, uint8_t* scales, void* workspace, size_t workspace_bytes, void* stream) {
  if (!gate_up || !codes || !scales) return fail(NVFP4MOE_ERR_INVALID, "moe_swiglu: null pointer argument");
  if (dtype != NVFP4MOE_F32 && dtype != NVFP4MOE_BF16) return fail(NVFP4MOE_ERR_INVALID, "moe_swiglu: dtype %d", dtype);
  if (M <= 0 || I <= 0) return fail(NVFP4MOE_ERR_INVALID, "moe_swiglu: M, I must be > 0");
  if (I % 16 != 0) return fail(NVFP4MOE_ERR_INVALID, "moe_swiglu: I=%d not a multiple of 16", I);
  if (!aligned(gate_up, 16) || !aligned(codes, 8)) return fail(NVFP4MOE_ERR_INVALID, "moe_swiglu: misaligned pointer");
  if (prod_ge(M, I / 16, int64_t(1) << 40)) return fail(NVFP4MOE_ERR_UNSUPPORTED, "moe_swiglu: tensor too large");
  if (!g_in && (!workspace || workspace_bytes < kSmallWs))
    return fail(NVFP4MOE_ERR_WORKSPACE, "moe_swiglu: workspace of %zu bytes needed when g_in is NULL", kSmallWs);
  return hip_status(nvfp4::launch_swiglu(gate_up, dtype, M, I, g_in, g_out, codes, scales, workspace,
                                         static_cast<hipStream_t>(stream)),
                    "moe_swiglu");
}

// ------------------------------------------------------------------ combine
int moe_unpermute_combine(const void* y, int32_t y_dtype, const int32_t* perm_of_assignment, const float* topk_w,
                          int32_t T, int32_t k, int32_t H, void* out, int32_t out_dtype, void* stream) {
  if (!y || !out) return fail(NVFP4MOE_ERR_INVALID, "moe_unpermute_combine: null y or out");
  if ((y_dtype != NVFP4MOE_F32 && y_dtype != NVFP4MOE_BF16) || (out_dtype != NVFP4MOE_F32 && out_dtype != NVFP4MOE_BF16))
    return fail(NVFP4MOE_ERR_INVALID, "moe_unpermute_combine: dtype");
  if (T <= 0 || k <= 0 || H <= 0) return fail(NVFP4MOE_ERR_INVALID, "moe_unpermute_combine: T, k, H must be > 0");
  if (H % 8 != 0) return fail(NVFP4MOE_ERR_INVALID, "moe_unpermute_combine: H=%d not a multiple of 8", H);
  if (!aligned(y, 16) || !aligned(out, 16)) return fail(NVFP4MOE_ERR_INVALID, "moe_unpermute_combine: misaligned");
  if (static_cast<int64_t>(T) * k >= (int64_t(1) << 31)) return fail(NVFP4MOE_ERR_UNSUPPORTED, "moe_unpermute_combine: T*k too large");
  if (debug_checks()) {
    // the rows the routing calls produce: T * k
    const int st = debug_check_range("moe_unpermute_combine", "perm_of_assignment", perm_of_assignment,
                                     static_cast<int64_t>(T) * k, static_cast<int64_t>(T) * k,
                                     static_cast<hipStream_t>(stream));
    if (st != NVFP4MOE_OK) return st;
  }
  return hip_status(nvfp4::launch_combine(y, y_dtype, perm_of_assignment, topk_w, T, k, H, out, out_dtype,
                                          static_cast<hipStream_t>(stream)),
                    "moe_unpermute_combine");
}

}  // extern "C"
