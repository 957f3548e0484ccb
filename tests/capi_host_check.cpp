// Host-side check of the C ABI's argument validation, built with the host
// code of the library's entry points under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_capi_sanitized.py builds and runs
// it).  Every call below must be rejected (or be an empty problem) before
// anything is enqueued, so no device is touched: the device pointers are fake
// addresses that are never dereferenced.  Extreme sizes (INT32_MAX,
// INT64_MAX, negative values) exercise the size arithmetic of the checks and
// of the workspace-size queries, where a signed overflow would be reported by
// the sanitizer.  Prints one line per failed expectation and exits nonzero if
// any failed.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "nvfp4moe.h"

static int g_failed = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, nvfp4moe_last_error_detail());
    ++g_failed;
  }
}

static void expect_true(const char* what, bool ok) {
  if (!ok) {
    printf("FAIL %s\n", what);
    ++g_failed;
  }
}

static void* const F = reinterpret_cast<void*>(uintptr_t(1) << 20);        // aligned, never dereferenced
static void* const FM = reinterpret_cast<void*>((uintptr_t(1) << 20) + 2); // misaligned
static const int32_t I32MAX = 2147483647;
static const int64_t I64MAX = INT64_MAX;

template <class T>
static T* p(void* v) { return static_cast<T*>(v); }

static nvfp4moe_gemm_args gemm_args() {
  nvfp4moe_gemm_args a;
  memset(&a, 0, sizeof(a));
  a.a_codes = p<uint8_t>(F); a.a_scales = p<uint8_t>(F); a.a_g = p<float>(F); a.a_rows_total = 16;
  a.b_codes = p<uint8_t>(F); a.b_scales = p<uint8_t>(F); a.b_g = p<float>(F); a.offsets = p<int32_t>(F);
  a.E = 4; a.N = 64; a.K = 128; a.m_total = 16; a.epilogue = NVFP4MOE_EPI_F32; a.out = F;
  return a;
}

static nvfp4moe_fp8_gemm_args fp8_args() {
  nvfp4moe_fp8_gemm_args a;
  memset(&a, 0, sizeof(a));
  a.a_codes = p<uint8_t>(F); a.a_scales = p<float>(F); a.a_rows_total = 16; a.b_packed = p<uint8_t>(F);
  a.b_scales = p<float>(F); a.offsets = p<int32_t>(F); a.E = 4; a.N = 64; a.K = 256; a.m_total = 16;
  a.epilogue = NVFP4MOE_EPI_F32; a.out = F;
  return a;
}

static nvfp4moe_ffn_args ffn_args() {
  nvfp4moe_ffn_args a;
  memset(&a, 0, sizeof(a));
  a.x_codes = p<uint8_t>(F); a.x_scales = p<uint8_t>(F); a.x_g = p<float>(F); a.x_rows = 16;
  a.perm_src_token = p<int32_t>(F); a.offsets = p<int32_t>(F); a.E = 4; a.H = 256; a.I = 128; a.m_total = 32;
  a.w_gu_packed = p<uint8_t>(F); a.g_gu = p<float>(F); a.w_dn_packed = p<uint8_t>(F); a.g_dn = p<float>(F);
  a.g_h = p<float>(F); a.h_codes = p<uint8_t>(F); a.h_scales = p<uint8_t>(F); a.y = F;
  return a;
}

int main() {
  // ---------------------------------------------------------------- status
  for (int s = -3; s < 10; ++s) expect_true("status string", nvfp4moe_status_string(s) != nullptr);
  expect_true("version", nvfp4moe_version() >= 100);

  // ---------------------------------------------------------------- workspace queries at extremes
  volatile size_t sink = 0;
  const int32_t i32s[] = {-1, 0, 1, 7, 4096, 4097, I32MAX};
  for (int32_t T : i32s)
    for (int32_t E : i32s)
      for (int32_t k : {-1, 0, 1, 8, 32, 33, I32MAX}) {
        sink += moe_route_permute_workspace_size(T, E, k);
        sink += moe_route_quantize_workspace_size(T, E, k);
      }
  for (int32_t E : i32s)
    for (int64_t m : {int64_t(-1), int64_t(0), int64_t(1), int64_t(1) << 40, I64MAX})
      for (int32_t H : {-1, 0, 256, I32MAX})
        for (int32_t I : {-1, 0, 128, 256, I32MAX}) sink += moe_expert_ffn_workspace_size(E, m, H, I);
  for (int32_t E : i32s)
    for (int32_t N : i32s)
      for (int32_t K : {-1, 0, 32, 128, 4096, I32MAX}) {
        sink += nvfp4_weight_packed_size(E, N, K);
        sink += mxfp4_weight_packed_size(E, N, K);
        sink += fp8_weight_packed_size(E, N, K);
      }
  sink += nvfp4_quantize_workspace_size() + moe_swiglu_workspace_size() + moe_route_quantize_noalloc_max_workspace();
  (void)sink;

  // ---------------------------------------------------------------- route / quantize
  const size_t ws = size_t(1) << 20;
  expect("route null logits", moe_route_permute(nullptr, 4, 8, 2, p<int32_t>(F), p<float>(F), p<int32_t>(F),
                                                p<int32_t>(F), p<int32_t>(F), p<int32_t>(F), nullptr, F, ws, nullptr),
         NVFP4MOE_ERR_INVALID);
  for (int32_t T : {-5, 0})
    expect("route T", moe_route_permute(p<float>(F), T, 8, 2, p<int32_t>(F), p<float>(F), p<int32_t>(F),
                                        p<int32_t>(F), p<int32_t>(F), p<int32_t>(F), nullptr, F, ws, nullptr),
           NVFP4MOE_ERR_INVALID);
  expect("route huge T", moe_route_permute(p<float>(F), I32MAX, 256, 32, p<int32_t>(F), p<float>(F), p<int32_t>(F),
                                           p<int32_t>(F), p<int32_t>(F), p<int32_t>(F), nullptr, F, ws, nullptr),
         NVFP4MOE_ERR_UNSUPPORTED);
  expect("route k > E", moe_route_permute(p<float>(F), 4, 8, 9, p<int32_t>(F), p<float>(F), p<int32_t>(F),
                                          p<int32_t>(F), p<int32_t>(F), p<int32_t>(F), nullptr, F, ws, nullptr),
         NVFP4MOE_ERR_INVALID);
  expect("route workspace", moe_route_permute(p<float>(F), 4, 8, 2, p<int32_t>(F), p<float>(F), p<int32_t>(F),
                                              p<int32_t>(F), p<int32_t>(F), p<int32_t>(F), nullptr, F, 4, nullptr),
         NVFP4MOE_ERR_WORKSPACE);
  expect("quantize cols", nvfp4_quantize(F, NVFP4MOE_BF16, 4, 48, nullptr, nullptr, p<uint8_t>(F), p<uint8_t>(F), F,
                                         256, nullptr),
         NVFP4MOE_ERR_INVALID);
  expect("quantize misaligned", nvfp4_quantize(FM, NVFP4MOE_BF16, 4, 64, nullptr, nullptr, p<uint8_t>(F),
                                               p<uint8_t>(F), F, 256, nullptr),
         NVFP4MOE_ERR_INVALID);
  {
    const int st = nvfp4_quantize(F, NVFP4MOE_F32, I64MAX, I64MAX / 32 * 32, nullptr, nullptr, p<uint8_t>(F),
                                  p<uint8_t>(F), F, ws, nullptr);
    expect_true("quantize huge rejected", st == NVFP4MOE_ERR_UNSUPPORTED || st == NVFP4MOE_ERR_INVALID);
  }
  expect("route_quantize cols", moe_route_quantize(p<float>(F), 16, 8, 2, p<int32_t>(F), p<float>(F), p<int32_t>(F),
                                                   p<int32_t>(F), p<int32_t>(F), p<int32_t>(F), nullptr, F,
                                                   NVFP4MOE_BF16, 48, nullptr, nullptr, p<uint8_t>(F), p<uint8_t>(F),
                                                   F, ws, nullptr),
         NVFP4MOE_ERR_INVALID);
  {
    const int st = moe_route_quantize(p<float>(F), I32MAX, 4096, 32, p<int32_t>(F), p<float>(F), p<int32_t>(F),
                                      p<int32_t>(F), p<int32_t>(F), p<int32_t>(F), nullptr, F, NVFP4MOE_BF16,
                                      I64MAX / 32 * 32, nullptr, nullptr, p<uint8_t>(F), p<uint8_t>(F), F, ws,
                                      nullptr);
    expect_true("route_quantize huge rejected", st != NVFP4MOE_OK);
  }
  expect("noalloc too large", moe_route_quantize_noalloc(p<float>(F), 200000, 256, 8, p<int32_t>(F), p<float>(F),
                                                         p<int32_t>(F), p<int32_t>(F), p<int32_t>(F), p<int32_t>(F),
                                                         nullptr, F, NVFP4MOE_BF16, 64, nullptr, nullptr,
                                                         p<uint8_t>(F), p<uint8_t>(F), nullptr),
         NVFP4MOE_ERR_UNSUPPORTED);

  // ---------------------------------------------------------------- grouped GEMMs
  expect("gemm null", nvfp4_grouped_gemm(nullptr, nullptr), NVFP4MOE_ERR_INVALID);
  {
    nvfp4moe_gemm_args a = gemm_args(); a.K = 48;
    expect("gemm K", nvfp4_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_INVALID);
    a = gemm_args(); a.E = I32MAX; a.N = I32MAX - 15; a.K = I32MAX - 31;
    expect_true("gemm huge rejected", nvfp4_grouped_gemm(&a, nullptr) != NVFP4MOE_OK);
    a = gemm_args(); a.a_rows_total = I64MAX; a.K = I32MAX - 31;
    expect("gemm huge A", nvfp4_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
    a = gemm_args(); a.m_total = I64MAX;
    expect("gemm huge m_total", nvfp4_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
    a = gemm_args(); a.m_total = -1;
    expect("gemm negative m_total", nvfp4_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_INVALID);
    a = gemm_args(); a.m_total = 0;
    expect("gemm empty", nvfp4_grouped_gemm(&a, nullptr), NVFP4MOE_OK);
    a = gemm_args(); a.out = FM;
    expect("gemm out misaligned", nvfp4_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_INVALID);
    expect("mx gemm out misaligned", mxfp4_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_INVALID);
    a = gemm_args(); a.K = I32MAX - 31;
    expect_true("mx gemm huge K rejected", mxfp4_grouped_gemm(&a, nullptr) != NVFP4MOE_OK);
    a = gemm_args(); a.epilogue = NVFP4MOE_EPI_COMBINE_F32;
    expect("mx gemm combine", mxfp4_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
    a = gemm_args(); a.m_total = 0;
    expect("mx gemm empty", mxfp4_grouped_gemm(&a, nullptr), NVFP4MOE_OK);
  }
  {
    nvfp4moe_fp8_gemm_args a = fp8_args(); a.K = 192;
    expect("fp8 gemm K", fp8_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_INVALID);
    a = fp8_args(); a.a_rows_total = I64MAX;
    expect("fp8 gemm huge A", fp8_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
    a = fp8_args(); a.E = 5000;
    expect("fp8 gemm E", fp8_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
    a = fp8_args(); a.epilogue = NVFP4MOE_EPI_COMBINE_F32;
    expect("fp8 gemm epilogue", fp8_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
    a = fp8_args(); a.epilogue = NVFP4MOE_EPI_SWIGLU_NVFP4;
    expect("fp8 gemm swiglu N", fp8_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_INVALID);
    a = fp8_args(); a.epilogue = NVFP4MOE_EPI_SWIGLU_NVFP4; a.N = 512;
    expect("fp8 gemm swiglu outputs", fp8_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_INVALID);
    a.out_codes = p<uint8_t>(F); a.out_scales = p<float>(FM);
    expect("fp8 gemm swiglu scales misaligned", fp8_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_INVALID);
    a = fp8_args(); a.m_total = 0;
    expect("fp8 gemm empty", fp8_grouped_gemm(&a, nullptr), NVFP4MOE_OK);
    a = fp8_args(); a.out = FM;
    expect("fp8 gemm out misaligned", fp8_grouped_gemm(&a, nullptr), NVFP4MOE_ERR_INVALID);
    expect("fp8 gemm null", fp8_grouped_gemm(nullptr, nullptr), NVFP4MOE_ERR_INVALID);
  }
  expect("fp8 quantize block_rows", fp8_quantize(F, NVFP4MOE_F32, 1, 4, 128, 64, p<uint8_t>(F), p<float>(F), nullptr),
         NVFP4MOE_ERR_INVALID);
  expect("fp8 quantize huge", fp8_quantize(F, NVFP4MOE_F32, I64MAX, I64MAX, I64MAX / 128 * 128, 1, p<uint8_t>(F),
                                           p<float>(F), nullptr),
         NVFP4MOE_ERR_UNSUPPORTED);
  expect("fp8 repack N", fp8_weight_repack(p<uint8_t>(F), 2, 24, 128, p<uint8_t>(F), size_t(1) << 30, nullptr),
         NVFP4MOE_ERR_INVALID);
  expect("fp8 repack huge", fp8_weight_repack(p<uint8_t>(F), I32MAX, I32MAX - 15, I32MAX - 127, p<uint8_t>(F),
                                              SIZE_MAX, nullptr),
         NVFP4MOE_ERR_UNSUPPORTED);
  expect("mx quantize cols", mxfp4_quantize(F, NVFP4MOE_BF16, 4, 48, p<uint8_t>(F), p<uint8_t>(F), nullptr),
         NVFP4MOE_ERR_INVALID);
  expect("mx quantize huge", mxfp4_quantize(F, NVFP4MOE_BF16, I64MAX, I64MAX / 32 * 32, p<uint8_t>(F),
                                            p<uint8_t>(F), nullptr),
         NVFP4MOE_ERR_UNSUPPORTED);
  expect("mx repack huge", mxfp4_weight_repack(p<uint8_t>(F), p<uint8_t>(F), I32MAX, I32MAX, I32MAX - 31,
                                               p<uint8_t>(F), SIZE_MAX, nullptr),
         NVFP4MOE_ERR_UNSUPPORTED);
  expect("nvfp4 repack workspace", nvfp4_weight_repack(p<uint8_t>(F), p<uint8_t>(F), 2, 64, 256, p<uint8_t>(F), 16,
                                                       nullptr),
         NVFP4MOE_ERR_WORKSPACE);

  // ---------------------------------------------------------------- expert FFN
  {
    const size_t fws = size_t(1) << 24;
    expect("ffn null", moe_expert_ffn(nullptr, F, fws, nullptr), NVFP4MOE_ERR_INVALID);
    nvfp4moe_ffn_args a = ffn_args(); a.I = 512;
    expect("ffn I", moe_expert_ffn(&a, F, fws, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
    a = ffn_args(); a.E = 5000;
    expect("ffn E", moe_expert_ffn(&a, F, fws, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
    a = ffn_args(); a.m_total = I64MAX;
    expect_true("ffn huge m_total rejected", moe_expert_ffn(&a, F, fws, nullptr) != NVFP4MOE_OK);
    a = ffn_args(); a.x_rows = I64MAX; a.H = I32MAX - 31;
    expect_true("ffn huge x rejected", moe_expert_ffn(&a, F, fws, nullptr) != NVFP4MOE_OK);
    a = ffn_args();
    expect("ffn workspace", moe_expert_ffn(&a, F, 8, nullptr), NVFP4MOE_ERR_WORKSPACE);
    expect("ffn misaligned workspace", moe_expert_ffn(&a, FM, fws, nullptr), NVFP4MOE_ERR_INVALID);
    a = ffn_args(); a.m_total = 0;
    expect("ffn empty", moe_expert_ffn(&a, F, fws, nullptr), NVFP4MOE_OK);
    // the fused combine's arguments
    a = ffn_args(); a.out = F;
    expect("ffn combine without perm", moe_expert_ffn(&a, F, fws, nullptr), NVFP4MOE_ERR_INVALID);
    a = ffn_args(); a.out = F; a.perm_of_assignment = p<int32_t>(F); a.topk_w = p<float>(F); a.T = 5; a.k = 8;
    expect("ffn combine T*k != m_total", moe_expert_ffn(&a, F, fws, nullptr), NVFP4MOE_ERR_INVALID);
    a.T = 4; a.k = 8; a.out = FM;
    expect("ffn combine misaligned out", moe_expert_ffn(&a, F, fws, nullptr), NVFP4MOE_ERR_INVALID);
    a.out = F; a.T = I32MAX; a.k = I32MAX;
    expect("ffn combine huge T*k", moe_expert_ffn(&a, F, fws, nullptr), NVFP4MOE_ERR_INVALID);
  }

  // ---------------------------------------------------------------- swiglu / combine
  expect("swiglu I", moe_swiglu(F, NVFP4MOE_F32, 4, 24, p<float>(F), nullptr, p<uint8_t>(F), p<uint8_t>(F), nullptr,
                                0, nullptr),
         NVFP4MOE_ERR_INVALID);
  expect_true("swiglu huge rejected", moe_swiglu(F, NVFP4MOE_F32, I64MAX, I32MAX - 15, p<float>(F), nullptr,
                                                 p<uint8_t>(F), p<uint8_t>(F), nullptr, 0, nullptr) != NVFP4MOE_OK);
  expect("combine H", moe_unpermute_combine(F, NVFP4MOE_BF16, p<int32_t>(F), p<float>(F), 4, 2, 12, F, NVFP4MOE_BF16,
                                            nullptr),
         NVFP4MOE_ERR_INVALID);
  expect_true("combine huge rejected", moe_unpermute_combine(F, NVFP4MOE_BF16, p<int32_t>(F), p<float>(F), I32MAX,
                                                             I32MAX, I32MAX - 7, F, NVFP4MOE_BF16,
                                                             nullptr) != NVFP4MOE_OK);

  printf("%s: %d failed\n", g_failed ? "FAILED" : "ok", g_failed);
  return g_failed ? 1 : 0;
}
