// Internal declarations shared by the HIP sources of libnvfp4moe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_budget.h"
#include "nvfp4_device.h"

namespace nvfp4 {

enum : int { EPI_F32 = 0, EPI_BF16 = 1, EPI_SWIGLU = 2, EPI_COMBINE = 3 };

// Kernel-side arguments of the grouped GEMM (validated on the host first).
struct GemmParams {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_g;
  const int32_t* a_rows;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const uint8_t* b_packed;   // packed weight tiles (nvfp4_weight_repack) or nullptr
  const float* b_g;
  const int32_t* offsets;
  int E, N, K;
  int n_tiles;            // column tiles per expert (set by the launcher)
  int slots;              // workgroups of the kernel resident at once (set by the launcher)
  int m_total;            // rows of the outputs indexed by GEMM row
  int a_rows_total;       // rows of A (bound for gathered row indices)
  int out_rows;           // rows of the combine accumulator
  void* out;
  uint8_t* out_codes;
  uint8_t* out_scales;
  const float* out_g;
  const int32_t* row_token;
  const float* row_weight;
};

size_t route_permute_ws_bytes(int T, int E, int k);
hipError_t launch_route_permute(const float* logits, int T, int E, int k, int* topk_ids, float* topk_w,
                                int* counts, int* offsets, int* perm_src_token, int* perm_of_assignment,
                                float* perm_weight, void* ws, hipStream_t stream);
size_t route_quantize_ws_bytes(int T, int E, int k);
hipError_t launch_route_quantize(const float* logits, int T, int E, int k, int* topk_ids, float* topk_w,
                                 int* counts, int* offsets, int* perm_src_token, int* perm_of_assignment,
                                 float* perm_weight, const void* x, int dtype, int64_t cols, const float* g_in,
                                 float* g_out, uint8_t* codes, uint8_t* scales, void* ws, hipStream_t stream);
hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t cols, const float* g_in, float* g_out,
                           uint8_t* codes, uint8_t* scales, void* ws, hipStream_t stream);
hipError_t launch_swiglu(const void* y, int dtype, int64_t M, int I, const float* g_in, float* g_out,
                         uint8_t* codes, uint8_t* scales, void* ws, hipStream_t stream);
hipError_t launch_combine(const void* y, int y_dtype, const int* perm, const float* w, int T, int k, int H,
                          void* out, int out_dtype, hipStream_t stream);
size_t packed_weight_bytes(int E, int N, int K);
hipError_t launch_repack(const uint8_t* codes, const uint8_t* scales, int E, int N, int K, uint8_t* packed,
                         hipStream_t stream);
hipError_t launch_grouped_gemm(const GemmParams& prm, int epilogue, int64_t m_total, int hint, hipStream_t stream);
bool gemm_large_fits(const GemmParams& prm, int64_t rows_per_expert);
hipError_t launch_gemm_large(const GemmParams& prm, int epilogue, int64_t m_total, hipStream_t stream);
hipError_t launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream);
hipError_t launch_mx_gemm(const GemmParams& prm, int epilogue, int64_t m_total, int hint, hipStream_t stream);
size_t mx_packed_weight_bytes(int E, int N, int K);

hipError_t launch_mx_repack(const uint8_t* codes, const uint8_t* scales, int E, int N, int K, uint8_t* packed,
                            hipStream_t stream);
size_t moe_ffn_ws_bytes(int E, int64_t m_total, int H, int I);
// the weighted top-k combine fused into the expert-FFN launch
struct FfnCombine {
  const int32_t* perm_of;   // [T, k] row of assignment (t, j)
  const float* topk_w;      // [T, k]
  int T, k;
  void* out;                // bf16 [T, H]
};
hipError_t launch_moe_ffn(GemmParams gu, GemmParams dn, int64_t m_total, bool cached, void* ws, int spin_limit,
                          const FfnCombine* comb, hipStream_t stream);

// Kernel-side arguments of the grouped FP8 GEMM (validated on the host first).
struct Fp8Params {
  const uint8_t* a_codes;
  const float* a_scales;       // [a_rows_total, K/128]
  const int32_t* a_rows;
  const uint8_t* b_packed;
  const float* b_scales;       // [E, ceil(N/128), K/128]
  const int32_t* offsets;
  int E, N, K, m_total, a_rows_total;
  void* out;
  uint8_t* out_codes;          // SwiGLU epilogue: h E4M3 codes [m_total, N/2]
  float* out_scales;           // SwiGLU epilogue: h block scales [m_total, N/256]
};

hipError_t launch_fp8_quantize(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols, int block_rows,
                               uint8_t* codes, float* scales, hipStream_t stream);
size_t fp8_packed_weight_bytes(int E, int N, int K);
hipError_t launch_fp8_swiglu(const void* y, int dtype, int64_t M, int I, uint8_t* codes, float* scales,
                             hipStream_t stream);
hipError_t launch_fp8_repack(const uint8_t* codes, int E, int N, int K, uint8_t* packed, hipStream_t stream);
hipError_t launch_fp8_gemm(const Fp8Params& p, int epilogue, int64_t m_total, int hint, hipStream_t stream);

}  // namespace nvfp4
