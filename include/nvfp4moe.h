/*
 * nvfp4moe — NVFP4 block-scaled Mixture-of-Experts layer for AMD MI355X (gfx950).
 *
 * Plain C ABI.  Every pointer argument is a DEVICE pointer unless stated
 * otherwise; sizes are host integers.  Every compute call enqueues its kernels
 * on `stream` (a hipStream_t passed as void*, NULL = the null stream), returns
 * without synchronising the host, and allocates nothing: the caller owns every
 * buffer, including workspaces.  The library keeps no pointer past the work it
 * enqueued and holds no global state, so calls on different streams may run
 * concurrently (calls that share a workspace or an output must not overlap).
 *
 * Number format (the block-scaled MMA described in "From Empirical Limits to
 * Research-Driven Optimization: The SM120 FP4 Kernel Research Campaign",
 * section "Section 1: CUTLASS Kernels - The Foundation": E2M1 operands, one
 * unsigned E4M3 block scale per 16 elements along K, FP32 accumulation), plus a
 * float32 per-tensor scale:
 *   codes   uint8 [rows, cols/2]   two E2M1 codes per byte, element 2i in the
 *                                  low nibble of byte i, row-major, blocks run
 *                                  along the last (reduction) axis
 *   scales  uint8 [rows, cols/16]  one E4M3 code per 16-element block
 *   g       float32 (device)       per-tensor scale; value = E2M1*E4M3*g
 *
 * Quantiser (a reading of the pages, which print none):
 *   g = amax/2688, block scale = E4M3_satfinite((absmax_b/6)/g) (nearest even),
 *   code = E2M1(x / (scale*g)) (nearest even, saturating at 6, sign copied from
 *   x, a zero block scale gives code 0).  All decisions in float32 with correctly
 *   rounded division, so codes are reproducible bit for bit.
 *
 * Errors: every call validates its arguments on the host BEFORE enqueuing
 * anything.  A non-OK status means nothing was enqueued, except
 * NVFP4MOE_ERR_HIP, which reports a failed kernel launch (earlier kernels of
 * the same call may have been enqueued).  nvfp4moe_last_error_detail() gives a
 * thread-local explanation of the last failure on the calling thread.  The
 * *_workspace_size() and *_packed_size() queries return 0 for arguments the
 * matching call rejects.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4moe_status {
  NVFP4MOE_OK = 0,
  NVFP4MOE_ERR_INVALID = 1,      /* null pointer, negative/zero size, k > E, K % 32 != 0, misaligned pointer */
  NVFP4MOE_ERR_UNSUPPORTED = 2,  /* valid request outside what the compiled kernels cover (size limits) */
  NVFP4MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the *_workspace_size() query */
  NVFP4MOE_ERR_HIP = 4           /* the HIP runtime rejected a kernel launch */
} nvfp4moe_status;

/* Index arrays that live on the device (expert offsets, gathered rows,
 * combine rows) are not read by the host: the kernels clamp entries that
 * break the documented ranges, which then gives wrong rows but never an
 * access outside a buffer.  With the environment variable NVFP4MOE_DEBUG set
 * (to anything but "" or "0"; read at every call) the grouped GEMMs,
 * moe_expert_ffn and moe_unpermute_combine first copy those arrays to the
 * host and check them (offsets non-decreasing from 0 to at most m_total,
 * gathered rows in [0, a_rows_total), combine rows in [0, T * k) or
 * [0, out_rows)), returning NVFP4MOE_ERR_INVALID with the first bad entry in
 * nvfp4moe_last_error_detail() before any launch.  The copies synchronise
 * the stream: a debugging aid, not for use under graph capture. */

typedef enum nvfp4moe_dtype {
  NVFP4MOE_F32 = 0,
  NVFP4MOE_BF16 = 1
} nvfp4moe_dtype;

typedef enum nvfp4moe_epilogue {
  /* y[p, n] = acc * (g_a * g_b[e]) written as float32 to out[p*N + n], p < m_total */
  NVFP4MOE_EPI_F32 = 0,
  /* same, rounded to bfloat16 (nearest even) */
  NVFP4MOE_EPI_BF16 = 1,
  /* SwiGLU + NVFP4 re-quantisation of the gate_up output (N = 2I):
   * h[p, i] = silu(y[p, i]) * y[p, I + i]  (rows [0,I) of each expert's B are the
   * gate, rows [I,2I) the up projection), quantised with the caller's per-tensor
   * scale *out_g into out_codes [m_total, I/2] and out_scales [m_total, I/16].
   * Requires I % 16 == 0. */
  NVFP4MOE_EPI_SWIGLU_NVFP4 = 2,
  /* weighted scatter-add (the combine fused into the down GEMM):
   * out[row_token[p]*N + n] += row_weight[p] * y[p, n]   (float32 atomics;
   * out is float32 [out_rows, N] and must be zeroed by the caller; the order of
   * the additions is not fixed, so results may differ in the last bits between
   * runs). */
  NVFP4MOE_EPI_COMBINE_F32 = 3
} nvfp4moe_epilogue;

/* Arguments of nvfp4_grouped_gemm (a struct keeps the ABI stable). */
typedef struct nvfp4moe_gemm_args {
  /* A operand: NVFP4 rows (activations). */
  const uint8_t* a_codes;     /* [a_rows_total, K/2], 16-byte aligned */
  const uint8_t* a_scales;    /* [a_rows_total, K/16] */
  const float* a_g;           /* device, 1 float */
  const int32_t* a_rows;      /* device [m_total]: A row read by GEMM row p, or NULL for row p.
                                 Every entry must lie in [0, a_rows_total). */
  int64_t a_rows_total;
  /* B operand: per-expert NVFP4 weights, row n of expert e is output column n. */
  const uint8_t* b_codes;     /* [E, N, K/2], 16-byte aligned */
  const uint8_t* b_scales;    /* [E, N, K/16] */
  const float* b_g;           /* device [E]: one per-tensor scale per expert */
  /* grouping: rows [offsets[e], offsets[e+1]) of the GEMM belong to expert e. */
  const int32_t* offsets;     /* device [E+1], non-decreasing, offsets[0] = 0, offsets[E] <= m_total */
  int32_t E;
  int32_t N;                  /* multiple of 16 */
  int32_t K;                  /* multiple of 32 */
  int64_t m_total;            /* host-side bound on offsets[E] (rows of out) */
  int32_t epilogue;           /* nvfp4moe_epilogue */
  void* out;                  /* EPI_F32: float [m_total, N]; EPI_BF16: bf16 [m_total, N]
                                 (16-byte aligned: rows leave as 16-byte stores);
                                 EPI_COMBINE_F32: float [out_rows, N]; unused for SWIGLU */
  int64_t out_rows;           /* EPI_COMBINE_F32: rows of the accumulator (tokens) */
  uint8_t* out_codes;         /* EPI_SWIGLU_NVFP4 */
  uint8_t* out_scales;        /* EPI_SWIGLU_NVFP4 */
  const float* out_g;         /* EPI_SWIGLU_NVFP4: device, 1 float, > 0 */
  const int32_t* row_token;   /* EPI_COMBINE_F32: device [m_total], values in [0, out_rows) */
  const float* row_weight;    /* EPI_COMBINE_F32: device [m_total] */
  int32_t max_rows_per_expert_hint;  /* rows per expert the caller expects (the pages' tune_max_num_tokens);
                                        0: m_total / E.  Picks the tile shape (>= 128: the large-M tile)
                                        and the weight-load cache policy (>= 64: cached, else
                                        non-temporal); never changes the result. */
  /* Optional: B in the packed tile layout written by nvfp4_weight_repack (16-byte
     aligned).  When set, b_codes / b_scales are not read (and may be NULL). */
  const uint8_t* b_packed;
} nvfp4moe_gemm_args;

/* ---------------------------------------------------------------- route + permute
 * Top-k routing and the expert-first permutation ("Discovering SM120-Specific
 * CUTLASS MoE Kernels", section "Input Knowledge Required": a router picks
 * experts per token; "From Empirical Limits ...", section "Sections 5-6:
 * Algorithmic Techniques": expert-first layout, token reordering).
 *   logits             float32 [T, E]
 *   topk_ids   (out)   int32 [T, k]   k largest logits by descending value, ties to the lower id
 *   topk_w     (out)   float32 [T, k] exp(l_j - l_max) / sum over the k chosen (softmax over E,
 *                                     renormalised over the k), computed in float64
 *   counts     (out)   int32 [E]      assignments per expert
 *   offsets    (out)   int32 [E+1]    exclusive prefix sum of counts
 *   perm_src_token     (out) int32 [T*k]  token of permuted row p
 *   perm_of_assignment (out) int32 [T*k]  permuted row of assignment t*k+j
 *   perm_weight        (out, nullable) float32 [T*k]  topk_w of permuted row p
 * Rows of one expert keep ascending t*k+j (stable): every output is
 * deterministic and bit-exact.  Limits: 1 <= k <= min(E, 32), E <= 4096,
 * T*k < 2^30.  Logits must be finite. */
size_t moe_route_permute_workspace_size(int32_t T, int32_t E, int32_t k);
int moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k,
                      int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                      int32_t* perm_src_token, int32_t* perm_of_assignment, float* perm_weight,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- quantise
 * The NVFP4 encoding of an operand (e2m1 values with one ue4m3 scale per 16
 * along the reduction axis: "From Empirical Limits ...", section "Section 1:
 * CUTLASS Kernels - The Foundation"; the quantiser rule is the reading given
 * at the top of this file).
 * x [rows, cols] (bf16 or float32, finite) -> NVFP4 codes/scales as described
 * above.  g_in (device, nullable): a caller-supplied per-tensor scale; NULL
 * computes g = amax/2688 (1 if the tensor is zero) on the device.  g_out
 * (device, nullable) receives the scale used.  cols % 32 == 0, x 16-byte
 * aligned. */
size_t nvfp4_quantize_workspace_size(void);
int nvfp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                   const float* g_in, float* g_out, uint8_t* codes, uint8_t* scales,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- route + quantise
 * moe_route_permute and nvfp4_quantize of the layer's activations in one
 * call, with the same arguments and the same, bit-identical outputs (x has
 * T rows).  The two steps read different inputs; their kernels share launches,
 * so their short launches overlap instead of running one after another.
 * workspace: moe_route_quantize_workspace_size(T, E, k) bytes, 16-byte
 * aligned, caller-owned (the routing scratch followed by the quantiser's amax
 * partials).  Errors as for the two calls. */
size_t moe_route_quantize_workspace_size(int32_t T, int32_t E, int32_t k);
int moe_route_quantize(const float* logits, int32_t T, int32_t E, int32_t k,
                       int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                       int32_t* perm_src_token, int32_t* perm_of_assignment, float* perm_weight,
                       const void* x, int32_t x_dtype, int64_t cols, const float* g_in, float* g_out,
                       uint8_t* codes, uint8_t* scales,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- route + quantise, no allocation
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and bit-identical outputs as
 * moe_route_quantize, minus the workspace: the scratch comes from one fixed
 * block of device memory that the library holds on each GPU it runs on until
 * the process ends (moe_route_quantize_noalloc_max_workspace() bytes, 4 MiB).
 * A call whose moe_route_quantize_workspace_size(T, E, k) exceeds that block
 * returns NVFP4MOE_ERR_UNSUPPORTED (about T*k <= 900k at E = 256).  Nothing is
 * allocated: the device address of the block is looked up once per device, on
 * the first call with that device current.  Every call on one GPU shares the
 * block, so calls that overlap on one GPU (concurrent streams, or threads)
 * race and must be serialised by the caller.  Other errors as for
 * moe_route_quantize. */
size_t moe_route_quantize_noalloc_max_workspace(void);
int moe_route_quantize_noalloc(const float* logits, int32_t T, int32_t E, int32_t k,
                               int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                               int32_t* perm_src_token, int32_t* perm_of_assignment, float* perm_weight,
                               const void* x, int32_t x_dtype, int64_t cols, const float* g_in, float* g_out,
                               uint8_t* codes, uint8_t* scales, void* stream);

/* ---------------------------------------------------------------- grouped GEMM
 * For expert e and GEMM row p in [offsets[e], offsets[e+1]) with A row
 * r = a_rows ? a_rows[p] : p:
 *   y[p, n] = (g_a * g_b[e]) * sum_kb s_a[r,kb] s_b[e,n,kb] sum_{i<16} q_a[r,16kb+i] q_b[e,n,16kb+i]
 * FP32 accumulation; the block products are formed exactly (E2M1*E4M3 values
 * are exact in FP16 and their products exact in FP32).  The MoE grouped GEMM of
 * "From Empirical Limits ...", section "Sections 2-4: Framework and Community
 * Landscape", with the epilogues listed in nvfp4moe_epilogue (the "finalize"
 * epilogue of "The Critical Search: Uncovering SM120 CUTLASS Collective
 * Implementations", section "Context: The Optimization Journey", is
 * NVFP4MOE_EPI_COMBINE_F32).  Rows p >= offsets[E] are not written.  Experts
 * with no rows read no weight bytes.  Size limits (NVFP4MOE_ERR_UNSUPPORTED
 * beyond them): A codes (a_rows_total * K / 2 bytes) below 2 GiB; fewer than
 * 2^31 rows. */
int nvfp4_grouped_gemm(const nvfp4moe_gemm_args* args, void* stream);

/* ---------------------------------------------------------------- expert FFN in one call
 * gate_up grouped GEMM + SwiGLU + NVFP4 requantisation of h, then the down
 * grouped GEMM, for all experts: the two nvfp4_grouped_gemm calls of the
 * layer (EPI_SWIGLU_NVFP4 on gathered x rows, then EPI_BF16 on h), with the
 * same results bit for bit.  From 48 rows per expert (the hint, else
 * m_total / E) both run in ONE persistent launch whose down tasks start as soon
 * as the gate_up tasks of their row chunk are done, filling the slots the light
 * chunks leave free ("From Empirical Limits ...", section "Sections 5-6:
 * Algorithmic Techniques": adaptive grid sizing; section "Key Findings and
 * Their Impact": fusion; "Discovering SM120-Specific CUTLASS MoE Kernels",
 * section "The Discovery": a min-latency kernel for small batches, tuned to the
 * expected tokens).  The tile table, by rows per expert (measured):
 *   < 48       two launches, decode tile, non-temporal weight loads (while
 *              every expert fits one 64-row chunk gate_up fills every slot in
 *              one round: no tail to fill)
 *   48 .. 63   one launch, decode tile, non-temporal weight loads
 *   >= 64      one launch, decode tile, cached weight loads (from 128 rows
 *              the MFMA-bound regime, where it still beats two launches of
 *              the large-M tile: down overlaps gate_up's tail)
 * Arguments (device pointers):
 *   x_codes/x_scales/x_g   NVFP4 activations [x_rows, H/2], [x_rows, H/16], g
 *   perm_src_token         [m_total]: x row of GEMM row p (moe_route_permute)
 *   offsets                [E+1] expert offsets (moe_route_permute)
 *   w_gu_packed, g_gu      gate_up weights [E, 2I, H] repacked by
 *                          nvfp4_weight_repack, per-expert scales [E]
 *   w_dn_packed, g_dn      down weights [E, H, I] repacked, scales [E]
 *   g_h                    per-tensor scale of h (1 float)
 *   h_codes, h_scales      (out) h [m_total, I/2], [m_total, I/16]
 *   y                      (out) bf16 [m_total, H], the down rows (then
 *                          moe_unpermute_combine, or the fused combine below)
 *   out, perm_of_assignment, topk_w, T, k   optional weighted top-k combine
 *                          of the down rows, with moe_unpermute_combine's
 *                          arithmetic and result bit for bit (bf16 in, bf16
 *                          out): out [T, H] bf16, perm_of_assignment and topk_w
 *                          [T, k] from moe_route_permute, T * k == m_total,
 *                          m_total * H * 2 < 2^31.  out == NULL: no combine
 *                          (y holds the result).  In the one-launch regime the
 *                          combine runs inside the launch - the down task that
 *                          writes the last of a token's k rows of a column
 *                          group combines that group (the pages' finalize:
 *                          "The Critical Search ...", section "Context: The
 *                          Optimization Journey") - otherwise as one more
 *                          kernel on the stream after the down GEMM.
 * I % 32 == 0, I <= 256 (one K step of the down GEMM), H % 32 == 0, E <= 4096.
 * workspace: moe_expert_ffn_workspace_size(E, m_total, H, I) bytes, 256-byte
 * aligned, caller-owned; it holds the task lists and chunk counters, which the
 * call rewrites (a planning kernel, no memset).  Its first 64 int32 words are a
 * header; word 8 is nonzero after a launch in which a down task stopped waiting
 * for its h rows past a bounded spin (a fault of the scheduling, never expected:
 * the results of that launch are then invalid).  Calls sharing a workspace must
 * not overlap. */
typedef struct nvfp4moe_ffn_args {
  const uint8_t* x_codes;
  const uint8_t* x_scales;
  const float* x_g;
  int64_t x_rows;
  const int32_t* perm_src_token;
  const int32_t* offsets;
  int32_t E;
  int32_t H;
  int32_t I;
  int64_t m_total;
  const uint8_t* w_gu_packed;
  const float* g_gu;
  const uint8_t* w_dn_packed;
  const float* g_dn;
  const float* g_h;
  uint8_t* h_codes;
  uint8_t* h_scales;
  void* y;
  int32_t max_rows_per_expert_hint;
  void* out;
  const int32_t* perm_of_assignment;
  const float* topk_w;
  int32_t T;
  int32_t k;
} nvfp4moe_ffn_args;
size_t moe_expert_ffn_workspace_size(int32_t E, int64_t m_total, int32_t H, int32_t I);
int moe_expert_ffn(const nvfp4moe_ffn_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- MXFP4 variant
 * The MXFP4 format: E2M1 values with one E8M0 scale (a power of two, code c =
 * 2^(c-127)) per 32 consecutive values along the reduction axis and no
 * per-tensor scale (the OCP MX format; the pages list an MXFP4 grouped GEMM
 * with 128x128x128 tiles among the kernels they survey: "From Empirical Limits
 * ...", section "Sections 2-4: Framework and Community Landscape").  It maps
 * onto gfx950's block-scaled MFMA with no decode in registers.
 *   codes  uint8 [rows, cols/2]   as NVFP4 (element 2i in the low nibble of byte i)
 *   scales uint8 [rows, cols/32]  E8M0 codes
 * Quantiser: X = floor(log2(absmax_block)) - 2 clamped to [-127, 127], scale
 * code X + 127, code = E2M1 nearest-even of x / 2^X (exact), saturating at 6,
 * sign copied from x; an all-zero block gets scale code 0 and codes 0.
 * x: bf16 or float32 [rows, cols], finite, 16-byte aligned, cols % 32 == 0. */
int mxfp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                   void* stream);
/* Grouped MXFP4 GEMM with the nvfp4_grouped_gemm argument struct, read as:
 *   y[p, n] = a_g * b_g[e] * sum_k A^[r, k] B^[e, n, k]   (A^, B^ dequantised MX values)
 * a_scales [a_rows_total, K/32], b_scales [E, N, K/32] (E8M0); a_g, b_g are
 * float32 multipliers (pass 1.0 for plain MX tensors); b_packed: optional B in
 * the layout written by mxfp4_weight_repack (then b_codes/b_scales are not read).  Epilogues: EPI_F32, EPI_BF16, and EPI_SWIGLU_NVFP4
 * read as SwiGLU + MXFP4 requantisation of h: out_codes [m_total, I/2],
 * out_scales [m_total, I/32] (out_g unused; I % 32 == 0).  EPI_COMBINE_F32 is
 * NVFP4MOE_ERR_UNSUPPORTED.  K % 32 == 0.  FP32 accumulation of exact
 * E2M1 x E2M1 x 2^k products; other limits as for nvfp4_grouped_gemm. */
int mxfp4_grouped_gemm(const nvfp4moe_gemm_args* args, void* stream);
/* MXFP4 weights [E, N, K] repacked once into streaming tiles of 16 rows x 256
 * K (2176 bytes: each lane's 32 code bytes and 2 scale bytes, in the order the
 * kernel's lanes read them; zero codes past N and K).  Private layout, pure
 * data movement.  K % 32 == 0; 16-byte aligned codes and packed. */
size_t mxfp4_weight_packed_size(int32_t E, int32_t N, int32_t K);
int mxfp4_weight_repack(const uint8_t* codes, const uint8_t* scales, int32_t E, int32_t N, int32_t K,
                        uint8_t* packed, size_t packed_bytes, void* stream);

/* ---------------------------------------------------------------- FP8 block-scaled variant
 * FP8 E4M3 operands with float32 block scales along K (the FP8 grouped GEMM
 * the pages list beside the FP4 ones: "From Empirical Limits ...", section
 * "Sections 2-4: Framework and Community Landscape"; the blockwise-scaled
 * FP8 collective: "The Critical Search: Uncovering SM120 CUTLASS Collective
 * Implementations", section "Output Knowledge Created").  Blocks of 128
 * values along K: one scale per row and block for activations (1 x 128), one
 * per 128 x 128 tile for weights.
 *   codes  uint8 [rows, cols]   E4M3 (OCP E4M3FN) bytes, sign in bit 7
 *   scales float [ceil(rows/block_rows), cols/128]
 * Quantiser: s = absmax_block / 448 (float32 division; 1 for an all-zero
 * block), code = E4M3 nearest-even of |x| / s (correctly rounded float32
 * quotient), saturating at 448, sign copied from x.
 * fp8_quantize: x bf16 or float32 [batch, rows, cols] (finite, 16-byte aligned,
 * cols % 128 == 0); block_rows 1 (activations: batch is folded into rows) or
 * 128 (weights: each of the batch matrices has its own row blocks, scales
 * [batch, ceil(rows/128), cols/128]; rows <= 8388480, batch <= 65535,
 * cols < 2^31).  Block rows 1: fewer than 2^26 blocks in all.  codes 16-byte,
 * scales 4-byte aligned. */
int fp8_quantize(const void* x, int32_t x_dtype, int64_t batch, int64_t rows, int64_t cols, int32_t block_rows,
                 uint8_t* codes, float* scales, void* stream);
/* SwiGLU between the FP8 grouped GEMMs: h = silu(gate) * up of gate_up [M, 2I]
 * (float32 or bf16; gate = columns [0, I), up = [I, 2I), as moe_swiglu), in
 * float32, quantised as fp8_quantize with 1 x 128 blocks: codes [M, I], scales
 * [M, I/128].  I % 128 == 0; gate_up 8-byte, codes 2-byte, scales 4-byte
 * aligned. */
int fp8_swiglu_quantize(const void* gate_up, int32_t dtype, int64_t M, int32_t I, uint8_t* codes, float* scales,
                        void* stream);
/* FP8 weights [E, N, K] repacked once into tiles of 16 rows x 128 K (2048
 * bytes, each lane's 32 bytes in the order the kernel's lanes read them; zero
 * codes past N).  Private layout, pure data movement.  K % 128 == 0, N % 16 ==
 * 0, 16-byte aligned codes and packed. */
size_t fp8_weight_packed_size(int32_t E, int32_t N, int32_t K);
int fp8_weight_repack(const uint8_t* codes, int32_t E, int32_t N, int32_t K, uint8_t* packed, size_t packed_bytes,
                      void* stream);
/* Grouped FP8 GEMM, per expert e and GEMM row p in [offsets[e], offsets[e+1])
 * with A row r = a_rows[p] (or p):
 *   y[p, n] = sum_kb sa[r, kb] * sb[e, n / 128, kb] * sum_{k in block kb} A[r, k] B[e, n, k]
 * Each block's partial sum comes from the FP8 matrix instruction in float32
 * and enters the float32 accumulator scaled by sa * sb.  Same grouping and
 * bounds rules as nvfp4_grouped_gemm; epilogues EPI_F32, EPI_BF16, and
 * EPI_SWIGLU_NVFP4 read as SwiGLU + FP8 requantisation of h (the gate_up GEMM
 * with fp8_swiglu_quantize fused into it, the same bits): N = 2I with
 * I % 128 == 0, h = silu(y[:, :I]) * y[:, I:], out_codes [m_total, I] E4M3 and
 * out_scales float32 [m_total, I/128] as fp8_swiglu_quantize writes them.
 * This epilogue runs the decode tile at every size (the large tile has no
 * SwiGLU epilogue). */
typedef struct nvfp4moe_fp8_gemm_args {
  const uint8_t* a_codes;     /* [a_rows_total, K] E4M3, 16-byte aligned */
  const float* a_scales;      /* [a_rows_total, K/128] */
  const int32_t* a_rows;      /* device [m_total] or NULL; entries in [0, a_rows_total) */
  int64_t a_rows_total;
  const uint8_t* b_packed;    /* fp8_weight_repack layout of [E, N, K], 16-byte aligned */
  const float* b_scales;      /* [E, ceil(N/128), K/128] */
  const int32_t* offsets;     /* device [E+1], as for nvfp4_grouped_gemm */
  int32_t E;
  int32_t N;                  /* multiple of 16 */
  int32_t K;                  /* multiple of 128 */
  int64_t m_total;
  int32_t epilogue;           /* NVFP4MOE_EPI_F32, NVFP4MOE_EPI_BF16 or NVFP4MOE_EPI_SWIGLU_NVFP4 (see above) */
  void* out;                  /* float or bf16 [m_total, N], 16-byte aligned; unused for SwiGLU */
  int32_t max_rows_per_expert_hint;  /* as for nvfp4_grouped_gemm: < 64 streams weights non-temporally */
  uint8_t* out_codes;         /* SwiGLU: h codes [m_total, N/2] */
  float* out_scales;          /* SwiGLU: h block scales [m_total, N/256], 4-byte aligned */
} nvfp4moe_fp8_gemm_args;
int fp8_grouped_gemm(const nvfp4moe_fp8_gemm_args* args, void* stream);

/* ---------------------------------------------------------------- packed weights
 * Weights are static, so they can be repacked once into a tile layout that the
 * grouped GEMM streams with fully contiguous, non-temporal loads: tile
 * (e, 16-row tile rt, 256-K step st) is 2304 bytes (the 16 rows' 128 code bytes
 * and 16 scale bytes of the step, ordered by the lane that consumes them),
 * tiles ordered by (e, rt, st), zero padded past N and K.  The layout is private
 * to this library (it may change between versions; nvfp4moe_version() tells
 * them apart); the row-major NVFP4 tensors stay the reference format.
 *   codes   [E, N, K/2]  row-major NVFP4 codes (16-byte aligned)
 *   scales  [E, N, K/16] E4M3 block scales
 *   packed  (out) nvfp4_weight_packed_size(E, N, K) bytes, 16-byte aligned
 * K % 32 == 0.  Pure data movement: no rounding, bit-exact. */
size_t nvfp4_weight_packed_size(int32_t E, int32_t N, int32_t K);
int nvfp4_weight_repack(const uint8_t* codes, const uint8_t* scales, int32_t E, int32_t N, int32_t K,
                        uint8_t* packed, size_t packed_bytes, void* stream);

/* ---------------------------------------------------------------- SwiGLU (unfused)
 * The activation between the two expert GEMMs, re-quantised to NVFP4 so that
 * the down GEMM runs on e2m1 operands too (the e2m1 x e2m1 block-scaled MMA of
 * "From Empirical Limits ...", section "Section 1: CUTLASS Kernels - The
 * Foundation"; the same step fused into the gate_up epilogue is
 * NVFP4MOE_EPI_SWIGLU_NVFP4, the kind of epilogue fusion that section "Key
 * Findings and Their Impact" of that page weighs more when bandwidth is tight).
 * gate_up [M, 2I] (float32 or bf16) -> h = silu(gate) * up, gate = columns
 * [0, I), up = [I, 2I), quantised to NVFP4 codes [M, I/2], scales [M, I/16].
 * g_in (nullable): per-tensor scale of h; NULL computes amax(h)/2688 on the
 * device (two passes).  g_out (nullable) receives the scale used.  I % 16 == 0. */
size_t moe_swiglu_workspace_size(void);
int moe_swiglu(const void* gate_up, int32_t dtype, int64_t M, int32_t I,
               const float* g_in, float* g_out, uint8_t* codes, uint8_t* scales,
               void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- combine (unfused)
 * out[t, :] = sum_{j<k} topk_w[t, j] * y[perm_of_assignment[t*k + j], :]
 * ("token reordering with fused reduction", "From Empirical Limits ...", section
 * "Sections 5-6: Algorithmic Techniques").  y [rows, H] float32 or bf16; out
 * [T, H] float32 or bf16 (nearest even); float32 accumulation in j order.
 * perm_of_assignment NULL means row t*k + j; topk_w NULL means weight 1, so
 * (perm NULL, w NULL, k = 1) converts a float32 accumulator to bf16.
 * Every perm_of_assignment entry must lie in [0, rows of y): the kernel reads
 * the rows it names without a bounds check (the routing calls produce such
 * entries).  Without perm_of_assignment, y needs at least T*k rows.
 * H % 8 == 0. */
int moe_unpermute_combine(const void* y, int32_t y_dtype, const int32_t* perm_of_assignment,
                          const float* topk_w, int32_t T, int32_t k, int32_t H,
                          void* out, int32_t out_dtype, void* stream);

/* ---------------------------------------------------------------- status */
const char* nvfp4moe_status_string(int status);
const char* nvfp4moe_last_error_detail(void);
/* library version: major*10000 + minor*100 + patch */
int nvfp4moe_version(void);   /* 101: packed weight tiles of 16 rows x 256 K */

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MOE_H */
