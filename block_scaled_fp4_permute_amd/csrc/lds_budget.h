// Shared-memory (LDS) budget of block-scaled GEMM tiles.
//
// The pages size every tile configuration against the per-block shared memory
// of the GPU they target ("From Empirical Limits to Research-Driven
// Optimization", section "The Shared Memory Budget Analysis"; a 128 x 256 x 128
// tile with the finalize epilogue needing about 155 KB in "The Critical
// Search: Uncovering SM120 CUTLASS Collective Implementations", section
// "Context: The Optimization Journey").  The accounting here: one pipeline
// stage of a BM x BN x BK tile holds the E2M1 codes of A and B (half a byte per
// value) and their E4M3 block scales (one byte per 16 values along K); an
// epilogue staged in shared memory adds BM x BN values of its own width.
// gfx950 gives a workgroup up to the whole 160 KiB of its CU's LDS; a kernel
// that wants W resident workgroups per CU must fit W times its LDS in it.
// Plain constexpr arithmetic: no HIP types, so host tools can include it.
#pragma once

#include <stddef.h>

namespace nvfp4 {

constexpr size_t kLdsBytesPerCU = 160 * 1024;

constexpr size_t nvfp4_stage_bytes(size_t BM, size_t BN, size_t BK) {
  return (BM + BN) * BK / 2 + (BM + BN) * (BK / 16);
}

constexpr size_t tile_lds_bytes(size_t BM, size_t BN, size_t BK, size_t stages, size_t epilogue_bytes_per_value) {
  return stages * nvfp4_stage_bytes(BM, BN, BK) + BM * BN * epilogue_bytes_per_value;
}

constexpr bool fits_lds(size_t bytes_per_workgroup, size_t workgroups_per_cu) {
  return bytes_per_workgroup * workgroups_per_cu <= kLdsBytesPerCU;
}

}  // namespace nvfp4
