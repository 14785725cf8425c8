// Internal launch interface of the fused-MLP kernels (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmx {

// C[M][N] = [A | A2][M][K + K2] [W | B2][N][K + K2]^T, bf16 in and out, fp32 accumulation: the
// LoRA term enters as K2 extra reduction columns (A2 = LoRA-A products, B2 = scaled LoRA-B).
// Gate/up form (swiglu): W0 is the gate and W1 the up weight; B2 has 2N rows (gate rows then up
// rows) and C = silu(gate) * up. K and K2 are multiples of 32; rows 16-byte aligned.
struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* W0;
  const uint16_t* W1;
  int64_t ldw;
  const uint16_t* A2;
  int64_t lda2;
  const uint16_t* B2;
  int64_t ldb2;
  uint16_t* C;
  int64_t ldc;
  int M, N, K, K2;
};

hipError_t launch_gemm_lora(const GemmArgs& a, bool swiglu, hipStream_t st);

// One scaled copy: dst[i][col0 + j] = round(scale * src[i][j]) for j < r, rows i < n; every
// other column of the dst rows [0, ld_dst) is written as 0.
struct ScaleJob {
  const uint16_t* src;
  int64_t ld_src;
  uint16_t* dst;
  int64_t ld_dst;
  int n, col0;
};
struct ScaleJobs {
  ScaleJob job[3];
};

// The three scaled copies in one launch (same scale and rank).
hipError_t launch_scale_lora_b(const ScaleJobs& jobs, float scale, int r, hipStream_t st);

}  // namespace lmx
