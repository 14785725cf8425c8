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

// dst[i][j] = round(scale * src[i][j]) for j < r, 0 for r <= j < ld_dst, rows i < n, written at
// column offset `col0` of dst rows (the rest of each dst row is zeroed too).
hipError_t launch_scale_lora_b(const uint16_t* src, int64_t ld_src, int n, int r, float scale,
                               uint16_t* dst, int64_t ld_dst, int col0, hipStream_t st);

}  // namespace lmx
