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
  // kSwigluSave: the gate and up pre-activations are also stored, E = round(g), V = round(u).
  // kSwigluBwd: E and V are read (the saved pre-activations), C receives hmid = round(silu(E) V)
  // and D the SwiGLU gradients: D[m][n] = round(acc V silu'(E)), D[m][N + n] = round(acc silu(E)).
  uint16_t* E;
  uint16_t* V;
  int64_t lde;
  uint16_t* D;
  int64_t ldd;
  // Plain mode only: up to 3 column groups in one launch (the query/key/value projections of
  // one x). Group g owns column blocks [gblk[g], gblk[g + 1]) of 256 columns and replaces W0 by
  // gW[g], B2 by gB2[g], A2 by A2 + ga2[g], C by gC[g], ldc by gldc[g] and N by gN[g].
  // ngroups <= 1: one group, the fields above.
  int ngroups;
  int gblk[4];
  const uint16_t* gW[3];
  const uint16_t* gB2[3];
  int64_t ga2[3];
  uint16_t* gC[3];
  int64_t gldc[3];
  int gN[3];
};

// Epilogue modes of the GEMM: plain store; SwiGLU of the gate/up pair; the same also storing the
// pre-activations; the SwiGLU backward (256-column tiles like the plain mode).
enum GemmMode { kGemmPlain = 0, kGemmSwiglu = 1, kGemmSwigluSave = 2, kGemmSwigluBwd = 3 };

hipError_t launch_gemm_lora(const GemmArgs& a, int mode, hipStream_t st);

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

// Transposed, scaled, zero-padded copies of small LoRA operands, up to 6 in one launch:
// dst[i][c] = round(scale * src[c - c0][i]) for c0 <= c < c0 + cn, else 0, for i < rows,
// c < cols (bf16).
struct TJob {
  const uint16_t* src;
  int64_t lds;
  uint16_t* dst;
  int64_t ldd;
  int rows, cols, c0, cn;
  float scale;
};
struct TJobs {
  TJob job[6];
  int n;
};
hipError_t launch_small_transposes(const TJobs& jobs, hipStream_t st);

// Plain bf16 transpose dst[c][r] = src[r][c] of a rows x cols matrix (LDS tiles of 64 x 64).
hipError_t launch_transpose(const uint16_t* src, int64_t lds, uint16_t* dst, int64_t ldd, int rows,
                            int cols, hipStream_t st);

// Sums over tokens for the LoRA weight gradients, up to 6 in one pass:
// out[c * osc + j * osj] = round(scale * sum_m P[m][c] * Q[m][j]) for c < C, j < nq,
// computed as fp32 partial sums over row chunks (part, chunks x ceil(nq/16) x C x 16 floats per
// job) and a fixed-order reduction. C is a multiple of 4; P rows 8-byte aligned.
struct ColJob {
  const uint16_t* P;
  int64_t ldp;
  const uint16_t* Q;
  int64_t ldq;
  uint16_t* out;
  int64_t osc, osj;
  int C, nq;
  float scale;
};
struct ColJobs {
  ColJob job[6];
  int n, M, chunks;
};
size_t colred_partial_floats(const ColJobs& jobs);
hipError_t launch_colred(const ColJobs& jobs, float* part, hipStream_t st);

}  // namespace lmx
