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
// Estimated time of a plain-mode launch over M rows and nbn 256-column blocks, in rounds of
// 256-row tiles; *half (if given) tells whether the launch takes 128-row tiles.
double gemm_plain_cost(int M, int nbn, bool* half = nullptr);

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

// Small LoRA operand copies, up to 10 in one launch, bf16, for i < rows and c < cols:
//   transposed (plain = false): dst[i][c] = round(scale * src[c - c0][i]) for c0 <= c < c0 + cn
//   and i < rv, else 0;
//   row copy (plain = true):    dst[i][c] = round(scale * src[i][c - c0]) under the same bounds.
// (lds is the source row pitch in both forms.)
struct TJob {
  const uint16_t* src;
  int64_t lds;
  uint16_t* dst;
  int64_t ldd;
  int rows, cols, c0, cn, rv;
  float scale;
  bool plain;
};
struct TJobs {
  TJob job[10];
  int n;
};
hipError_t launch_small_transposes(const TJobs& jobs, hipStream_t st);

// Plain bf16 transpose dst[c][r] = src[r][c] of a rows x cols matrix (LDS tiles of 64 x 64).
hipError_t launch_transpose(const uint16_t* src, int64_t lds, uint16_t* dst, int64_t ldd, int rows,
                            int cols, hipStream_t st);
// Plain bf16 copy dst[m][c] = src[m][c] of a rows x cols matrix, 16 bytes per thread (cols,
// pitches and bases 16-byte multiples).
hipError_t launch_copy2d(const uint16_t* src, int64_t lds, uint16_t* dst, int64_t ldd, int rows,
                         int cols, hipStream_t st);

// Sums over one pass of a bf16 matrix P [M][C] (row pitch ldp), up to 4 matrices per launch, in
// fp32:
//   row side, R_h for h < nr <= 3:   Drow_h[m][j] = sum_c P[m][c] R_h[j][c]   (R_h [16 JB][C], pitch ldr)
//   column side, Q_h for h < nh <= 2: Dcol_h[c][j] = sum_m P[m][c] Q_h[m][j]   (Q_h [M], pitch ldq)
// for j < 16 JB, JB = the launch's rank blocks of 16; nr + nh >= 1. Results are partial sums:
// the row side per block of 512 columns, rowpart + rp0 + h * (ncb * M * JB * 16):
// [ncb = ceil(C / 512)][M][JB][16]; the column side per chunk of rows,
// colpart + cp0 + h * (chunks * C * JB * 16): [chunks][C][JB][16]. C is a multiple of 32; P, R
// and Q rows are 16-byte aligned and Q_h[m][16 jb .. 16 jb + 15] readable for every jb < JB.
struct SumJob {
  const uint16_t* P;
  int64_t ldp;
  const uint16_t* R[3];
  int64_t ldr;
  const uint16_t* Q[2];
  int64_t ldq;
  int C, nr, nh;
  int64_t rp0, cp0;  // float offsets of the job's partials in rowpart / colpart
};
struct SumJobs {
  SumJob job[4];
  int n, M, JB, chunks, rows_per;
  int blk0[5];  // first workgroup (grid x) of each job: ceil(C / 512) column blocks per job
};
// Chooses chunks / rows_per / blk0 and the partial offsets for about `target` workgroups;
// returns the floats of (rowpart, colpart).
void plan_sums(SumJobs& j, int target, int64_t* row_floats, int64_t* col_floats);
hipError_t launch_sums(const SumJobs& jobs, float* rowpart, float* colpart, hipStream_t st);

// Fixed-order reduction of partial planes into bf16 results, up to 6 outputs per launch:
//   out[a * osa + j * osj] = round(scale * sum_{p < np} src[p * pstride + (a * JB) * 16 + j])
// for a < A and j < r, and 0 for r <= j < J (zero padding of a rank-padded operand).
struct RedJob {
  const float* src;
  int64_t pstride;
  uint16_t* out;
  int64_t osa, osj;
  int A, J, r, np;
  float scale;
};
struct RedJobs {
  RedJob job[6];
  int n, JB;
};
hipError_t launch_reduce_sums(const RedJobs& jobs, hipStream_t st);

}  // namespace lmx
