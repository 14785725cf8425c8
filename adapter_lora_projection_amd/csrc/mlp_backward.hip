// Kernels of the single-adapter LoRA MLP backward beyond the GEMMs ("Add optional fast lora path
// for qwen2/qwen3 on npu", review thread and Verification advice: the backward of the fast path
// takes the saved X and gate/up projections, runs the SwiGLU backward, forms dX and the LoRA A/B
// gradients, and never overwrites X):
//   * transposes of the frozen weights (once per layer: the backward's GEMMs read them with the
//     reduction index contiguous, as the forward's do);
//   * small transposed / scaled / zero-padded copies of the LoRA operands;
//   * one pass over each of de, dv and hmid forming both its LoRA-A product (a sum over its
//     columns) and its LoRA weight-gradient sum (a sum over tokens), and the remaining sums over
//     tokens for x and dout (dA = dxa^T P, dB = s P^T xa), all on MFMA;
//   * the fixed-order reduction of their partial sums.
#include "device_common.hpp"
#include "mlp_kernels.hpp"

#include <algorithm>

namespace lmx {

// ---- small operand copies ----------------------------------------------------------------
// One thread per destination element; the jobs are laid end to end over the grid.
__global__ __launch_bounds__(256) void small_transposes_kernel(TJobs jobs) {
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
#pragma unroll
  for (int q = 0; q < 10; ++q) {
    if (q >= jobs.n) return;
    const TJob& jb = jobs.job[q];
    const int64_t total = int64_t(jb.rows) * jb.cols;
    if (i < total) {
      const int row = int(i / jb.cols), c = int(i - int64_t(i / jb.cols) * jb.cols);
      uint16_t v = 0;
      const int k = c - jb.c0;
      if (k >= 0 && k < jb.cn && row < jb.rv) {
        const int64_t at = jb.plain ? int64_t(row) * jb.lds + k : int64_t(k) * jb.lds + row;
        v = Traits<DT_BF16>::from_f32(jb.scale * Traits<DT_BF16>::to_f32(jb.src[at]));
      }
      jb.dst[int64_t(row) * jb.ldd + c] = v;
      return;
    }
    i -= total;
  }
}

hipError_t launch_small_transposes(const TJobs& jobs, hipStream_t st) {
  int64_t total = 0;
  for (int q = 0; q < jobs.n; ++q) total += int64_t(jobs.job[q].rows) * jobs.job[q].cols;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(small_transposes_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0,
                     st, jobs);
  return hipGetLastError();
}

// ---- transpose of a frozen weight ---------------------------------------------------------
// 64 x 64 tiles through LDS (row pitch 65 elements against bank conflicts); 256 threads, each
// moving 16 elements in and 16 out. Reads and writes are row-contiguous across the threads.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                        uint16_t* __restrict__ dst, int64_t ldd,
                                                        int rows, int cols) {
  __shared__ uint16_t t[64][65];
  const int r0 = int(blockIdx.y) * 64, c0 = int(blockIdx.x) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + ty + 4 * k, c = c0 + tx;
    if (r < rows && c < cols) t[ty + 4 * k][tx] = src[int64_t(r) * lds + c];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int c = c0 + ty + 4 * k, r = r0 + tx;  // dst row c, column r
    if (r < rows && c < cols) dst[int64_t(c) * ldd + r] = t[tx][ty + 4 * k];
  }
}

hipError_t launch_transpose(const uint16_t* src, int64_t lds, uint16_t* dst, int64_t ldd, int rows,
                            int cols, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel, dim3(unsigned((cols + 63) / 64), unsigned((rows + 63) / 64)),
                     dim3(256), 0, st, src, lds, dst, ldd, rows, cols);
  return hipGetLastError();
}

// ---- 2-D copy of a bf16 matrix ---------------------------------------------------------------
// dst[m][c] = src[m][c] for m < rows, c < cols; 16 bytes per thread (cols, the pitches and both
// bases 16-byte multiples, which the host checks); workgroup (x, y) copies 256 x 8 columns of
// rows y, y + gridDim.y, ...
__global__ __launch_bounds__(256) void copy2d_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                     uint16_t* __restrict__ dst, int64_t ldd,
                                                     int rows, int cols) {
  const int c = (int(blockIdx.x) * 256 + int(threadIdx.x)) * 8;
  if (c >= cols) return;
  for (int m = int(blockIdx.y); m < rows; m += int(gridDim.y))
    *reinterpret_cast<uint4*>(dst + int64_t(m) * ldd + c) =
        *reinterpret_cast<const uint4*>(src + int64_t(m) * lds + c);
}

hipError_t launch_copy2d(const uint16_t* src, int64_t lds, uint16_t* dst, int64_t ldd, int rows,
                         int cols, hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % 8 != 0 || lds % 8 != 0 || ldd % 8 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) ||
      (reinterpret_cast<uintptr_t>(dst) & 15))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy2d_kernel, dim3(unsigned((cols / 8 + 255) / 256), unsigned(std::min(rows, 4096))),
                     dim3(256), 0, st, src, lds, dst, ldd, rows, cols);
  return hipGetLastError();
}

// ---- sums over columns and over tokens in one pass over P --------------------------------
// Workgroup (x = block of 512 columns of one job, y = chunk of rows, z = rank block of 16): 4
// waves, wave w owning columns [128 w, 128 w + 128) of the block. Steps of 16 rows of P (and of
// the heads' Q rows) go straight to LDS (global_load_lds_dwordx4), three steps in flight; the LDS
// rows carry 16 bytes of padding so that the row-side reads below are bank-conflict free.
// Column side (v_mfma_f32_16x16x16_bf16): lane (g, t) = (l / 16, l % 16) reads rows 4g .. 4g+3,
// columns 8t .. 8t+7 of its wave's slice and regroups them with byte permutes into eight A
// operands, one per column 8t + i, each holding that column's four rows; B is the heads' Q rows
// 4g .. 4g+3 at rank column t. MFMA i thus sums P[m][8t + i] Q[m][j] over the step's rows for
// t = 0..15, and its accumulator lives for the whole chunk.
// Row side, R_h for h < nr <= 3 (v_mfma_f32_16x16x32_bf16): A is the step's 16 rows with 32
// columns per k block, B the R_h rows (rank) over the same columns, held in registers for the
// whole chunk; each wave's sum over its 128 columns goes to LDS and the next step adds the 4
// waves in order and stores the block's partial row.
// Rows past M read row M - 1 and are zeroed in both operands of the column side; their row-side
// results are not stored. Column blocks past C read a valid column; their column-side results are
// not stored and their row-side k blocks are skipped (C is a multiple of 32).
namespace {
constexpr int kSumWaves = 4;
constexpr int kSumThreads = 64 * kSumWaves;
constexpr int kSumCols = 128 * kSumWaves;                  // columns per workgroup
constexpr int kSumRows = 16;                               // rows per step
constexpr int kSumStages = 3;
constexpr int kSumPitch = kSumCols * 2 + 16;               // bytes per LDS row of P
constexpr int kSumQOff = kSumRows * kSumPitch;             // Q rows: [16][2 heads][16] bf16
constexpr int kSumStageBytes = kSumQOff + kSumRows * 64;
constexpr int kSumRedBytes = 2 * 3 * kSumWaves * 256 * 4;  // row-side sums: 2 steps x 3 heads
constexpr int kSumPLoads = kSumRows / kSumWaves;           // P loads per wave and step

__device__ __forceinline__ f32x4_t mma16x16x16(uint2 a, uint2 b, f32x4_t c) {
  typedef short s4_t __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, a),
                                                  __builtin_bit_cast(s4_t, b), c, 0, 0, 0);
}
}  // namespace

void plan_sums(SumJobs& j, int target, int64_t* row_floats, int64_t* col_floats) {
  j.blk0[0] = 0;
  for (int q = 0; q < j.n; ++q) j.blk0[q + 1] = j.blk0[q] + (j.job[q].C + kSumCols - 1) / kSumCols;
  const int blocks = j.blk0[j.n] * j.JB;
  const int steps = std::max(1, (j.M + kSumRows - 1) / kSumRows);
  int chunks = std::max(1, (target + blocks / 2) / std::max(blocks, 1));
  chunks = std::min(chunks, steps);
  j.rows_per = ((steps + chunks - 1) / chunks) * kSumRows;
  j.chunks = (j.M + j.rows_per - 1) / j.rows_per;
  int64_t rf = 0, cf = 0;
  for (int q = 0; q < j.n; ++q) {
    SumJob& jb = j.job[q];
    const int ncb = (jb.C + kSumCols - 1) / kSumCols;
    jb.rp0 = rf;
    rf += int64_t(jb.nr) * ncb * j.M * j.JB * 16;
    jb.cp0 = cf;
    cf += int64_t(jb.nh) * j.chunks * jb.C * j.JB * 16;
  }
  *row_floats = rf;
  *col_floats = cf;
}

__global__ __launch_bounds__(kSumThreads) void sums_kernel(SumJobs jobs, float* __restrict__ rowpart,
                                                           float* __restrict__ colpart) {
  __shared__ __attribute__((aligned(16))) char lds[kSumStages * kSumStageBytes + kSumRedBytes];
  float* red = reinterpret_cast<float*>(lds + kSumStages * kSumStageBytes);
  // this workgroup's job (uniform; constant-index selection keeps the job table in registers)
  int q = 0;
#pragma unroll
  for (int k = 1; k < 4; ++k)
    if (k < jobs.n && int(blockIdx.x) >= jobs.blk0[k]) q = k;
  SumJob jb = jobs.job[0];
  int blk0 = jobs.blk0[0];
#pragma unroll
  for (int k = 1; k < 4; ++k)
    if (q == k) { jb = jobs.job[k]; blk0 = jobs.blk0[k]; }
  const int c0 = (int(blockIdx.x) - blk0) * kSumCols;
  const int rb = int(blockIdx.y), jbk = int(blockIdx.z);
  const int M = jobs.M, C = jb.C, JB = jobs.JB;
  const int m0 = rb * jobs.rows_per, m1 = min(M, m0 + jobs.rows_per);
  if (m0 >= m1) return;  // uniform
  const int nsteps = (m1 - m0 + kSumRows - 1) / kSumRows;
  const int tid = int(threadIdx.x), lane = tid & 63, w = wave_id();
  const int g = lane >> 4, t = lane & 15;
  const int cw = c0 + 128 * w;  // first column of this wave's slice

  // direct-to-LDS loads of step s into buffer b: rows 4w .. 4w+3 of P (lane L: columns 8L ..
  // 8L+7 of the block) and of the heads' Q (lane L < 16: row 4w + L/4, head (L/2) % 2, half L % 2)
  const char* pbase = reinterpret_cast<const char*>(jb.P);
  const int64_t pcol = min(c0 + 8 * lane, C - 8);
  const int qrow = 4 * w + (lane >> 2), qh = (lane >> 1) & 1;
  const bool qload = lane < 16 && qh < jb.nh;
  const uint16_t* qsrc = qload ? (qh ? jb.Q[1] : jb.Q[0]) + 16 * jbk + 8 * (lane & 1) : nullptr;
  auto issue = [&](int s, int b) {
    char* st = lds + b * kSumStageBytes;
    const int m = m0 + kSumRows * s;
#pragma unroll
    for (int i = 0; i < kSumRows / kSumWaves; ++i) {
      const int row = (kSumRows / kSumWaves) * w + i;
      const int64_t mr = min(m + row, M - 1);
      dma16(pbase + (mr * jb.ldp + pcol) * 2, lds_addr(st + row * kSumPitch));
    }
    if (qload) {
      const int64_t mr = min(m + qrow, M - 1);
      dma16(qsrc + mr * jb.ldq, lds_addr(st + kSumQOff + 256 * w));
    }
  };

  // row side: rows 16 jbk + t of each R over the wave's columns, k block kb = columns
  // 32 kb + 8 g ..
  uint4 rreg[3][4];
#pragma unroll
  for (int h = 0; h < 3; ++h) {
    if (h < jb.nr) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int c = min(cw + 32 * kb + 8 * g, C - 8);
        rreg[h][kb] = *reinterpret_cast<const uint4*>(jb.R[h] + int64_t(16 * jbk + t) * jb.ldr + c);
      }
    }
  }
  f32x4_t acc[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = f32x4_t{};

  // sums of the 4 waves' row-side results of step s (in red[s & 1][h]) and their stores:
  // thread u owns row u / 16, rank column u % 16
  const int ncb = (C + kSumCols - 1) / kSumCols;
  auto store_rows = [&](int s) {
    const int rho = tid >> 4, j = tid & 15;
    const int m = m0 + kSumRows * s + rho;
#pragma unroll
    for (int h = 0; h < 3; ++h) {
      if (h < jb.nr) {
        const float* rr = red + ((s & 1) * 3 + h) * kSumWaves * 256 + (j + 16 * (rho >> 2)) * 4 + (rho & 3);
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < kSumWaves; ++ww) sum += rr[ww * 256];
        if (m < m1)
          rowpart[jb.rp0 + ((int64_t(h * ncb + int(blockIdx.x) - blk0) * M + m) * JB + jbk) * 16 + j] = sum;
      }
    }
  };

#pragma unroll
  for (int s = 0; s < kSumStages - 1; ++s)
    if (s < nsteps) issue(s, s);
  for (int s = 0; s < nsteps; ++s) {
    // this wave's loads of step s are done (over-waits by the stores issued after them); after
    // the barrier, every wave's are, and every wave is done reading step s - 1's buffer
    if (s + 1 >= nsteps) vm_wait<0>();
    else if (jb.nh > 0) vm_wait<kSumPLoads + 1>();
    else vm_wait<kSumPLoads>();
    __syncthreads();
    if (s + kSumStages - 1 < nsteps) issue(s + kSumStages - 1, (s + kSumStages - 1) % kSumStages);
    const char* st = lds + (s % kSumStages) * kSumStageBytes;
    const int valid = m1 - (m0 + kSumRows * s);  // rows of the step inside the chunk (uniform)

    // column side
    if (jb.nh > 0) {
      uint4 pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pr[e] = *reinterpret_cast<const uint4*>(st + (4 * g + e) * kSumPitch + (128 * w + 8 * t) * 2);
      uint2 qb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint16_t* qr = reinterpret_cast<const uint16_t*>(st + kSumQOff + 32 * h) + t;
        const uint32_t e0 = qr[(4 * g) * 32], e1 = qr[(4 * g + 1) * 32], e2 = qr[(4 * g + 2) * 32],
                       e3 = qr[(4 * g + 3) * 32];
        qb[h] = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
      }
      if (valid < kSumRows) {  // ragged last step: rows at or past M contribute exact zeros
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * g + e >= valid) pr[e] = make_uint4(0u, 0u, 0u, 0u);
        const uint32_t lo = 4 * g + 1 < valid ? 0xffffffffu : (4 * g < valid ? 0x0000ffffu : 0u);
        const uint32_t hi = 4 * g + 3 < valid ? 0xffffffffu : (4 * g + 2 < valid ? 0x0000ffffu : 0u);
#pragma unroll
        for (int h = 0; h < 2; ++h) qb[h] = make_uint2(qb[h].x & lo, qb[h].y & hi);
      }
      const uint32_t pw[4][4] = {{pr[0].x, pr[0].y, pr[0].z, pr[0].w},
                                 {pr[1].x, pr[1].y, pr[1].z, pr[1].w},
                                 {pr[2].x, pr[2].y, pr[2].z, pr[2].w},
                                 {pr[3].x, pr[3].y, pr[3].z, pr[3].w}};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        const uint2 a = make_uint2(__builtin_amdgcn_perm(pw[1][i >> 1], pw[0][i >> 1], sel),
                                   __builtin_amdgcn_perm(pw[3][i >> 1], pw[2][i >> 1], sel));
        acc[0][i] = mma16x16x16(a, qb[0], acc[0][i]);
        if (jb.nh > 1) acc[1][i] = mma16x16x16(a, qb[1], acc[1][i]);
      }
    }

    // row side
    if (jb.nr > 0) {
      f32x4_t ar[3] = {f32x4_t{}, f32x4_t{}, f32x4_t{}};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (cw + 32 * kb < C) {  // uniform
          const uint4 a = *reinterpret_cast<const uint4*>(st + t * kSumPitch + (128 * w + 32 * kb + 8 * g) * 2);
          ar[0] = mma_step<DT_BF16>(a, rreg[0][kb], ar[0]);
          if (jb.nr > 1) ar[1] = mma_step<DT_BF16>(a, rreg[1][kb], ar[1]);
          if (jb.nr > 2) ar[2] = mma_step<DT_BF16>(a, rreg[2][kb], ar[2]);
        }
      }
#pragma unroll
      for (int h = 0; h < 3; ++h)
        if (h < jb.nr)
          *reinterpret_cast<f32x4_t*>(red + (((s & 1) * 3 + h) * kSumWaves + w) * 256 + lane * 4) = ar[h];
      if (s > 0) store_rows(s - 1);
    }
  }
  if (jb.nr > 0) {
    __syncthreads();
    store_rows(nsteps - 1);
  }

  // column-side partials: MFMA i, register v of lane (g, t) = column cw + 8 (4 g + v) + i,
  // rank column 16 jbk + t
  const int64_t hstride = int64_t(jobs.chunks) * C * JB * 16;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h >= jb.nh) break;
    float* dst = colpart + jb.cp0 + h * hstride + (int64_t(rb) * C * JB + jbk) * 16 + t;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int c = cw + 8 * (4 * g + v) + i;
        if (c < C) dst[int64_t(c) * JB * 16] = acc[h][i][v];
      }
  }
}

hipError_t launch_sums(const SumJobs& jobs, float* rowpart, float* colpart, hipStream_t st) {
  if (jobs.n == 0 || jobs.M == 0) return hipSuccess;
  hipLaunchKernelGGL(sums_kernel, dim3(unsigned(jobs.blk0[jobs.n]), unsigned(jobs.chunks), unsigned(jobs.JB)),
                     dim3(kSumThreads), 0, st, jobs, rowpart, colpart);
  return hipGetLastError();
}

// One thread per (a, 4 adjacent columns) of each output: the np partial planes added in plane
// order (4 planes in flight), scaled, rounded once; columns r .. J - 1 written as zeros.
// Consecutive threads read consecutive 16-byte pieces of a plane.
__global__ __launch_bounds__(256) void reduce_sums_kernel(RedJobs jobs) {
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int JB = jobs.JB;
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    if (q >= jobs.n) return;
    const RedJob& jb = jobs.job[q];
    const int nb = (jb.J + 3) / 4;  // 4-column pieces per output row
    const int64_t total = int64_t(jb.A) * nb;
    if (i < total) {
      const int a = int(i / nb), b = int(i - int64_t(i / nb) * nb);
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * b < jb.r) {
        const float4* src = reinterpret_cast<const float4*>(jb.src + int64_t(a) * JB * 16) + b;
        const int64_t ps = jb.pstride / 4;
        int p = 0;
        for (; p + 4 <= jb.np; p += 4) {
          float4 v[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = src[(p + k) * ps];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            sum.x += v[k].x; sum.y += v[k].y; sum.z += v[k].z; sum.w += v[k].w;
          }
        }
        for (; p < jb.np; ++p) {
          const float4 v = src[p * ps];
          sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
        }
      }
      uint16_t* out = jb.out + int64_t(a) * jb.osa;
      const float sv[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = 4 * b + k;
        if (j < jb.J)
          out[int64_t(j) * jb.osj] = j < jb.r ? Traits<DT_BF16>::from_f32(jb.scale * sv[k]) : uint16_t(0);
      }
      return;
    }
    i -= total;
  }
}

hipError_t launch_reduce_sums(const RedJobs& jobs, hipStream_t st) {
  int64_t total = 0;
  for (int q = 0; q < jobs.n; ++q) total += int64_t(jobs.job[q].A) * ((jobs.job[q].J + 3) / 4);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_sums_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, st, jobs);
  return hipGetLastError();
}

}  // namespace lmx
