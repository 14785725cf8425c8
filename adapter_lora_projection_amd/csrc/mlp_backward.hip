// Kernels of the single-adapter LoRA MLP backward beyond the GEMMs ("Add optional fast lora path
// for qwen2/qwen3 on npu", review thread and Verification advice: the backward of the fast path
// takes the saved X and gate/up projections, runs the SwiGLU backward, forms dX and the LoRA A/B
// gradients, and never overwrites X):
//   * transposes of the frozen weights (once per layer: the backward's GEMMs read them with the
//     reduction index contiguous, as the forward's do);
//   * small transposed / scaled / zero-padded copies of the LoRA operands;
//   * sums over tokens for the LoRA weight gradients (dA = dxa^T P, dB = s dP^T xa).
#include "device_common.hpp"
#include "mlp_kernels.hpp"

namespace lmx {

// ---- small transposed copies -------------------------------------------------------------
// One thread per destination element; the jobs are laid end to end over the grid.
__global__ __launch_bounds__(256) void small_transposes_kernel(TJobs jobs) {
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    if (q >= jobs.n) return;
    const TJob& jb = jobs.job[q];
    const int64_t total = int64_t(jb.rows) * jb.cols;
    if (i < total) {
      const int row = int(i / jb.cols), c = int(i - int64_t(i / jb.cols) * jb.cols);
      uint16_t v = 0;
      const int k = c - jb.c0;
      if (k >= 0 && k < jb.cn)
        v = Traits<DT_BF16>::from_f32(jb.scale * Traits<DT_BF16>::to_f32(jb.src[int64_t(k) * jb.lds + row]));
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

// ---- sums over tokens --------------------------------------------------------------------
// Workgroup (x = column block of 1024 columns of one job, y = chunk of rows, z = block of 16 of
// the nq columns of Q): each thread owns 4 adjacent columns of P and the 16 Q columns, so it
// keeps 64 fp32 sums and reads P with 8-byte loads (a wave covers 512 contiguous bytes of a row).
// The Q values of 256 rows at a time are staged once in LDS as fp32 and read back as broadcasts;
// P rows are loaded 8 at a time, two groups in flight, so the loads of one group overlap the FMAs
// of the previous one. The partial sums of the chunk go to part[job][(chunk * JB + z) * C + c][16];
// a second kernel adds the chunks in order.
namespace {
constexpr int kColThreads = 256;
constexpr int kColPerThread = 4;
constexpr int kColBlock = kColThreads * kColPerThread;  // 1024 columns per workgroup
constexpr int kColRows = 256;                            // Q rows staged in LDS at a time
constexpr int kColGroup = 8;                             // P rows per load group

struct ColGeom {
  int blk0[7];       // first column block of each job (prefix)
  int64_t part0[7];  // first partial float of each job
};

int jblocks(int nq) { return (nq + 15) / 16; }

ColGeom col_geom(const ColJobs& j) {
  ColGeom g{};
  for (int q = 0; q < j.n; ++q) {
    g.blk0[q + 1] = g.blk0[q] + (j.job[q].C + kColBlock - 1) / kColBlock;
    g.part0[q + 1] = g.part0[q] + int64_t(j.chunks) * jblocks(j.job[q].nq) * j.job[q].C * 16;
  }
  return g;
}
}  // namespace

size_t colred_partial_floats(const ColJobs& jobs) { return size_t(col_geom(jobs).part0[jobs.n]); }

__global__ __launch_bounds__(kColThreads) void colred_kernel(ColJobs jobs, ColGeom geo, float* part) {
  __shared__ __align__(16) float qs[kColRows][16];
  // this workgroup's job (uniform; constant-index selection keeps the job table in registers)
  int q = 0;
#pragma unroll
  for (int k = 1; k < 6; ++k)
    if (k < jobs.n && int(blockIdx.x) >= geo.blk0[k]) q = k;
  ColJob jb = jobs.job[0];
  int blk0 = geo.blk0[0];
  int64_t part0 = geo.part0[0];
#pragma unroll
  for (int k = 1; k < 6; ++k)
    if (q == k) { jb = jobs.job[k]; blk0 = geo.blk0[k]; part0 = geo.part0[k]; }
  const int JB = (jb.nq + 15) / 16;
  const int zb = int(blockIdx.z);
  if (zb >= JB) return;  // uniform over the workgroup
  const int tid = int(threadIdx.x);
  const int c = (int(blockIdx.x) - blk0) * kColBlock + tid * kColPerThread;
  const bool active = c < jb.C;
  const int cc = active ? c : 0;  // inactive threads read column 0 (never stored)
  const int rows_per = (jobs.M + jobs.chunks - 1) / jobs.chunks;
  const int m0 = int(blockIdx.y) * rows_per, m1 = min(jobs.M, m0 + rows_per);
  const int nvalid = min(16, jb.nq - 16 * zb);  // Q columns of this block (uniform)
  const uint16_t* __restrict__ P = jb.P + cc;
  const uint16_t* __restrict__ Q = jb.Q + 16 * zb;

  float acc[kColPerThread][16];
#pragma unroll
  for (int a = 0; a < kColPerThread; ++a)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[a][j] = 0.f;

  auto load_group = [&](uint2* dst, int mg, int mend) {
#pragma unroll
    for (int i = 0; i < kColGroup; ++i) {
      const int m = min(mg + i, mend - 1);  // past the end: a valid row, never added
      dst[i] = *reinterpret_cast<const uint2*>(P + int64_t(m) * jb.ldp);
    }
  };
  auto add_group = [&](const uint2* src, int mg, int mend, int sb) {
#pragma unroll
    for (int i = 0; i < kColGroup; ++i) {
      if (mg + i < mend) {  // uniform
        float pf[4];
        pf[0] = __uint_as_float(src[i].x << 16);
        pf[1] = __uint_as_float(src[i].x & 0xffff0000u);
        pf[2] = __uint_as_float(src[i].y << 16);
        pf[3] = __uint_as_float(src[i].y & 0xffff0000u);
        const float4* qr = reinterpret_cast<const float4*>(qs[mg + i - sb]);
        float qv[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 t = qr[k];
          qv[4 * k] = t.x; qv[4 * k + 1] = t.y; qv[4 * k + 2] = t.z; qv[4 * k + 3] = t.w;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
          for (int a = 0; a < kColPerThread; ++a) acc[a][j] = fmaf(pf[a], qv[j], acc[a][j]);
      }
    }
  };

  for (int sb = m0; sb < m1; sb += kColRows) {
    const int se = min(m1, sb + kColRows);
    // stage the Q rows [sb, se) as fp32 (zeros past the block's valid columns)
    __syncthreads();  // the previous rows' reads of qs are done
    if (sb + tid < se) {
      const uint16_t* qrow = Q + int64_t(sb + tid) * jb.ldq;
#pragma unroll
      for (int j = 0; j < 16; ++j) qs[tid][j] = j < nvalid ? Traits<DT_BF16>::to_f32(qrow[j]) : 0.f;
    }
    __syncthreads();
    uint2 ga[kColGroup], gb[kColGroup];
    load_group(ga, sb, se);
    for (int mg = sb; mg < se; mg += 2 * kColGroup) {
      load_group(gb, mg + kColGroup, se);
      add_group(ga, mg, se, sb);
      load_group(ga, mg + 2 * kColGroup, se);
      add_group(gb, mg + kColGroup, se, sb);
    }
  }

  if (active) {
    float* dst = part + part0 + ((int64_t(blockIdx.y) * JB + zb) * jb.C + c) * 16;
#pragma unroll
    for (int a = 0; a < kColPerThread; ++a)
#pragma unroll
      for (int j = 0; j < 16; j += 4)
        *reinterpret_cast<float4*>(dst + a * 16 + j) =
            make_float4(acc[a][j], acc[a][j + 1], acc[a][j + 2], acc[a][j + 3]);
  }
}

// One thread per output element (c, j) of each job: the chunk partials added in chunk order,
// scaled, rounded once and stored at out[c * osc + j * osj].
__global__ __launch_bounds__(256) void colred_reduce_kernel(ColJobs jobs, ColGeom geo,
                                                            const float* __restrict__ part) {
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    if (q >= jobs.n) return;
    const ColJob& jb = jobs.job[q];
    const int64_t total = int64_t(jb.C) * jb.nq;
    if (i < total) {
      const int c = int(i / jb.nq), j = int(i - int64_t(i / jb.nq) * jb.nq);
      const int JB = (jb.nq + 15) / 16;
      const int64_t plane = int64_t(JB) * jb.C * 16;  // floats per chunk
      const float* src = part + geo.part0[q] + (int64_t(j >> 4) * jb.C + c) * 16 + (j & 15);
      float sum = 0.f;
      for (int ch = 0; ch < jobs.chunks; ++ch) sum += src[ch * plane];
      jb.out[int64_t(c) * jb.osc + int64_t(j) * jb.osj] = Traits<DT_BF16>::from_f32(jb.scale * sum);
      return;
    }
    i -= total;
  }
}

hipError_t launch_colred(const ColJobs& jobs, float* part, hipStream_t st) {
  if (jobs.n == 0 || jobs.M == 0) return hipSuccess;
  const ColGeom geo = col_geom(jobs);
  int jbmax = 1;
  int64_t outs = 0;
  for (int q = 0; q < jobs.n; ++q) {
    jbmax = max(jbmax, jblocks(jobs.job[q].nq));
    outs += int64_t(jobs.job[q].C) * jobs.job[q].nq;
  }
  hipLaunchKernelGGL(colred_kernel, dim3(unsigned(geo.blk0[jobs.n]), unsigned(jobs.chunks), unsigned(jbmax)),
                     dim3(kColThreads), 0, st, jobs, geo, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colred_reduce_kernel, dim3(unsigned((outs + 255) / 256)), dim3(256), 0, st,
                     jobs, geo, part);
  return hipGetLastError();
}

}  // namespace lmx
