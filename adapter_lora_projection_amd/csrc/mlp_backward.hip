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
// The Q values of 256 rows at a time are staged once in LDS as bf16 pairs of consecutive rows and
// read back as broadcasts; each thread pairs its P values of the same two rows, so one packed dot
// product (fp32 sum) adds both rows' terms. P rows are loaded 8 at a time, two groups in flight,
// so the loads of one group overlap the arithmetic of the previous one. The partial sums of the chunk go to part[job][(chunk * JB + z) * C + c][16];
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
  // Q of 256 rows at a time as bf16 pairs of consecutive rows: qs[p][j] = (Q[2p][j], Q[2p+1][j])
  __shared__ __align__(16) uint32_t qs[kColRows / 2][16];
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
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

  float acc[kColPerThread][16];
#pragma unroll
  for (int a = 0; a < kColPerThread; ++a)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[a][j] = 0.f;

  auto load_group = [&](uint2* dst, int mg, int mend) {
#pragma unroll
    for (int i = 0; i < kColGroup; ++i) {
      const int m = min(mg + i, mend - 1);  // past the end: a valid row, weighted by zero
      dst[i] = *reinterpret_cast<const uint2*>(P + int64_t(m) * jb.ldp);
    }
  };
  // rows mg + i, mg + i + 1 (i even): the second may lie past mend, where its Q pair half is 0
  auto add_group = [&](const uint2* src, int mg, int mend, int sb) {
#pragma unroll
    for (int i = 0; i < kColGroup; i += 2) {
      if (mg + i < mend) {  // uniform
        const bool two = mg + i + 1 < mend;
        const uint2 r0 = src[i];
        const uint2 r1 = two ? src[i + 1] : make_uint2(0u, 0u);
        // (P[m][c + a], P[m + 1][c + a]) for the lane's 4 columns
        uint32_t pp[4];
        pp[0] = __builtin_amdgcn_perm(r1.x, r0.x, 0x05040100u);
        pp[1] = __builtin_amdgcn_perm(r1.x, r0.x, 0x07060302u);
        pp[2] = __builtin_amdgcn_perm(r1.y, r0.y, 0x05040100u);
        pp[3] = __builtin_amdgcn_perm(r1.y, r0.y, 0x07060302u);
        const uint4* qr = reinterpret_cast<const uint4*>(qs[(mg + i - sb) >> 1]);
        uint32_t qp[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint4 t = qr[k];
          qp[4 * k] = t.x; qp[4 * k + 1] = t.y; qp[4 * k + 2] = t.z; qp[4 * k + 3] = t.w;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
          for (int a = 0; a < kColPerThread; ++a)
            acc[a][j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2_t, pp[a]),
                                                        __builtin_bit_cast(bf2_t, qp[j]),
                                                        acc[a][j], false);
      }
    }
  };

  for (int sb = m0; sb < m1; sb += kColRows) {
    const int se = min(m1, sb + kColRows);
    // stage the Q row pairs of [sb, se) (zeros past the block's valid columns and past se)
    __syncthreads();  // the previous rows' reads of qs are done
    if (tid < kColRows / 2 && sb + 2 * tid < se) {
      const uint16_t* q0 = Q + int64_t(sb + 2 * tid) * jb.ldq;
      const bool has1 = sb + 2 * tid + 1 < se;
      const uint16_t* q1 = has1 ? q0 + jb.ldq : q0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t lo = j < nvalid ? q0[j] : 0u;
        const uint32_t hi = (j < nvalid && has1) ? q1[j] : 0u;
        qs[tid][j] = lo | (hi << 16);
      }
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
