// Embedding LoRA-A product of the multi-adapter LoRA ops ("Decode LoRA kernels are optimized",
// Summary and Behaviour changes: the embedding LoRA-A forward, driven by the same segment
// metadata, with no per-call device-to-host read): for sorted position i of a segment with
// adapter a and rank r,
//     h[i][j] = A[a][j][input_ids[perm[i]]]  for j < r,   0 for r <= j < R,
// a gather of one column of the adapter's A per token (values copied bit for bit).
//
// No tile list: every wave owns 64 consecutive sorted positions and finds their segments
// itself, so one launch of ceil(T / 256) workgroups does the whole op with no workspace and no
// segment-count-dependent serial step (the 16,384 one-token segments of the page's test cost the
// same as 4 long ones).
//   1. The wave's first covered position q0 is located with a 64-ary search over seg_indptr: each
//      lane tests one of 64 evenly spaced candidates and a ballot keeps the last one at or
//      before q0 (3 rounds for 16k segments).
//   2. Lane l loads the end of segment g0 + l; each lane counts the ends at or before its own
//      position with a 6-step shuffle search. Only when more than 63 segments end inside the
//      wave's 64 positions (empty segments) does a lane fall back to a binary search in memory.
//   3. The wave writes its [64][R] block of h with the rank index fastest across lanes: 16-byte
//      vectors when A has a unit rank stride (A kept as [L][V][R]: a token's r values are one
//      contiguous run), else one element per lane (A as [L][R][V]: every value is its own
//      memory sector).
// Every index is bounded for any metadata: a token whose id, adapter or permutation entry is out
// of range gets a row of zeros and reads nothing.
#include "device_common.hpp"
#include "embedding.hpp"

namespace lmx {

template <typename E, bool VEC>
__global__ __launch_bounds__(256) void embedding_a_kernel(EmbeddingArgs p) {
  const int lane = int(threadIdx.x & 63);
  const int p0 = (int(blockIdx.x) * 4 + int(threadIdx.x >> 6)) * 64;
  const int* __restrict__ indptr = p.seg_indptr;
  const int q0 = max(p0, indptr[0]);
  const int qend = min(min(p0 + 64, indptr[p.G]), p.T);
  if (q0 >= qend) return;  // nothing of this wave is covered (uniform over the wave)

  // 1. largest g in [0, G) with indptr[g] <= q0
  int lo = 0, hi = p.G - 1;
  while (lo < hi) {
    const int stride = (hi - lo + 64) / 64;
    const int c = lo + lane * stride;
    const bool pred = c <= hi && indptr[c] <= q0;
    const int nt = __popcll(__ballot(pred));
    lo += (nt > 0 ? nt - 1 : 0) * stride;
    hi = min(hi, lo + stride - 1);
  }
  const int g0 = lo;

  // 2. segment of this lane's position: g0 + #(ends of g0, g0 + 1, ... at or before it)
  const int pos = p0 + lane;
  const bool covered = pos >= q0 && pos < qend;
  const int e = indptr[min(g0 + 1 + lane, p.G)];
  const int e63 = __shfl(e, 63);
  int n = 0;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const int ev = __shfl(e, n + s - 1);
    if (ev <= pos) n += s;
  }
  int g = g0 + n;
  if (covered && n == 63 && e63 <= pos) {  // more than 63 segment ends in the way
    int a = g0 + 64, b = p.G - 1;
    while (a < b) {
      const int mid = a + (b - a + 1) / 2;
      if (indptr[mid] <= pos) a = mid; else b = mid - 1;
    }
    g = a;
  }
  int ad = 0, r = 0, id = 0;
  if (covered) {
    const int a = p.weight_indices[g];
    const int tok = p.permutation != nullptr ? p.permutation[pos] : pos;
    if (a >= 0 && a < p.L && tok >= 0 && tok < p.T) {
      id = p.input_ids[tok];
      if (id >= 0 && id < p.V) {
        ad = a;
        r = min(max(p.lora_ranks[a], 0), p.R);
      }
    }
  }

  // 3. the wave's [64][R] block of h
  const E* __restrict__ wa = reinterpret_cast<const E*>(p.w_a);
  E* __restrict__ h = reinterpret_cast<E*>(p.h);
  if constexpr (VEC) {
    constexpr int VE = 16 / int(sizeof(E));
    const int upr = p.R / VE;  // 16-byte units per row
    for (int it = 0; it < upr; ++it) {
      const int u = it * 64 + lane;
      const int m = u / upr, c = u - (u / upr) * upr;
      const int cov_m = __shfl(int(covered), m);
      const int a_m = __shfl(ad, m), r_m = __shfl(r, m), id_m = __shfl(id, m);
      if (!cov_m) continue;
      const int j0 = c * VE;
      const E* src = wa + int64_t(a_m) * p.stride_l + int64_t(id_m) * p.stride_v + j0;
      uint4 v = {0u, 0u, 0u, 0u};
      if (j0 + VE <= r_m) {
        v = *reinterpret_cast<const uint4*>(src);
      } else if (j0 < r_m) {
        E t[VE];
#pragma unroll
        for (int k = 0; k < VE; ++k) t[k] = (j0 + k < r_m) ? src[k] : E(0);
        v = *reinterpret_cast<const uint4*>(t);
      }
      *reinterpret_cast<uint4*>(h + int64_t(p0 + m) * p.ldh + j0) = v;
    }
  } else {
    for (int it = 0; it < p.R; ++it) {
      const int u = it * 64 + lane;
      const int m = u / p.R, j = u - (u / p.R) * p.R;
      const int cov_m = __shfl(int(covered), m);
      const int a_m = __shfl(ad, m), r_m = __shfl(r, m), id_m = __shfl(id, m);
      if (!cov_m) continue;
      E v = E(0);
      if (j < r_m)
        v = wa[int64_t(a_m) * p.stride_l + int64_t(j) * p.stride_r + int64_t(id_m) * p.stride_v];
      h[int64_t(p0 + m) * p.ldh + j] = v;
    }
  }
}

hipError_t launch_embedding_a(const EmbeddingArgs& a, int esize, bool vec, hipStream_t st) {
  const dim3 grid(unsigned((a.T + 255) / 256)), block(256);
  if (esize == 4) {
    if (vec) hipLaunchKernelGGL((embedding_a_kernel<uint32_t, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((embedding_a_kernel<uint32_t, false>), grid, block, 0, st, a);
  } else {
    if (vec) hipLaunchKernelGGL((embedding_a_kernel<uint16_t, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((embedding_a_kernel<uint16_t, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace lmx
