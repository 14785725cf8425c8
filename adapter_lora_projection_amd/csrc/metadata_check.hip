// Value checks of the LoRA metadata ("Decode LoRA kernels are optimized", Behaviour changes: the
// checks of seg_indptr, the index range and the permutation are taken off the fast path; invalid
// metadata there is undefined behaviour). Here they are an explicit call that waits for its own
// result. Rules, in the order their codes are reported:
//   1 seg_indptr: starts at 0, never decreases, ends at T;
//   2 weight_indices: inside [0, L);
//   3 lora_ranks: inside [0, R];
//   4 permutation (when given): every value in [0, T) exactly once;
//   5 slice_offsets (when given): start >= 0, never decrease, end at N.
// Every access is bounded by the sizes, so any metadata values are safe to check.
#include "device_common.hpp"
#include "metadata_check.hpp"

namespace lmx {

__global__ __launch_bounds__(256) void meta_clear_kernel(int* __restrict__ flag, int* __restrict__ counts,
                                                         int T) {
  const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (i == 0) *flag = 0;
  if (counts != nullptr && i < T) counts[i] = 0;
}

__global__ __launch_bounds__(256) void meta_check_kernel(MetaArgs a, int* __restrict__ flag,
                                                         int* __restrict__ counts) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  int bad = 0;
  if (i <= a.G) {
    const int v = a.seg_indptr[i];
    if (i == 0 && v != 0) bad |= 1 << 1;
    if (i == a.G && v != a.T) bad |= 1 << 1;
    if (i > 0 && v < a.seg_indptr[i - 1]) bad |= 1 << 1;
  }
  if (i < a.G) {
    const int w = a.weight_indices[i];
    if (w < 0 || w >= a.L) bad |= 1 << 2;
  }
  if (i < a.L) {
    const int r = a.lora_ranks[i];
    if (r < 0 || r > a.R) bad |= 1 << 3;
  }
  if (a.permutation != nullptr && i < a.T) {
    const int p = a.permutation[i];
    if (p < 0 || p >= a.T) bad |= 1 << 4;
    else atomicAdd(&counts[p], 1);
  }
  if (a.slice_offsets != nullptr && i <= a.S) {
    const int o = a.slice_offsets[i];
    if (i == 0 && o < 0) bad |= 1 << 5;
    if (i == a.S && int64_t(o) != a.N) bad |= 1 << 5;
    if (i > 0 && o < a.slice_offsets[i - 1]) bad |= 1 << 5;
  }
  if (bad) atomicOr(flag, bad);
}

__global__ __launch_bounds__(256) void meta_perm_kernel(const int* __restrict__ counts, int T,
                                                        int* __restrict__ flag) {
  const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (i < T && counts[i] != 1) atomicOr(flag, 1 << 4);
}

hipError_t launch_metadata_check(const MetaArgs& a, int* flag, int* counts, hipStream_t st) {
  const int64_t n = std::max<int64_t>({int64_t(a.G) + 1, int64_t(a.T), int64_t(a.L), int64_t(a.S) + 1});
  int* cnt = a.permutation != nullptr ? counts : nullptr;
  hipLaunchKernelGGL(meta_clear_kernel, dim3(unsigned((std::max<int64_t>(a.T, 1) + 255) / 256)), dim3(256),
                     0, st, flag, cnt, a.T);
  hipLaunchKernelGGL(meta_check_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, a, flag, cnt);
  if (cnt != nullptr && a.T > 0)
    hipLaunchKernelGGL(meta_perm_kernel, dim3(unsigned((a.T + 255) / 256)), dim3(256), 0, st, cnt, a.T,
                       flag);
  return hipGetLastError();
}

}  // namespace lmx
