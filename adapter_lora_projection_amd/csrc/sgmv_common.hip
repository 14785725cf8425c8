// Dispatch of the SGMV kernels by storage type, kernel-shape tables, and the standalone segment
// scheduler with its tile-list export.
#include "device_common.hpp"
#include "schedule.hpp"
#include "sgmv_kernels.hpp"

namespace lmx {

hipError_t launch_shrink_bf16(const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st);
hipError_t launch_shrink_f16(const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st);
hipError_t launch_shrink_f32(const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st);
hipError_t launch_expand_bf16(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st);
hipError_t launch_shrink_sk_reduce_bf16(const ShrinkArgs& a, int bm, hipStream_t st);
hipError_t launch_shrink_sk_reduce_f16(const ShrinkArgs& a, int bm, hipStream_t st);
hipError_t launch_shrink_sk_reduce_f32(const ShrinkArgs& a, int bm, hipStream_t st);
hipError_t launch_expand_f16(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st);
hipError_t launch_expand_f32(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st);
hipError_t launch_pair_bf16(const ShrinkArgs& s, const ExpandArgs& e, const PairArgs& pa,
                            bool kfull, bool aligned_y, hipStream_t st);
hipError_t launch_pair_f16(const ShrinkArgs& s, const ExpandArgs& e, const PairArgs& pa,
                           bool kfull, bool aligned_y, hipStream_t st);

// Token rows per tile (16 * token groups) and waves of each kernel shape; these tables mirror the
// variant lists of sgmv_impl.hpp.
static const int kShrinkBM[] = {16, 32, 16, 32, 32};
static const int kShrinkWaves[] = {8, 4, 8, 4, 4};
static const int kShrinkCB[] = {1, 4, 1, 3, 3};
static const int kExpandBM[] = {16, 16, 16, 16, 16, 16, 16, 16, 64, 64};
static const int kExpandWaves[] = {4, 8, 4, 4, 8, 4, 4, 8, 1, 1};  // column-splitting waves
static const int kExpandChunk[] = {64, 64, 64, 64, 64, 128, 128, 128, 128, 128};

int num_shrink_variants() { return int(sizeof(kShrinkBM) / sizeof(int)); }
int num_expand_variants() { return int(sizeof(kExpandBM) / sizeof(int)); }
int shrink_plan_bm(int dtype, int variant) { return dtype == DT_F32 ? 16 : kShrinkBM[variant]; }
int shrink_plan_waves(int dtype, int variant) { return dtype == DT_F32 ? 8 : kShrinkWaves[variant]; }
int shrink_plan_cb(int dtype, int variant) { return dtype == DT_F32 ? 1 : kShrinkCB[variant]; }
// mirrors LMX_SHRINK_LDS_VARIANTS of shrink_lds.hpp
static const int kShrinkLdsNCB[] = {2, 3, 4, 8, 12, 3, 3, 3, 3, 3, 3, 3, 3};
static const int kShrinkLdsBMs[] = {128, 128, 128, 128, 128, 64, 64, 64, 32, 32, 64, 48, 48};
int num_shrink_lds_variants() { return int(sizeof(kShrinkLdsNCB) / sizeof(int)); }
int shrink_lds_ncb(int variant) { return kShrinkLdsNCB[variant]; }
int shrink_lds_bm(int variant) { return kShrinkLdsBMs[variant]; }
int expand_plan_bm(int dtype, int variant) { return dtype == DT_F32 ? 16 : kExpandBM[variant]; }
int expand_plan_waves(int dtype, int variant) { return dtype == DT_F32 ? 4 : kExpandWaves[variant]; }
int expand_plan_chunk(int dtype, int variant) { return dtype == DT_F32 ? 64 : kExpandChunk[variant]; }
int expand_max_rank(int dtype) { return 2 * (dtype == DT_F32 ? Traits<DT_F32>::kStep : Traits<DT_BF16>::kStep); }

hipError_t launch_shrink(int dtype, const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st) {
  switch (dtype) {
    case DT_F32: return launch_shrink_f32(a, plan, st);
    case DT_BF16: return launch_shrink_bf16(a, plan, st);
    default: return launch_shrink_f16(a, plan, st);
  }
}

hipError_t launch_shrink_sk_reduce(int dtype, const ShrinkArgs& a, int bm, hipStream_t st) {
  switch (dtype) {
    case DT_F32: return launch_shrink_sk_reduce_f32(a, bm, st);
    case DT_BF16: return launch_shrink_sk_reduce_bf16(a, bm, st);
    default: return launch_shrink_sk_reduce_f16(a, bm, st);
  }
}

hipError_t launch_expand(int dtype, const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st) {
  switch (dtype) {
    case DT_F32: return launch_expand_f32(a, plan, st);
    case DT_BF16: return launch_expand_bf16(a, plan, st);
    default: return launch_expand_f16(a, plan, st);
  }
}

hipError_t launch_pair(int dtype, const ShrinkArgs& s, const ExpandArgs& e, const PairArgs& pa,
                       bool kfull, bool aligned_y, hipStream_t st) {
  switch (dtype) {
    case DT_BF16: return launch_pair_bf16(s, e, pa, kfull, aligned_y, st);
    case DT_F16: return launch_pair_f16(s, e, pa, kfull, aligned_y, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_schedule(const int* seg_indptr, const int* weight_indices, int G, int BM,
                           int4* tiles, int* count, hipStream_t st) {
  hipLaunchKernelGGL((schedule_kernel<1024>), dim3(1), dim3(1024), 0, st, seg_indptr,
                     weight_indices, G, BM, tiles, count);
  return hipGetLastError();
}

// Export of the inline search: workgroup t runs the same search the compute kernels run and
// writes its tile (g, m0, mlen, a, r) at position t; the count is the number of valid tiles.
template <int NT>
__global__ __launch_bounds__(NT) void export_inline_tiles_kernel(
    const int* __restrict__ seg_indptr, const int* __restrict__ weight_indices,
    const int* __restrict__ lora_ranks, int G, int BM, int* __restrict__ out,
    int* __restrict__ count) {
  __shared__ Tile s_tile;
  __shared__ int s_scan[NT / 64];
  find_tile_inline<NT>(seg_indptr, weight_indices, lora_ranks, nullptr, G, BM, int(blockIdx.x),
                       &s_tile, s_scan);
  if (threadIdx.x == 0 && s_tile.g >= 0) {
    int* o = out + int64_t(blockIdx.x) * 5;
    o[0] = s_tile.g; o[1] = s_tile.m0; o[2] = s_tile.mlen; o[3] = s_tile.a; o[4] = s_tile.r;
    atomicAdd(count, 1);
  }
}

__global__ void export_list_tiles_kernel(const int4* __restrict__ tiles,
                                         const int* __restrict__ tile_count,
                                         const int* __restrict__ lora_ranks, int bound,
                                         int* __restrict__ out, int* __restrict__ count) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = *tile_count;
  if (t == 0) *count = n;
  if (t < n && t < bound) {
    const int4 v = tiles[t];
    int* o = out + int64_t(t) * 5;
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w; o[4] = lora_ranks[v.w];
  }
}

__global__ void zero_int_kernel(int* p) { *p = 0; }

hipError_t launch_zero_int(int* p, hipStream_t st) {
  hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, st, p);
  return hipGetLastError();
}

__global__ void zero_ints_kernel(int* p, int n) {
  const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_ints(int* p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_ints_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_export_tiles(int method, const int* seg_indptr, const int* weight_indices,
                               const int* lora_ranks, int G, int BM, int bound, int* out,
                               int* count, int4* ws_tiles, int* ws_count, hipStream_t st) {
  if (method == 0) {
    hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, st, count);
    hipLaunchKernelGGL((export_inline_tiles_kernel<256>), dim3(bound), dim3(256), 0, st,
                       seg_indptr, weight_indices, lora_ranks, G, BM, out, count);
    return hipGetLastError();
  }
  hipError_t e = launch_schedule(seg_indptr, weight_indices, G, BM, ws_tiles, ws_count, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(export_list_tiles_kernel, dim3((bound + 255) / 256), dim3(256), 0, st,
                     ws_tiles, ws_count, lora_ranks, bound, out, count);
  return hipGetLastError();
}

}  // namespace lmx
