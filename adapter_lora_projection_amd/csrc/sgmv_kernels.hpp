// Internal launch interface of the SGMV kernels (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmx {

struct ShrinkArgs {
  const void* x;
  const void* w_a;
  const int* seg_indptr;
  const int* weight_indices;
  const int* permutation;
  const int* lora_ranks;
  void* h;
  const int4* tiles;      // prebuilt tile list, or null for the inline search
  const int* tile_count;  // its length (device), when tiles is non-null
  int64_t K, ldx, lda, ldh;
  int S, R, G;
};

struct ExpandArgs {
  const void* h;
  const void* w_b;
  const int* slice_offsets;
  const int* seg_indptr;
  const int* weight_indices;
  const int* permutation;
  const int* lora_ranks;
  const float* scalings;
  void* y;
  const int4* tiles;
  const int* tile_count;
  int64_t N, ldh, ldb, ldy;
  int S, R, G;
};

struct ShrinkPlan {
  int variant;  // kernel shape, see shrink_plan_bm
  int grid_x;   // tile-dimension bound ceil(T / BM) + G
};

struct ExpandPlan {
  int variant;
  int grid_x;
};

int shrink_plan_bm(int variant);
int expand_plan_bm(int variant);
int expand_plan_bn(int variant);

hipError_t launch_shrink(int dtype, const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st);
hipError_t launch_expand(int dtype, const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st);
hipError_t launch_schedule(const int* seg_indptr, const int* weight_indices, int G, int BM,
                           int4* tiles, int* count, hipStream_t st);
hipError_t launch_zero_int(int* p, hipStream_t st);
hipError_t launch_export_tiles(int method, const int* seg_indptr, const int* weight_indices,
                               const int* lora_ranks, int G, int BM, int bound, int* out,
                               int* count, int4* ws_tiles, int* ws_count, hipStream_t st);

}  // namespace lmx
