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
  int T;  // tokens (rows of x and of h); permutation == nullptr means the identity
  // Stream-K mode when sk_q > 0: the work [0, sk_tiles * steps) is cut into ranges of sk_q
  // steps, one per workgroup x; the pieces go to part[plane < sk_mp][T][S*R] (fp32, rows by
  // sorted position) and launch_shrink_sk_reduce adds them into h.
  int64_t sk_q;
  int sk_tiles, sk_mp;
  int sk_unit;  // reduction indices per unit of work (the kernel's step)
  float* part;
  // Non-null in stream-K mode: arrival counters [tiles bound][grid rows], zero on entry and on
  // exit; the last workgroup to store a piece of a tile adds the tile's planes into h in the
  // same launch (no launch_shrink_sk_reduce).
  int* counters;
  int ctr_shift;  // counter (tile, grid row) sits at index (tile * rows + row) << ctr_shift
  // Direct mode only (register-ring and LDS-staged kernels): > 0 launches a one-dimensional grid
  // that gives each XCD a contiguous range of tiles, the xcd_rows column-block groups of a tile
  // on consecutive workgroups of that XCD (0: a 2-D grid).
  int xcd_rows;
};

// Single-launch shrink + expand (decode sizes): workgroups [0, shrink_wgs) run the split shrink
// grid (sgx x sgy, x fastest; its arrival counters in ShrinkArgs::counters), the rest the 16-token
// expand grid (egx tiles x egy column blocks).
struct PairArgs {
  int shrink_wgs, sgx, sgy;
  int egx, egy;
  int* done;  // [tiles bound]: expand workgroups finished with the tile, zero on entry and exit
  int* err;   // set to 1 if a wait ever exceeded its bound (never cleared by the library)
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
  int BN;  // columns per workgroup block (a multiple of 64 * waves)
};

struct ShrinkPlan {
  int variant;   // kernel shape (of the register-ring kernel, or of the LDS-staged one)
  int grid_x;    // direct: tile bound ceil(T / BM) + G; stream-K: workgroups with work
  bool aligned;  // x, A bases and row strides are 16-byte aligned
  bool lds;      // the LDS-staged kernel (16-bit types, aligned rows, K % 8 == 0)
  bool gemv;     // the wave-reduction kernel (16-bit types, aligned rows, K % 8 == 0; direct)
};

struct ExpandPlan {
  int variant;
  int grid_x;
  bool aligned_b;  // h, B bases and row strides (and the slice width R) are 16-byte aligned
  bool aligned_y;  // y base and row stride are 16-byte aligned
};

int num_shrink_variants();
int num_expand_variants();
// Expand shapes of the shared-B kernel (64-token tiles, B chunks through LDS): slice rank exactly
// 16, 16-bit types, 16-byte aligned h, B and y rows. Their column unit is one 128-column chunk.
constexpr int kExpandSharedD1 = 8;
constexpr int kExpandSharedD2 = 9;
int shrink_plan_bm(int dtype, int variant);
int expand_plan_bm(int dtype, int variant);
int expand_plan_waves(int dtype, int variant);
int expand_plan_chunk(int dtype, int variant);  // columns per wave chunk (64 or 128)
int expand_max_rank(int dtype);  // largest padded rank the expand kernels take

hipError_t launch_shrink(int dtype, const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st);
// Second launch of a stream-K shrink: one workgroup per tile adds its pieces in order.
hipError_t launch_shrink_sk_reduce(int dtype, const ShrinkArgs& a, int bm, hipStream_t st);
int shrink_plan_waves(int dtype, int variant);
int shrink_plan_cb(int dtype, int variant);
int num_shrink_lds_variants();
int shrink_lds_ncb(int variant);          // 16-column blocks per workgroup
int shrink_lds_bm(int variant);           // positions per tile
constexpr int kShrinkLdsUnit = 64;        // reduction indices per stage
hipError_t launch_expand(int dtype, const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st);
// Single-launch shrink + expand (16-bit types; shrink shape 2, split with in-launch completion,
// 16-byte aligned x and A rows; 64-column expand with 16-byte aligned h and B rows, padded rank
// <= 32).
hipError_t launch_pair(int dtype, const ShrinkArgs& s, const ExpandArgs& e, const PairArgs& pa,
                       bool kfull, bool aligned_y, hipStream_t st);
hipError_t launch_schedule(const int* seg_indptr, const int* weight_indices, int G, int BM,
                           int4* tiles, int* count, hipStream_t st);
hipError_t launch_zero_int(int* p, hipStream_t st);
// Clears n ints with a fill kernel (no memset node when captured in a graph).
hipError_t launch_zero_ints(int* p, int n, hipStream_t st);
hipError_t launch_export_tiles(int method, const int* seg_indptr, const int* weight_indices,
                               const int* lora_ranks, int G, int BM, int bound, int* out,
                               int* count, int4* ws_tiles, int* ws_count, hipStream_t st);

}  // namespace lmx
