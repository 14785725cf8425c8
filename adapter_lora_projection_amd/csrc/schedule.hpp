// Device-side segment scheduler.
//
// The compute kernels are launched on a grid whose tile dimension is the host-known bound
// ceil(T / BM) + G, so no device-to-host read is needed to size a launch (the on-device segment
// scheduler of "Decode LoRA kernels are optimized", Summary). Tile t of the segment-major list is
// found from seg_indptr by each workgroup (inline search: one coalesced pass over seg_indptr in
// chunks of the workgroup size and a block scan of per-segment tile counts), or read from a list
// built once by the standalone scheduler kernel when the segment count is large.
#pragma once

#include "device_common.hpp"

namespace lmx {

// Tile record: segment, first sorted position, rows, adapter, its rank and scaling.
struct Tile {
  int g, m0, mlen, a, r;
  float sigma;
};

// Inclusive scan over the workgroup; `scratch` holds one int per wave. Contains barriers:
// every thread of the workgroup must call it.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* scratch, int* total) {
  constexpr int NWAVE = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) scratch[w] = v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) {
    int s = scratch[i];
    before += (i < w) ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

// Finds tile `t` (segment-major, BM rows) by scanning seg_indptr. Result in `out` (LDS),
// out->g = -1 when t is past the last tile. Every thread must call it. RANK: the winning thread
// also loads the adapter's rank and (when `scalings` is non-null) scaling into the record, one
// more dependent load before the record is published; without it they are left 0 and the
// caller loads them itself, off the chain that leads to its operand loads.
template <int NT, bool RANK = true>
__device__ __forceinline__ void find_tile_inline(const int* __restrict__ seg_indptr,
                                                 const int* __restrict__ weight_indices,
                                                 const int* __restrict__ lora_ranks,
                                                 const float* __restrict__ scalings, int G,
                                                 int BM, int t, Tile* out, int* scan_scratch) {
  if (threadIdx.x == 0) out->g = -1;
  int carry = 0;
  for (int c0 = 0; c0 < G; c0 += NT) {
    const int g = c0 + int(threadIdx.x);
    int lo = 0, len = 0, a = 0;
    if (g < G) {
      lo = seg_indptr[g];
      len = max(seg_indptr[g + 1] - lo, 0);
      a = weight_indices[g];
    }
    const int nt = (len + BM - 1) / BM;
    int total;
    const int incl = block_inclusive_scan<NT>(nt, scan_scratch, &total);
    const int excl = incl - nt;
    if (g < G && t >= carry + excl && t < carry + incl) {
      const int k = t - carry - excl;
      out->g = g;
      out->m0 = lo + k * BM;
      out->mlen = min(BM, len - k * BM);
      out->a = a;
      out->r = RANK ? lora_ranks[a] : 0;
      out->sigma = (RANK && scalings != nullptr) ? scalings[a] : 0.f;
    }
    carry += total;
    if (t < carry) break;  // uniform: carry and t are the same in every thread
  }
  __syncthreads();
}

// Standalone scheduler: one workgroup writes the whole tile list and its length.
template <int NT>
__global__ __launch_bounds__(NT) void schedule_kernel(const int* __restrict__ seg_indptr,
                                                      const int* __restrict__ weight_indices,
                                                      int G, int BM, int4* __restrict__ tiles,
                                                      int* __restrict__ count) {
  __shared__ int s_scan[NT / 64];
  __shared__ int s_incl[NT];
  __shared__ int s_lo[NT];
  int carry = 0;
  for (int c0 = 0; c0 < G; c0 += NT) {
    const int g = c0 + int(threadIdx.x);
    int lo = 0, len = 0;
    if (g < G) {
      lo = seg_indptr[g];
      len = max(seg_indptr[g + 1] - lo, 0);
    }
    const int nt = (len + BM - 1) / BM;
    int total;
    const int incl = block_inclusive_scan<NT>(nt, s_scan, &total);
    s_incl[threadIdx.x] = incl;
    s_lo[threadIdx.x] = lo;
    __syncthreads();
    const int nseg = min(NT, G - c0);
    for (int t = int(threadIdx.x); t < total; t += NT) {
      // first segment of the chunk whose inclusive count exceeds t
      int lo_i = 0, hi_i = nseg - 1;
      while (lo_i < hi_i) {
        const int mid = (lo_i + hi_i) >> 1;
        if (s_incl[mid] > t) hi_i = mid; else lo_i = mid + 1;
      }
      const int excl = (lo_i == 0) ? 0 : s_incl[lo_i - 1];
      const int k = t - excl;
      const int seg_lo = s_lo[lo_i];
      const int seg_len = seg_indptr[c0 + lo_i + 1] - seg_lo;
      tiles[carry + t] = make_int4(c0 + lo_i, seg_lo + k * BM, min(BM, seg_len - k * BM),
                                   weight_indices[c0 + lo_i]);
    }
    carry += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) *count = carry;
}

// Tile for this workgroup: from the prebuilt list when `tiles` is non-null, else inline. RANK as
// for find_tile_inline.
template <int NT, bool RANK = true>
__device__ __forceinline__ void get_tile(const int* __restrict__ seg_indptr,
                                         const int* __restrict__ weight_indices,
                                         const int* __restrict__ lora_ranks,
                                         const float* __restrict__ scalings, int G, int BM,
                                         const int4* __restrict__ tiles,
                                         const int* __restrict__ tile_count, int t, Tile* out,
                                         int* scan_scratch) {
  if (tiles != nullptr) {
    if (threadIdx.x == 0) {
      if (t < *tile_count) {
        const int4 v = tiles[t];
        out->g = v.x; out->m0 = v.y; out->mlen = v.z; out->a = v.w;
        out->r = RANK ? lora_ranks[v.w] : 0;
        out->sigma = (RANK && scalings != nullptr) ? scalings[v.w] : 0.f;
      } else {
        out->g = -1;
      }
    }
    __syncthreads();
  } else {
    find_tile_inline<NT, RANK>(seg_indptr, weight_indices, lora_ranks, scalings, G, BM, t, out,
                               scan_scratch);
  }
}

// The adapter's rank and scaling of a tile found without them (get_tile<NT, false>). Operand
// loads issued before their first use do not wait for these two loads.
__device__ __forceinline__ void tile_rank(const int* __restrict__ lora_ranks,
                                          const float* __restrict__ scalings, Tile* t) {
  const int a = __builtin_amdgcn_readfirstlane(t->a);
  t->r = lora_ranks[a];
  t->sigma = scalings != nullptr ? scalings[a] : 0.f;
}

// Column blocks from slice bounds held one slice per lane (S <= 64): slice_lanes loads them
// (before the tile search, so the loads overlap its own), find_nblock_lanes finds block b with
// a wave prefix sum. Same blocking as find_nblock.
struct SliceLane {
  int lo, hi;
};
__device__ __forceinline__ SliceLane slice_lanes(const int* __restrict__ slice_offsets, int S) {
  const int k = int(threadIdx.x) & 63;
  SliceLane v{0, 0};
  if (k < S) {
    v.lo = slice_offsets[k];
    v.hi = slice_offsets[k + 1];
  }
  return v;
}
__device__ __forceinline__ bool find_nblock_lanes(SliceLane v, int S, int BN, int b, int* s_out,
                                                  int* n0_out, int* nlen_out) {
  const int k = int(threadIdx.x) & 63;
  const int len = k < S ? max(v.hi - v.lo, 0) : 0;
  const int nb = (len + BN - 1) / BN;
  int incl = nb;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (k >= d) incl += o;
  }
  const int excl = incl - nb;
  const unsigned long long hit = __ballot(k < S && b >= excl && b < incl);
  if (hit == 0) return false;
  const int ks = __ffsll(hit) - 1;
  const int lo = __shfl(v.lo, ks, 64), ln = __shfl(len, ks, 64), ex = __shfl(excl, ks, 64);
  *s_out = ks;
  *n0_out = lo + (b - ex) * BN;
  *nlen_out = min(BN, ln - (b - ex) * BN);
  return true;
}

}  // namespace lmx
