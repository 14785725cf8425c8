#pragma once
// Wave-reduction (GEMV-form) chunked-SGMV shrink for 16-bit types: the alternative to the MFMA
// tiles for skinny decode segments ("Decode LoRA kernels are optimized", Summary: gathered-A
// mainloop, one rank block per output slice).
//
// A workgroup owns one row tile of up to 16 sorted positions of one segment and one block of 16
// rank columns; each of its 4 waves owns 4 of those columns. Lane l reads 16 contiguous bytes
// (8 elements) of every row at k = 8 l + 512 i, so one load instruction covers 1 KiB of a row;
// the tile's x rows (through the permutation) are read by all 4 waves (the repeats hit the L1).
// Each lane accumulates its share of the 16 x 4 dot products with packed dot-product
// instructions (v_dot2, fp32 sums); the 64 partial sums of each product are then added across
// the wave with butterfly shuffles in a fixed order, and lane 0 of each 16-lane group rounds and
// stores. Requires 16-byte aligned x and A rows and K a multiple of 8 (the host checks); rows
// past the tile and rank columns past the padded rank read a valid row whose products are never
// stored (columns at or past the adapter's rank are stored as zeros).
#include "sgmv_impl.hpp"  // shrink_tile

namespace lmx {

template <int DT>
__device__ __forceinline__ float dot8(uint4 a, uint4 b, float acc) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == DT_BF16) {
      typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2_t, av[i]),
                                            __builtin_bit_cast(bf2_t, bv[i]), acc, false);
    } else {
      typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, av[i]), __builtin_bit_cast(h2_t, bv[i]),
                                   acc, false);
    }
  }
  return acc;
}

template <int DT>
__global__ __launch_bounds__(256) void shrink_gemv_kernel(ShrinkArgs p) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  constexpr int BM = 16, CPW = 4;  // tokens per tile, rank columns per wave
  __shared__ Tile s_tile;
  __shared__ int s_scan[4];
  const Tile tile = shrink_tile<256>(p, BM, int(blockIdx.x), &s_tile, s_scan);
  if (tile.g < 0) return;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int NB = (p.R + 15) >> 4;
  const int blk = int(blockIdx.y), s = blk / NB, b = blk - (blk / NB) * NB;
  const int K = int(p.K);
  const S* __restrict__ x = reinterpret_cast<const S*>(p.x);
  const S* __restrict__ wa = reinterpret_cast<const S*>(p.w_a);

  const S* xrow[BM];
#pragma unroll
  for (int t = 0; t < BM; ++t) {
    const int pos = tile.m0 + (t < tile.mlen ? t : 0);
    const int tok = p.permutation != nullptr ? p.permutation[pos] : pos;
    xrow[t] = x + int64_t(tok) * p.ldx;
  }
  const S* arow[CPW];
  {
    const S* base = wa + int64_t(tile.a * p.S + s) * p.R * p.lda;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int j = 16 * b + CPW * w + c;
      arow[c] = base + int64_t(j < p.R ? j : 0) * p.lda;
    }
  }

  float acc[BM][CPW];
#pragma unroll
  for (int t = 0; t < BM; ++t)
#pragma unroll
    for (int c = 0; c < CPW; ++c) acc[t][c] = 0.f;
  if (16 * b + CPW * w < p.R) {  // uniform per wave: this wave has a column inside the padded rank
    for (int k = 8 * lane; k < K; k += 512) {
      uint4 av[CPW], xv[BM];
#pragma unroll
      for (int c = 0; c < CPW; ++c) av[c] = gload16(arow[c] + k);
#pragma unroll
      for (int t = 0; t < BM; ++t) xv[t] = gload16(xrow[t] + k);
#pragma unroll
      for (int t = 0; t < BM; ++t)
#pragma unroll
        for (int c = 0; c < CPW; ++c) acc[t][c] = dot8<DT>(xv[t], av[c], acc[t][c]);
    }
  }
  // butterfly sums over the 64 lanes (the same order in every lane and every call)
#pragma unroll
  for (int t = 0; t < BM; ++t)
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      float v = acc[t][c];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      acc[t][c] = v;
    }
  // lane t * 4 + c (t < 16, c < 4) stores product (t, c)
  const int t = lane >> 2, c = lane & 3;
  float mine = 0.f;
#pragma unroll
  for (int tt = 0; tt < BM; ++tt)
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc)
      if (tt == t && cc == c) mine = acc[tt][cc];
  const int j = 16 * b + CPW * w + c;  // rank column inside the slice
  if (t < tile.mlen && j < p.R) {
    S* hrow = reinterpret_cast<S*>(p.h) + int64_t(tile.m0 + t) * p.ldh + s * p.R;
    hrow[j] = j < tile.r ? Tr::from_f32(mine) : S(0);
  }
}

template <int DT>
hipError_t launch_shrink_gemv_dt(const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st) {
  const int NB = (a.R + 15) / 16;
  hipLaunchKernelGGL((shrink_gemv_kernel<DT>), dim3(plan.grid_x, a.S * NB), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lmx
