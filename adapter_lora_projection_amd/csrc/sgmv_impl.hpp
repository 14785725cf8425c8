#pragma once
// Chunked-SGMV LoRA shrink and expand kernel templates for gfx950 (instantiated per storage type
// in sgmv_<type>.hip).
//
// Shrink ("Decode LoRA kernels are optimized", Summary: gathered-A mainloop, one rank block per
// output slice): a workgroup owns one row tile of one segment (up to 16*MT sorted positions) and
// CB column blocks of 16 rank columns. Its NW waves split the reduction dimension K in chunks of
// U fragment steps (chunk c goes to wave c mod NW); each wave reads the tile's x rows through the
// permutation and the adapter's A rows straight from global memory into MFMA operand registers
// (16 contiguous bytes per lane per step), double-buffering chunks in registers so the next
// chunk's loads are in flight during the current chunk's MFMAs. The waves' fp32 partial sums
// are added in a fixed order through LDS and rounded once to the storage type.
//
// Expand (same page: scatter epilogue applying scaling and slice offsets): a workgroup owns one
// row tile and a block of columns inside one slice; its waves walk the block in chunks of 64
// columns. For each chunk a wave computes D[col][token] = sum_j B[a][col][j] * h[token][s*R + j]
// (the rank is the reduction dimension) with its MFMA rows mapped so that every lane ends up
// holding 16 consecutive output columns of one token row; the lane's 16 entries of y are
// prefetched one chunk ahead, updated as round(y + scale * acc) and written back in place.
//
// Every operand load is branch-free (see Frag), so each wave keeps all its loads of a chunk in
// flight at once; the ALIGNED template variants are chosen by the host when base pointers and
// row strides keep every fragment 16-byte aligned.
#include "device_common.hpp"
#include "schedule.hpp"
#include "sgmv_kernels.hpp"

#include <type_traits>
#include <utility>

namespace lmx {

// ------------------------------------------------------------------------------------ shrink

// AL: x and A rows 16-byte aligned. KFULL: additionally K is a multiple of the chunk width, so
// no fragment is partial or past the end and no operand needs masking (a lane outside the tile
// or the rank only produces outputs that are never stored).
template <int DT, int MT, int CB, int NW, int D, bool AL, bool KFULL>
__global__ __launch_bounds__(NW * 64) void shrink_kernel(ShrinkArgs p) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  constexpr int NT = NW * 64;
  constexpr int KSTEP = Tr::kStep;
  constexpr int EPF = Tr::kPerFrag;
  constexpr int BM = 16 * MT;

  __shared__ Tile s_tile;
  __shared__ int s_scan[NW];
  __shared__ f32x4_t s_red[(NW > 1) ? NW : 1][CB * MT][64];

  Tile tile;
  if (p.seg_indptr != nullptr) {
    get_tile<NT>(p.seg_indptr, p.weight_indices, p.lora_ranks, nullptr, p.G, BM, p.tiles,
                 p.tile_count, int(blockIdx.x), &s_tile, s_scan);
    tile = s_tile;
  } else {  // dense: one segment over all rows
    tile.g = int(blockIdx.x) * BM < p.T ? 0 : -1;
    tile.m0 = int(blockIdx.x) * BM;
    tile.mlen = min(BM, p.T - tile.m0);
    tile.a = 0;
    tile.r = p.dense_rank;
  }
  if (tile.g < 0) return;

  const int lane = threadIdx.x & 63, w = wave_id();
  const int li = lane & 15, lg = lane >> 4;
  const int a = tile.a;
  const int r = tile.r;
  const int NB = (p.R + 15) >> 4;  // 16-column blocks per slice
  const int nblk = p.S * NB;
  const int K = int(p.K);

  const S* __restrict__ x = reinterpret_cast<const S*>(p.x);
  const S* __restrict__ wa = reinterpret_cast<const S*>(p.w_a);
  S* __restrict__ h = reinterpret_cast<S*>(p.h);

  // Operand rows of this lane; masked lanes keep a valid row and load nothing useful from it.
  const S* xrow[MT];
  bool tok_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + li;
    tok_ok[mt] = m < tile.mlen;
    const int pos = tile.m0 + (tok_ok[mt] ? m : 0);
    const int tok = p.permutation != nullptr ? p.permutation[pos] : pos;
    xrow[mt] = x + int64_t(tok) * p.ldx;
  }
  const S* arow[CB];
  bool col_ok[CB];
  bool any_col = false;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int blk = int(blockIdx.y) * CB + cb;
    const int s = blk / NB, b = blk - (blk / NB) * NB;
    const int j = 16 * b + li;
    col_ok[cb] = (blk < nblk) && (j < r);
    any_col |= (blk < nblk) && (16 * b < r);
    const int ss = blk < nblk ? s : 0;
    const S* slice_base = (ss < 4 && p.w_a_slice[ss] != nullptr)
                              ? reinterpret_cast<const S*>(p.w_a_slice[ss])
                              : wa + int64_t(a * p.S + ss) * p.R * p.lda;
    arow[cb] = slice_base + int64_t(col_ok[cb] ? j : 0) * p.lda;
  }

  f32x4_t acc[CB][MT];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[cb][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (any_col) {
    // Each wave owns a contiguous range of fragment steps. x (streamed from HBM) is fetched D
    // steps ahead in a register ring; A (small, L2-resident) one step ahead.
    const int nsteps = (K + KSTEP - 1) / KSTEP;
    const int per = (nsteps + NW - 1) / NW;
    const int s0 = w * per, s1 = min(s0 + per, nsteps);
    Frag<S, AL> xr[D][MT], ar[2][CB];
    auto fetch_x = [&](auto slot, int st) {
      constexpr int d = decltype(slot)::value;
      const int k = st * KSTEP + lg * EPF;
      const bool in = st < s1;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xr[d][mt].fetch(xrow[mt] + k, in ? (KFULL ? EPF : (tok_ok[mt] ? K - k : 0)) : 0, xrow[mt]);
    };
    auto fetch_a = [&](auto slot, int st) {
      constexpr int d = decltype(slot)::value;
      const int k = st * KSTEP + lg * EPF;
      const bool in = st < s1;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        ar[d][cb].fetch(arow[cb] + k, in ? (KFULL ? EPF : (col_ok[cb] ? K - k : 0)) : 0, arow[cb]);
    };
    using I0 = std::integral_constant<int, 0>;
    [&]<int... dd>(std::integer_sequence<int, dd...>) {
      (fetch_x(std::integral_constant<int, dd>{}, s0 + dd), ...);
    }(std::make_integer_sequence<int, D>{});
    fetch_a(I0{}, s0);
    for (int s = s0; s < s1; s += D) {
      [&]<int... dd>(std::integer_sequence<int, dd...>) {
        auto step = [&](auto ddc) {
          constexpr int d = decltype(ddc)::value;
          const int st = s + d;
          if (st < s1) {
            fetch_a(std::integral_constant<int, (d + 1) & 1>{}, st + 1);
            uint4 av[CB], xv[MT];
            const int kk = st * KSTEP + lg * EPF;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
              av[cb] = KFULL ? ar[d & 1][cb].raw() : ar[d & 1][cb].masked(col_ok[cb] ? K - kk : 0);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              xv[mt] = KFULL ? xr[d][mt].raw() : xr[d][mt].masked(tok_ok[mt] ? K - kk : 0);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) acc[cb][mt] = mma_step<DT>(av[cb], xv[mt], acc[cb][mt]);
            fetch_x(ddc, st + D);
          }
        };
        (step(std::integral_constant<int, dd>{}), ...);
      }(std::make_integer_sequence<int, D>{});
    }
  }

  // fixed-order reduction of the waves' partial sums
  if constexpr (NW > 1) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) s_red[w][cb * MT + mt][lane] = acc[cb][mt];
    __syncthreads();
  }

  for (int idx = w; idx < CB * MT; idx += NW) {
    const int cb = idx / MT, mt = idx - (idx / MT) * MT;
    f32x4_t sum;
    if constexpr (NW > 1) {
      sum = s_red[0][idx][lane];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) sum += s_red[w2][idx][lane];
    } else {
      sum = acc[0][0];
#pragma unroll
      for (int c2 = 0; c2 < CB; ++c2)
#pragma unroll
        for (int m2 = 0; m2 < MT; ++m2)
          if (c2 * MT + m2 == idx) sum = acc[c2][m2];
    }
    const int blk = int(blockIdx.y) * CB + cb;
    if (blk >= nblk) continue;
    const int m = mt * 16 + li;
    if (m >= tile.mlen) continue;
    const int s = blk / NB, b = blk - (blk / NB) * NB;
    S* hrow = h + int64_t(tile.m0 + m) * p.ldh + s * p.R;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = 16 * b + 4 * lg + v;  // rank column inside the slice
      if (c < p.R) hrow[c] = (c < r) ? Tr::from_f32(sum[v]) : S(0);
    }
  }
}

// ------------------------------------------------------------------------------------ expand

// One wave computes a 16-token x 64-column chunk as D[token][col] = sum_j h[token][s*R+j] *
// B[a][col][j]: h rows are the MFMA A operand (constant over the chunks), B rows the B operand.
// MFMA column block q, column index c maps to output column cbase + 4c + q, so lane (g, c) holds
// the 4 consecutive columns cbase + 4c .. +3 of tokens 4g .. 4g+3, and one 8-byte access per token
// covers 128 contiguous bytes of 4 rows per instruction. y and B of a chunk are fetched together
// into a D-deep ring, so data are consumed in the order they were requested.
template <int DT, int NW, int JS, int D, bool ALB, bool ALY>
__device__ __forceinline__ void expand_body(const ExpandArgs& p, const Tile& tile, int s, int nb0,
                                            int nblen) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  constexpr int KSTEP = Tr::kStep;
  constexpr int EPF = Tr::kPerFrag;
  constexpr int NY = 4 * int(sizeof(S)) / 8;  // 8-byte pieces per lane and token (4 elements)

  const int lane = threadIdx.x & 63, w = wave_id();
  const int c = lane & 15, g = lane >> 4;
  const int a = tile.a, r = tile.r;
  const float sigma = tile.sigma;
  const int nend = nb0 + nblen;
  const int nchunks = (nblen + 63) >> 6;
  const int nci = w < nchunks ? (nchunks - w + NW - 1) / NW : 0;  // this wave's chunks

  const S* __restrict__ hbuf = reinterpret_cast<const S*>(p.h);
  const S* __restrict__ wb = reinterpret_cast<const S*>(p.w_b);
  S* __restrict__ y = reinterpret_cast<S*>(p.y);

  // A operand: h row of token c of the tile (constant over the chunks)
  uint4 hv[JS];
  {
    const bool ok = c < tile.mlen;
    const S* hrow = hbuf + int64_t(tile.m0 + (ok ? c : 0)) * p.ldh + s * p.R;
    Frag<S, ALB> hf[JS];
#pragma unroll
    for (int js = 0; js < JS; ++js) {
      const int j = js * KSTEP + g * EPF;
      hf[js].fetch(hrow + j, r - j, hrow);
    }
#pragma unroll
    for (int js = 0; js < JS; ++js) hv[js] = hf[js].masked(r - (js * KSTEP + g * EPF));
  }
  // output rows of tokens 4g .. 4g+3
  S* yrow[4];
  bool tok_ok[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    tok_ok[v] = m < tile.mlen;
    yrow[v] = y + int64_t(p.permutation[tile.m0 + (tok_ok[v] ? m : 0)]) * p.ldy;
  }
  const S* bblk = wb + int64_t(a) * p.N * p.ldb;  // adapter a's rows of B

  Frag8<S, ALY> yr[D][4][NY];
  Frag<S, ALB> br[D][JS][4];
  auto fetch = [&](auto slot, int i) {
    constexpr int d = decltype(slot)::value;
    const int cbase = nb0 + (w + i * NW) * 64;
    const bool in = i < nci;
    // B rows of columns cbase + 4c + q (first so that they are consumed first)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = cbase + 4 * c + q;
      const S* brow = bblk + int64_t((in && col < nend) ? col : nb0) * p.ldb;
#pragma unroll
      for (int js = 0; js < JS; ++js) {
        const int j = js * KSTEP + g * EPF;
        br[d][js][q].fetch(brow + j, in ? r - j : 0, brow);
      }
    }
    const int c0 = cbase + 4 * c;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int valid = (in && tok_ok[v]) ? nend - c0 : 0;
#pragma unroll
      for (int n = 0; n < NY; ++n) {
        constexpr int per = 8 / int(sizeof(S));
        yr[d][v][n].fetch(yrow[v] + c0 + n * per, valid - n * per, yrow[v] + nb0);
      }
    }
  };
  auto do_chunk = [&](auto slot, int i) {
    constexpr int d = decltype(slot)::value;
    f32x4_t acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int js = 0; js < JS; ++js) {
      uint4 bv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) bv[q] = br[d][js][q].masked(r - (js * KSTEP + g * EPF));
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = mma_step<DT>(hv[js], bv[q], acc[q]);
    }
    // epilogue: y = round(y + scale * acc) for tokens 4g+v, columns c0 .. c0+3
    const int c0 = nb0 + (w + i * NW) * 64 + 4 * c;
    const int ncols = min(4, nend - c0);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      union {
        uint2 u[NY];
        S e[4];
      } o;
#pragma unroll
      for (int n = 0; n < NY; ++n) o.u[n] = yr[d][v][n].raw();
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o.e[q] = Tr::from_f32(__builtin_fmaf(sigma, acc[q][v], Tr::to_f32(o.e[q])));
      if (tok_ok[v] && ncols > 0) {
        S* dst = yrow[v] + c0;
        if (ALY && ncols == 4) {
#pragma unroll
          for (int n = 0; n < NY; ++n) reinterpret_cast<uint2*>(dst)[n] = o.u[n];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q < ncols) dst[q] = o.e[q];
        }
      }
    }
    fetch(slot, i + D);
  };
  [&]<int... dd>(std::integer_sequence<int, dd...>) {
    (fetch(std::integral_constant<int, dd>{}, dd), ...);
  }(std::make_integer_sequence<int, D>{});
  for (int i = 0; i < nci; i += D) {
    [&]<int... dd>(std::integer_sequence<int, dd...>) {
      auto one = [&](auto ddc) {
        constexpr int d = decltype(ddc)::value;
        if (i + d < nci) do_chunk(ddc, i + d);
      };
      (one(std::integral_constant<int, dd>{}), ...);
    }(std::make_integer_sequence<int, D>{});
  }
}

template <int DT, int NW, int JS, int D, bool ALB, bool ALY>
__global__ __launch_bounds__(NW * 64) void expand_kernel(ExpandArgs p) {
  constexpr int NT = NW * 64;
  constexpr int BM = 16;

  __shared__ Tile s_tile;
  __shared__ int s_scan[NW];

  get_tile<NT>(p.seg_indptr, p.weight_indices, p.lora_ranks, p.scalings, p.G, BM, p.tiles,
               p.tile_count, int(blockIdx.x), &s_tile, s_scan);
  const Tile tile = s_tile;
  if (tile.g < 0 || tile.r <= 0) return;  // a rank-0 adapter leaves y untouched
  int s, nb0, nblen;
  if (!find_nblock(p.slice_offsets, p.S, p.BN, int(blockIdx.y), &s, &nb0, &nblen)) return;
  if constexpr (ALY) {
    // whole 8-byte pieces only when the block starts on an 8-byte boundary
    if ((nb0 * int(sizeof(typename Traits<DT>::store_t))) % 8 != 0) {
      expand_body<DT, NW, JS, D, ALB, false>(p, tile, s, nb0, nblen);
      return;
    }
  }
  expand_body<DT, NW, JS, D, ALB, ALY>(p, tile, s, nb0, nblen);
}

// ------------------------------------------------------------------------------------ launchers

// Kernel shapes. Shrink: (token groups of 16 per tile, 16-column blocks per workgroup, waves,
// ring depth of the streamed x fragments). Expand: (waves, ring depth of the
// streamed y chunks); expand tiles are 16 tokens. fp32 (small correctness workloads) has one
// shape of each.
#define LMX_SHRINK_VARIANTS(X) \
  X(0, 1, 1, 16, 4)            \
  X(1, 2, 4, 8, 8)             \
  X(2, 2, 4, 4, 4)             \
  X(3, 1, 1, 8, 4)
#define LMX_EXPAND_VARIANTS(X) \
  X(0, 4, 3)                   \
  X(1, 8, 2)                   \
  X(2, 4, 4)

template <int DT, int MT, int CB, int NW, int D>
static hipError_t launch_shrink_t(const ShrinkArgs& a, bool aligned, int grid_x, hipStream_t st) {
  const int NB = (a.R + 15) / 16;
  const int nblk = a.S * NB;
  dim3 grid(grid_x, (nblk + CB - 1) / CB);
  const bool kfull = a.K % Traits<DT>::kStep == 0;
  if (aligned && kfull)
    hipLaunchKernelGGL((shrink_kernel<DT, MT, CB, NW, D, true, true>), grid, dim3(NW * 64), 0, st, a);
  else if (aligned)
    hipLaunchKernelGGL((shrink_kernel<DT, MT, CB, NW, D, true, false>), grid, dim3(NW * 64), 0, st, a);
  else
    hipLaunchKernelGGL((shrink_kernel<DT, MT, CB, NW, (D > 2 ? D / 2 : D), false, false>), grid,
                       dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_shrink_dt(const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st) {
  if constexpr (DT == DT_F32) {
    return launch_shrink_t<DT, 1, 1, 8, 4>(a, plan.aligned, plan.grid_x, st);
  } else {
    switch (plan.variant) {
#define X(V, MT, CB, NW, D) \
      case V: return launch_shrink_t<DT, MT, CB, NW, D>(a, plan.aligned, plan.grid_x, st);
      LMX_SHRINK_VARIANTS(X)
#undef X
    }
    return hipErrorInvalidValue;
  }
}

template <int DT, int NW, int JS, int D>
static void launch_expand_al(const ExpandArgs& a, const ExpandPlan& plan, dim3 grid, hipStream_t st) {
  dim3 block(NW * 64);
  if (plan.aligned_b && plan.aligned_y)
    hipLaunchKernelGGL((expand_kernel<DT, NW, JS, D, true, true>), grid, block, 0, st, a);
  else if (plan.aligned_b)
    hipLaunchKernelGGL((expand_kernel<DT, NW, JS, D, true, false>), grid, block, 0, st, a);
  else if (plan.aligned_y)
    hipLaunchKernelGGL((expand_kernel<DT, NW, JS, D, false, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((expand_kernel<DT, NW, JS, D, false, false>), grid, block, 0, st, a);
}

template <int DT, int NW, int D>
static hipError_t launch_expand_t(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st) {
  const int64_t gy = (a.N + a.BN - 1) / a.BN + a.S;
  dim3 grid(plan.grid_x, unsigned(gy));
  constexpr int KS = Traits<DT>::kStep;
  const int js = (a.R + KS - 1) / KS;
  if (js <= 1) launch_expand_al<DT, NW, 1, D>(a, plan, grid, st);
  else if (js == 2) launch_expand_al<DT, NW, 2, D>(a, plan, grid, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int DT>
hipError_t launch_expand_dt(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st) {
  if constexpr (DT == DT_F32) {
    return launch_expand_t<DT, 4, 2>(a, plan, st);
  } else {
    switch (plan.variant) {
#define X(V, NW, D) \
      case V: return launch_expand_t<DT, NW, D>(a, plan, st);
      LMX_EXPAND_VARIANTS(X)
#undef X
    }
    return hipErrorInvalidValue;
  }
}

}  // namespace lmx
