// Chunked-SGMV LoRA shrink and expand kernels for gfx950.
//
// Shrink ("Decode LoRA kernels are optimized", Summary: gathered-A mainloop, one rank block per
// output slice): a workgroup owns one row tile of one segment (up to 16*MT sorted positions) and
// CB column blocks of 16 rank columns. Its NW waves split the reduction dimension K in
// interleaved fragment steps; each wave reads the tile's x rows through the permutation and the
// adapter's A rows straight from global memory into MFMA operand registers (16 contiguous bytes
// per lane per step), accumulates D[col][token] in fp32, and the partial sums of the waves are
// added in a fixed order through LDS before one rounding to the storage type.
//
// Expand (same page: scatter epilogue applying scaling and slice offsets): a workgroup owns one
// row tile and one column block of NW*64 columns inside one slice. Each wave computes a 64x(16*MT)
// block of D[col][token] = sum_j B[a][col][j] * h[token][s*R + j] with the rank as reduction
// dimension, its MFMA rows mapped so that every lane ends up holding 16 consecutive output
// columns of one token; the epilogue reads those y entries of the token's row, adds the scaled
// product and writes them back with one rounding.
#include "device_common.hpp"
#include "schedule.hpp"
#include "sgmv_kernels.hpp"

namespace lmx {

// ------------------------------------------------------------------------------------ shrink

template <int DT, int MT, int CB, int NW>
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

  get_tile<NT>(p.seg_indptr, p.weight_indices, p.G, BM, p.tiles, p.tile_count, int(blockIdx.x),
               &s_tile, s_scan);
  const Tile tile = s_tile;
  if (tile.g < 0) return;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int a = tile.a;
  const int r = p.lora_ranks[a];
  const int NB = (p.R + 15) >> 4;  // 16-column blocks per slice
  const int nblk = p.S * NB;

  const S* __restrict__ x = reinterpret_cast<const S*>(p.x);
  const S* __restrict__ wa = reinterpret_cast<const S*>(p.w_a);
  S* __restrict__ h = reinterpret_cast<S*>(p.h);

  // operand rows of this lane
  const S* xrow[MT];
  bool tok_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + li;
    tok_ok[mt] = m < tile.mlen;
    const int tok = tok_ok[mt] ? p.permutation[tile.m0 + m] : 0;
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
    arow[cb] = wa + (int64_t(a * p.S + s) * p.R + (col_ok[cb] ? j : 0)) * p.lda;
  }

  f32x4_t acc[CB][MT];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[cb][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (any_col) {
    const int64_t K = p.K;
    for (int64_t k0 = int64_t(w) * KSTEP; k0 < K; k0 += int64_t(NW) * KSTEP) {
      const int64_t k = k0 + lg * EPF;
      uint4 af[CB], xf[MT];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        af[cb] = col_ok[cb] ? load_frag<S>(arow[cb], k, K) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xf[mt] = tok_ok[mt] ? load_frag<S>(xrow[mt], k, K) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[cb][mt] = mma_step<DT>(af[cb], xf[mt], acc[cb][mt]);
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

template <int DT, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void expand_kernel(ExpandArgs p) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  constexpr int NT = NW * 64;
  constexpr int KSTEP = Tr::kStep;
  constexpr int EPF = Tr::kPerFrag;
  constexpr int BM = 16 * MT;
  constexpr int BN = NW * 64;

  __shared__ Tile s_tile;
  __shared__ int s_scan[NW];

  get_tile<NT>(p.seg_indptr, p.weight_indices, p.G, BM, p.tiles, p.tile_count, int(blockIdx.x),
               &s_tile, s_scan);
  const Tile tile = s_tile;
  if (tile.g < 0) return;
  int s, nb0, nblen;
  if (!find_nblock(p.slice_offsets, p.S, BN, int(blockIdx.y), &s, &nb0, &nblen)) return;
  const int a = tile.a;
  const int r = p.lora_ranks[a];
  if (r <= 0) return;  // a rank-0 adapter leaves y untouched
  const float sigma = p.scalings[a];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int wbase = w * 64;  // first column of this wave inside the block
  if (wbase >= nblen) return;
  const int nend = nb0 + nblen;  // one past the last column of the block

  const S* __restrict__ hbuf = reinterpret_cast<const S*>(p.h);
  const S* __restrict__ wb = reinterpret_cast<const S*>(p.w_b);
  S* __restrict__ y = reinterpret_cast<S*>(p.y);

  // B operand rows: MFMA row i of column group q holds column wbase + (i/4)*16 + q*4 + i%4, so
  // lane group lg ends up with the 16 consecutive columns wbase + 16*lg .. +15.
  const S* brow[4];
  bool bcol_ok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int col = nb0 + wbase + (li >> 2) * 16 + q * 4 + (li & 3);
    bcol_ok[q] = col < nend;
    brow[q] = wb + (int64_t(a) * p.N + (bcol_ok[q] ? col : nb0)) * p.ldb;
  }
  const S* hrow[MT];
  bool tok_ok[MT];
  int yrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + li;
    tok_ok[mt] = m < tile.mlen;
    hrow[mt] = hbuf + int64_t(tile.m0 + (tok_ok[mt] ? m : 0)) * p.ldh + s * p.R;
    yrow[mt] = tok_ok[mt] ? p.permutation[tile.m0 + m] : 0;
  }

  f32x4_t acc[4][MT];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[q][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int j0 = 0; j0 < r; j0 += KSTEP) {
    const int j = j0 + lg * EPF;
    uint4 bf[4], hf[MT];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      bf[q] = bcol_ok[q] ? load_frag<S>(brow[q], j, r) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      hf[mt] = tok_ok[mt] ? load_frag<S>(hrow[mt], j, r) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[q][mt] = mma_step<DT>(bf[q], hf[mt], acc[q][mt]);
  }

  // scatter epilogue: lane holds columns c0 .. c0+15 of token row yrow[mt]
  const int c0 = nb0 + wbase + 16 * lg;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (!tok_ok[mt]) continue;
    S* yp = y + int64_t(yrow[mt]) * p.ldy + c0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int cc = q * 4 + v;
        if (c0 + cc < nend) {
          const float old = Tr::to_f32(yp[cc]);
          yp[cc] = Tr::from_f32(__builtin_fmaf(sigma, acc[q][mt][v], old));
        }
      }
  }
}

// ------------------------------------------------------------------------------------ launchers

template <int DT, int MT, int CB, int NW>
static hipError_t launch_shrink_t(const ShrinkArgs& a, int grid_x, hipStream_t st) {
  const int NB = (a.R + 15) / 16;
  const int nblk = a.S * NB;
  dim3 grid(grid_x, (nblk + CB - 1) / CB);
  hipLaunchKernelGGL((shrink_kernel<DT, MT, CB, NW>), grid, dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_shrink_dt(const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st) {
  switch (plan.variant) {
    case 0: return launch_shrink_t<DT, 1, 1, 16>(a, plan.grid_x, st);
    case 1: return launch_shrink_t<DT, 2, 2, 8>(a, plan.grid_x, st);
    default: return launch_shrink_t<DT, 4, 4, 4>(a, plan.grid_x, st);
  }
}

hipError_t launch_shrink(int dtype, const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st) {
  switch (dtype) {
    case DT_F32: return launch_shrink_dt<DT_F32>(a, plan, st);
    case DT_BF16: return launch_shrink_dt<DT_BF16>(a, plan, st);
    default: return launch_shrink_dt<DT_F16>(a, plan, st);
  }
}

int shrink_plan_bm(int variant) { return variant == 0 ? 16 : (variant == 1 ? 32 : 64); }

template <int DT, int MT, int NW>
static hipError_t launch_expand_t(const ExpandArgs& a, int grid_x, hipStream_t st) {
  constexpr int BN = NW * 64;
  const int64_t gy = (a.N + BN - 1) / BN + a.S;
  dim3 grid(grid_x, unsigned(gy));
  hipLaunchKernelGGL((expand_kernel<DT, MT, NW>), grid, dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_expand_dt(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st) {
  switch (plan.variant) {
    case 0: return launch_expand_t<DT, 1, 4>(a, plan.grid_x, st);
    default: return launch_expand_t<DT, 4, 4>(a, plan.grid_x, st);
  }
}

hipError_t launch_expand(int dtype, const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st) {
  switch (dtype) {
    case DT_F32: return launch_expand_dt<DT_F32>(a, plan, st);
    case DT_BF16: return launch_expand_dt<DT_BF16>(a, plan, st);
    default: return launch_expand_dt<DT_F16>(a, plan, st);
  }
}

int expand_plan_bm(int variant) { return variant == 0 ? 16 : 64; }
int expand_plan_bn(int variant) { (void)variant; return 256; }

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
  find_tile_inline<NT>(seg_indptr, weight_indices, G, BM, int(blockIdx.x), &s_tile, s_scan);
  if (threadIdx.x == 0 && s_tile.g >= 0) {
    int* o = out + int64_t(blockIdx.x) * 5;
    o[0] = s_tile.g; o[1] = s_tile.m0; o[2] = s_tile.mlen; o[3] = s_tile.a;
    o[4] = lora_ranks[s_tile.a];
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
