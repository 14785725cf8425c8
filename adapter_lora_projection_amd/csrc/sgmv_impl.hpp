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

#include <algorithm>
#include <type_traits>
#include <utility>

namespace lmx {

// ------------------------------------------------------------------------------------ shrink

// Tile t of a shrink call, from the segment schedule. Every thread must call it. The adapter's
// rank is loaded after the search and first needed by the stores: operand loads read the padded
// rank (every padded row of the stacked A exists; rows at or past the adapter's rank only feed
// outputs that are stored as zeros) and do not wait for it.
template <int NT>
__device__ __forceinline__ Tile shrink_tile(const ShrinkArgs& p, int BM, int t, Tile* s_tile,
                                            int* s_scan) {
  get_tile<NT, false>(p.seg_indptr, p.weight_indices, p.lora_ranks, nullptr, p.G, BM, p.tiles,
                      p.tile_count, t, s_tile, s_scan);
  Tile tile = *s_tile;
  if (tile.g >= 0) tile_rank(p.lora_ranks, nullptr, &tile);
  return tile;
}

// Planes of tile t in a shared-work shrink: its (tile, step) units [t * nunits, (t+1) * nunits)
// fall into the ranges of workgroups first .. last, with first = t * nunits / q; plane j holds
// the piece of workgroup first + j.
__device__ __forceinline__ int sk_pieces(int t, int64_t nunits, int64_t q) {
  const int64_t first = (int64_t(t) * nunits) / q;
  const int64_t last = ((int64_t(t) + 1) * nunits - 1) / q;
  return int(last - first + 1);
}

// Partial sums of a shared-work shrink cross workgroups, and so compute units and XCDs. They are
// written and read as device-scope relaxed atomics (stores that write through the L2 to the
// device coherence point; loads that do not hit a stale cached copy), so no whole-cache
// write-back or invalidation fence is needed: a store is visible device-wide once it has
// completed (s_waitcnt vmcnt(0)).
__device__ __forceinline__ void part_store(float* q, float v) {
  __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float part_load(const float* q) {
  return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait of the single-launch shrink + expand for a counter to reach `target` (the whole
// wave reads the same counter, so the loop is uniform). Shrink workgroups come first in the
// launch and never wait, so the counters always fill; the bound (one second of the 100 MHz
// real-time counter) only guarantees that every wave ends: past it the wave sets *err and goes on.
constexpr uint64_t kPairWaitTicks = 100000000ull;
__device__ __forceinline__ void wait_count(const int* ctr, int target, int* err) {
  if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(4);
    if (__builtin_amdgcn_s_memrealtime() - t0 > kPairWaitTicks) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
}

// Completion of a shared-work shrink inside its own launch (p.counters non-null), called by
// every thread of the workgroup right after its piece of tile t went to plane j (fp32 sums of
// the rank columns of this grid row's CBY column blocks). Each workgroup waits until its
// partial stores have completed, then counts its piece in on the arrival counter of
// (tile, grid row); the workgroup that arrives last adds the np planes in plane order, whatever
// the order of arrival (so the result does not depend on timing), rounds once, writes h with
// exact zeros in the rank padding, and sets the counter back to zero, so every counter is zero
// again when the launch ends. A rank-0 tile stores no pieces: its plane-0 workgroup writes its
// zero rows. EU outputs per thread and pass keep their plane loads in flight together (the loads
// go to the device coherence point; one output at a time pays a full memory round trip each):
// the LDS-staged kernel's long tiles take 4, which took its 2048-token, four-piece split from
// 26.8 to 19.1 us; the register ring takes 1, since the 32 extra load addresses doubled its
// registers (78 -> 154 VGPRs, 6 -> 3 waves per SIMD) and its 288-workgroup decode grid at
// 128 tokens then needed a second round (10.1 -> 13.6 us).
template <int DT, int NT, int EU, bool KEEP = false>
__device__ void sk_finish(const ShrinkArgs& p, const Tile& tile, int t, int j, int np, int CBY,
                          int by, int ny, int* s_last) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  const int NB = (p.R + 15) >> 4;
  const int nblk = p.S * NB;
  const int SR = p.S * p.R;
  if (tile.r > 0) {
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
    __syncthreads();                // ... and every other thread's
    if (threadIdx.x == 0) {
      int* ctr = p.counters + ((int64_t(t) * ny + by) << p.ctr_shift);
      const int before = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = before == np - 1;
      // (KEEP: the single-launch shrink + expand, whose expand workgroups wait for the count
      // and clear it)
      if (last && !KEEP) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_last = last;
    }
    __syncthreads();
    if (!*s_last) return;  // uniform over the workgroup
  } else if (j != 0) {
    return;
  }
  const int b0 = by * CBY;
  const int nb = min(CBY, nblk - b0);
  const int W = nb * 16;
  const int n = tile.mlen * W;
  const int64_t plane = int64_t(p.T) * SR;
  for (int e0 = int(threadIdx.x); e0 < n; e0 += NT * EU) {
    int64_t off[EU], hoff[EU];
    bool live[EU], has[EU];
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      const int e = e0 + u * NT;
      live[u] = false;
      has[u] = false;
      off[u] = 0;
      hoff[u] = 0;
      if (e < n) {
        const int m = e / W, rem = e - (e / W) * W;
        const int blk = b0 + (rem >> 4);
        const int s = blk / NB, c = 16 * (blk - (blk / NB) * NB) + (rem & 15);
        if (c < p.R) {
          live[u] = true;
          has[u] = c < tile.r;
          off[u] = int64_t(tile.m0 + m) * SR + s * p.R + c;
          hoff[u] = int64_t(tile.m0 + m) * p.ldh + s * p.R + c;
        }
      }
    }
    float acc[EU];
#pragma unroll
    for (int u = 0; u < EU; ++u) acc[u] = 0.f;
    for (int q0 = 0; q0 < np; q0 += 8) {
      float b[EU][8];
#pragma unroll
      for (int u = 0; u < EU; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          b[u][i] = (has[u] && q0 + i < np) ? part_load(p.part + off[u] + (q0 + i) * plane) : 0.f;
#pragma unroll
      for (int u = 0; u < EU; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (q0 + i < np) acc[u] = (q0 + i == 0) ? b[u][i] : acc[u] + b[u][i];
    }
#pragma unroll
    for (int u = 0; u < EU; ++u)
      if (live[u]) reinterpret_cast<S*>(p.h)[hoff[u]] = has[u] ? Tr::from_f32(acc[u]) : S(0);
  }
}

// One piece of shrink work: reduction steps [k0, k1) of `tile` for the column blocks of this
// workgroup (grid y). Returns, in `out`, the workgroup's fp32 sums in MFMA layout for the
// (column block, token group) pairs idx = w, w + NW, ... that this wave finalises.
//
// AL: x and A rows 16-byte aligned. KFULL: additionally K is a multiple of the step width, so no
// fragment is partial or past the end and no operand needs masking (a lane outside the tile or
// the rank only produces outputs that are never stored).
template <int DT, int MT, int CB, int NW, int D, bool AL, bool KFULL>
__device__ __forceinline__ void shrink_piece(const ShrinkArgs& p, const Tile& tile, int by, int k0,
                                             int k1, f32x4_t (*s_red)[CB * MT][64],
                                             f32x4_t (&out)[(CB * MT + NW - 1) / NW]) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  constexpr int KSTEP = Tr::kStep;
  constexpr int EPF = Tr::kPerFrag;

  const int lane = threadIdx.x & 63, w = wave_id();
  const int li = lane & 15, lg = lane >> 4;
  const int a = tile.a;
  const int r = p.R;  // rows of A the loads may read (the rank applies in the stores)
  const int NB = (p.R + 15) >> 4;  // 16-column blocks per slice
  const int nblk = p.S * NB;
  const int K = int(p.K);

  const S* __restrict__ x = reinterpret_cast<const S*>(p.x);
  const S* __restrict__ wa = reinterpret_cast<const S*>(p.w_a);

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
    const int blk = by * CB + cb;
    const int s = blk / NB, b = blk - (blk / NB) * NB;
    const int j = 16 * b + li;
    col_ok[cb] = (blk < nblk) && (j < r);
    any_col |= (blk < nblk) && (16 * b < r);
    const int ss = blk < nblk ? s : 0;
    const S* slice_base = wa + int64_t(a * p.S + ss) * p.R * p.lda;
    arow[cb] = slice_base + int64_t(col_ok[cb] ? j : 0) * p.lda;
  }

  f32x4_t acc[CB][MT];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[cb][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (any_col) {
    // Each wave owns a contiguous part of the piece's steps. The A and x fragments of a step are
    // fetched together D steps ahead into one register ring, so the loads complete in the order
    // they are consumed and a wait for one step never drains a later step's loads.
    const int per = (max(0, k1 - k0) + NW - 1) / NW;
    const int s0 = k0 + w * per, s1 = min(s0 + per, k1);
    const int cnt = max(0, s1 - s0);
    Frag<S, AL> xr[D][MT], ar[D][CB];
    auto fetch = [&](auto slot, int q) {
      constexpr int d = decltype(slot)::value;
      const bool in = q < cnt;
      const int k = (in ? s0 + q : s0) * KSTEP + lg * EPF;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        ar[d][cb].fetch(arow[cb] + k, in ? (KFULL ? EPF : (col_ok[cb] ? K - k : 0)) : 0, arow[cb]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xr[d][mt].fetch(xrow[mt] + k, in ? (KFULL ? EPF : (tok_ok[mt] ? K - k : 0)) : 0, xrow[mt]);
    };
    // The scheduler must not reorder the ring's loads: a wait is a count of outstanding loads,
    // so a slot issued out of order makes the first wait inside the loop drain the whole ring.
    [&]<int... dd>(std::integer_sequence<int, dd...>) {
      ((fetch(std::integral_constant<int, dd>{}, dd), __builtin_amdgcn_sched_barrier(0)), ...);
    }(std::make_integer_sequence<int, D>{});
    auto consume = [&](auto slot, int q) {
      constexpr int d = decltype(slot)::value;
      uint4 av[CB], xv[MT];
      const int kk = (s0 + q) * KSTEP + lg * EPF;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        av[cb] = KFULL ? ar[d][cb].raw() : ar[d][cb].masked(col_ok[cb] ? K - kk : 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xv[mt] = KFULL ? xr[d][mt].raw() : xr[d][mt].masked(tok_ok[mt] ? K - kk : 0);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[cb][mt] = mma_step<DT>(av[cb], xv[mt], acc[cb][mt]);
    };
    // Full groups of D steps run without guards, so every path into a wait has the same loads
    // outstanding and each wait is exactly "this slot's loads have landed". The last partial
    // group consumes what the ring already holds and fetches nothing.
    const int nfull = cnt / D;
    for (int gi = 0; gi < nfull; ++gi) {
      const int q0 = gi * D;
      [&]<int... dd>(std::integer_sequence<int, dd...>) {
        auto step = [&](auto ddc) {
          constexpr int d = decltype(ddc)::value;
          consume(ddc, q0 + d);
          __builtin_amdgcn_sched_barrier(0);
          fetch(ddc, q0 + d + D);
          __builtin_amdgcn_sched_barrier(0);
        };
        (step(std::integral_constant<int, dd>{}), ...);
      }(std::make_integer_sequence<int, D>{});
    }
    const int rem = cnt - nfull * D;
    const int qt = nfull * D;
    [&]<int... dd>(std::integer_sequence<int, dd...>) {
      auto tail = [&](auto ddc) {
        constexpr int d = decltype(ddc)::value;
        if (d < rem) consume(ddc, qt + d);
      };
      (tail(std::integral_constant<int, dd>{}), ...);
    }(std::make_integer_sequence<int, D>{});
  }

  // fixed-order reduction of the waves' partial sums
  if constexpr (NW > 1) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) s_red[w][cb * MT + mt][lane] = acc[cb][mt];
    __syncthreads();
#pragma unroll
    for (int n = 0; n < (CB * MT + NW - 1) / NW; ++n) {
      const int idx = w + n * NW;
      if (idx < CB * MT) {
        f32x4_t sum = s_red[0][idx][lane];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) sum += s_red[w2][idx][lane];
        out[n] = sum;
      }
    }
    __syncthreads();  // s_red is reused by the next piece
  } else {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) out[cb * MT + mt] = acc[cb][mt];
  }
}

// Shrink. Direct mode (sk_q == 0): workgroup x = tile x, all K steps, h written here.
// Stream-K mode: the flattened work [0, tiles bound * steps) is cut into equal ranges of sk_q
// steps, one per workgroup x, so every compute unit streams the same amount whatever the
// segment lengths; each tile piece of a range is written as fp32 partial sums to plane
// j = workgroup - first workgroup of the tile, rows = the tile's sorted positions, and the
// planes are added in order by the tile's last workgroup (sk_finish, with arrival counters) or
// by shrink_sk_reduce_kernel in a second launch.
template <int MT, int CB, int NW>
struct ShrinkSmem {
  Tile tile;
  int scan[NW];
  int last;
  f32x4_t red[(NW > 1) ? NW : 1][CB * MT][64];
};

// One shrink workgroup (bx, by) of a gdx x gdy grid. KEEP (the single-launch shrink + expand):
// the arrival counters of a split are left at the piece count for the expand workgroups.
template <int DT, int MT, int CB, int NW, int D, bool AL, bool KFULL, bool KEEP>
__device__ __forceinline__ void shrink_wg(const ShrinkArgs& p, int bx, int by_in, int gdx,
                                          int gdy, ShrinkSmem<MT, CB, NW>& sm) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  constexpr int NT = NW * 64;
  constexpr int BM = 16 * MT;
  constexpr int NOUT = (CB * MT + NW - 1) / NW;
  Tile* const s_tile = &sm.tile;
  int* const s_scan = sm.scan;
  auto s_red = sm.red;

  const int lane = threadIdx.x & 63, w = wave_id();
  const int li = lane & 15, lg = lane >> 4;
  const int NB = (p.R + 15) >> 4;
  const int nblk = p.S * NB;
  const int64_t nsteps = (p.K + Tr::kStep - 1) / Tr::kStep;

  // Stores the sums this wave finalises: to h (rounded) or to a partial slot (fp32).
  auto store = [&](const Tile& tile, int by, const f32x4_t (&sums)[NOUT], float* slot) {
#pragma unroll
    for (int n = 0; n < NOUT; ++n) {
      const int idx = (NW > 1) ? w + n * NW : n;
      if (idx >= CB * MT) continue;
      const int cb = idx / MT, mt = idx - (idx / MT) * MT;
      const int blk = by * CB + cb;
      const int m = mt * 16 + li;
      if (blk >= nblk || m >= tile.mlen) continue;
      const int s = blk / NB, b = blk - (blk / NB) * NB;
      if (slot != nullptr) {
        float* prow = slot + int64_t(m) * (p.S * p.R) + s * p.R;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int c = 16 * b + 4 * lg + v;
          if (c < tile.r) part_store(prow + c, sums[n][v]);
        }
      } else {
        S* hrow = reinterpret_cast<S*>(p.h) + int64_t(tile.m0 + m) * p.ldh + s * p.R;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int c = 16 * b + 4 * lg + v;  // rank column inside the slice
          if (c < p.R) hrow[c] = (c < tile.r) ? Tr::from_f32(sums[n][v]) : S(0);
        }
      }
    }
  };

  if (p.sk_q == 0) {
    // Direct mode. With several grid rows (column-block groups) the grid is one-dimensional
    // (p.xcd_rows > 0): workgroup L runs on XCD L % 8, which takes a contiguous eighth of the
    // tiles, each tile's grid rows on consecutive workgroups of that XCD. The tile's x rows then
    // come from the XCD's L2 after the first read, and the tiles of one segment (one adapter's
    // A rows) stay on one or two XCDs.
    int tx = bx, by = by_in;
    if (p.xcd_rows > 0) {
      const int L = bx;
      const int tpx = (gdx / 8) / p.xcd_rows;  // tiles per XCD
      tx = (L % 8) * tpx + (L / 8) / p.xcd_rows;
      by = (L / 8) % p.xcd_rows;
    }
    const Tile tile = shrink_tile<NT>(p, BM, tx, s_tile, s_scan);
    if (tile.g < 0) return;
    f32x4_t sums[NOUT];
    shrink_piece<DT, MT, CB, NW, D, AL, KFULL>(p, tile, by, 0, int(nsteps), s_red, sums);
    store(tile, by, sums, nullptr);
    return;
  }

  const int64_t units = int64_t(p.sk_tiles) * nsteps;
  int64_t u = int64_t(bx) * p.sk_q;
  const int64_t uend = min(u + int64_t(p.sk_q), units);
  while (u < uend) {
    const int t = int(u / nsteps);
    const int k0 = int(u - int64_t(t) * nsteps);
    const int k1 = int(min(nsteps, int64_t(k0) + (uend - u)));
    const Tile tile = shrink_tile<NT>(p, BM, t, s_tile, s_scan);
    if (tile.g < 0) break;  // past the last tile (uniform over the workgroup)
    const int j = bx - int((int64_t(t) * nsteps) / p.sk_q);
    float* slot = p.part + (int64_t(j) * p.T + tile.m0) * (p.S * p.R);
    {  // (a rank-0 tile stores nothing: every column is at or past its rank)
      f32x4_t sums[NOUT];
      shrink_piece<DT, MT, CB, NW, D, AL, KFULL>(p, tile, by_in, k0, k1, s_red, sums);
      store(tile, by_in, sums, slot);
    }
    if (p.counters != nullptr)
      sk_finish<DT, NT, 1, KEEP>(p, tile, t, j, sk_pieces(t, nsteps, p.sk_q), CB, by_in, gdy,
                                &sm.last);
    u += k1 - k0;
    __syncthreads();  // every wave has read the shared tile record before the next search
  }
}

template <int DT, int MT, int CB, int NW, int D, bool AL, bool KFULL>
__global__ __launch_bounds__(NW * 64) void shrink_kernel(ShrinkArgs p) {
  __shared__ ShrinkSmem<MT, CB, NW> sm;
  shrink_wg<DT, MT, CB, NW, D, AL, KFULL, false>(p, int(blockIdx.x), int(blockIdx.y),
                                                 int(gridDim.x), int(gridDim.y), sm);
}

// Adds the stream-K pieces of tile blockIdx.x in workgroup order, rounds once and writes h,
// with exact zeros in the rank padding. Workgroup y covers elements [256 y, 256 y + 256) of the
// tile's [mlen][S*R] block, one per thread; each thread issues its plane loads eight at a time
// before adding them in order.
template <int DT>
__global__ __launch_bounds__(256) void shrink_sk_reduce_kernel(ShrinkArgs p, int BM) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  __shared__ Tile s_tile;
  __shared__ int s_scan[4];
  const int t = int(blockIdx.x);
  const Tile tile = shrink_tile<256>(p, BM, t, &s_tile, s_scan);
  const int SR = p.S * p.R;
  const int e = int(blockIdx.y) * 256 + int(threadIdx.x);
  if (tile.g < 0 || e >= tile.mlen * SR) return;
  const int64_t nsteps = (p.K + p.sk_unit - 1) / p.sk_unit;
  const int wfirst = int((int64_t(t) * nsteps) / p.sk_q);
  const int wlast = int((int64_t(t + 1) * nsteps - 1) / p.sk_q);
  const int np = wlast - wfirst + 1;
  const int m = e / SR, c = e - (e / SR) * SR;
  const int cr = c - (c / p.R) * p.R;
  S v = S(0);
  if (cr < tile.r) {
    const float* src = p.part + int64_t(tile.m0) * SR + e;
    const int64_t plane = int64_t(p.T) * SR;
    float acc = 0.f;
    for (int j0 = 0; j0 < np; j0 += 8) {
      float b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = (j0 + i < np) ? src[(j0 + i) * plane] : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (j0 + i < np) acc = (j0 + i == 0) ? b[i] : acc + b[i];
    }
    v = Tr::from_f32(acc);
  }
  reinterpret_cast<S*>(p.h)[int64_t(tile.m0 + m) * p.ldh + c] = v;
}

// ------------------------------------------------------------------------------------ expand

// One wave computes a 16-token x 64-column chunk as D[token][col] = sum_j h[token][s*R+j] *
// B[a][col][j]: h rows are the MFMA A operand (constant over the chunks), B rows the B operand.
// MFMA column block q, column index c maps to output column cbase + 4c + q, so lane (g, c) holds
// the 4 consecutive columns cbase + 4c .. +3 of tokens 4g .. 4g+3, and one 8-byte access per token
// covers 128 contiguous bytes of 4 rows per instruction. y and B of a chunk are fetched together
// into a D-deep ring, so data are consumed in the order they were requested.
//
// HFn (the single-launch shrink + expand): h is not ready when the wave starts. The wave primes
// its ring with the first chunks' y and B, then calls hfn(frag) -- with every wave of the
// workgroup, as it holds barriers -- which waits for the tile's shrink and returns the wave's h
// fragments; the y and B loads overlap the shrink.
template <int DT, int NW, int JS, int D, bool ALB, bool ALY, typename HFn = std::nullptr_t>
__device__ __forceinline__ void expand_body(const ExpandArgs& p, const Tile& tile, int s, int nb0,
                                            int nblen, int w, HFn hfn = nullptr) {
  constexpr bool PAIR = !std::is_same_v<HFn, std::nullptr_t>;
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  constexpr int KSTEP = Tr::kStep;
  constexpr int EPF = Tr::kPerFrag;
  constexpr int NY = 4 * int(sizeof(S)) / 8;  // 8-byte pieces per lane and token (4 elements)

  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int a = tile.a, r = tile.r;
  const float sigma = tile.sigma;
  const int nend = nb0 + nblen;
  const int nchunks = (nblen + 63) >> 6;
  const int nci = w < nchunks ? (nchunks - w + NW - 1) / NW : 0;  // this wave's chunks

  const S* __restrict__ hbuf = reinterpret_cast<const S*>(p.h);
  const S* __restrict__ wb = reinterpret_cast<const S*>(p.w_b);
  S* __restrict__ y = reinterpret_cast<S*>(p.y);

  // A operand: h row of token c of the tile (constant over the chunks), read over the padded
  // rank; the adapter's rank masks it once the first chunks are in flight
  Frag<S, ALB> hf[JS];
  uint4 hv[JS];
  const S* hrow = hbuf + int64_t(tile.m0 + (c < tile.mlen ? c : 0)) * p.ldh + s * p.R;
  if constexpr (!PAIR) {
#pragma unroll
    for (int js = 0; js < JS; ++js) {
      const int j = js * KSTEP + g * EPF;
      hf[js].fetch(hrow + j, p.R - j, hrow);
    }
  }
  // output rows of tokens 4g .. 4g+3
  S* yrow[4];
  bool tok_ok[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    tok_ok[v] = m < tile.mlen;
    const int pos = tile.m0 + (tok_ok[v] ? m : 0);
    yrow[v] = y + int64_t(p.permutation != nullptr ? p.permutation[pos] : pos) * p.ldy;
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
        br[d][js][q].fetch(brow + j, in ? p.R - j : 0, brow);
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
  auto do_chunk = [&](auto slot, int i, auto refill) {
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
    if constexpr (decltype(refill)::value) {
      __builtin_amdgcn_sched_barrier(0);
      fetch(slot, i + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Ring slots are issued strictly in order (waits count outstanding loads), and full groups of
  // D chunks run without guards so every path into a wait has the same loads outstanding; the
  // last partial group consumes what the ring holds and fetches nothing.
  [&]<int... dd>(std::integer_sequence<int, dd...>) {
    ((fetch(std::integral_constant<int, dd>{}, dd), __builtin_amdgcn_sched_barrier(0)), ...);
  }(std::make_integer_sequence<int, D>{});
  if (r <= 0) return;  // a rank-0 adapter leaves y untouched
  if constexpr (PAIR) {
    static_assert(ALB, "the single-launch form takes h as aligned 16-byte fragments");
    uint4 fr[JS];
    hfn(fr);
#pragma unroll
    for (int js = 0; js < JS; ++js) hf[js].a = fr[js];
  }
#pragma unroll
  for (int js = 0; js < JS; ++js) hv[js] = hf[js].masked(r - (js * KSTEP + g * EPF));
  const int nfull = nci / D;
  for (int gi = 0; gi < nfull; ++gi) {
    [&]<int... dd>(std::integer_sequence<int, dd...>) {
      (do_chunk(std::integral_constant<int, dd>{}, gi * D + dd, std::true_type{}), ...);
    }(std::make_integer_sequence<int, D>{});
  }
  const int rem = nci - nfull * D;
  [&]<int... dd>(std::integer_sequence<int, dd...>) {
    auto one = [&](auto ddc) {
      constexpr int d = decltype(ddc)::value;
      if (d < rem) do_chunk(ddc, nfull * D + d, std::false_type{});
    };
    (one(std::integral_constant<int, dd>{}), ...);
  }(std::make_integer_sequence<int, D>{});
}

// Wide form of the expand body for 16-bit types with 16-byte aligned y rows: a chunk is 128
// columns and lane (c, g) owns the 8 adjacent columns 8c .. 8c+7 of tokens 4g .. 4g+3 (MFMA
// column block q is output column 8c + q), so each token's y piece is one 16-byte load and one
// 16-byte store, half the memory instructions of the 8-byte form for the same bytes. Tail
// chunks load the aligned 16-byte granule holding their first valid column and store element by
// element.
template <int DT, int NW, int JS, int D, bool ALB>
__device__ __forceinline__ void expand_body_wide(const ExpandArgs& p, const Tile& tile, int s,
                                                 int nb0, int nblen) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  static_assert(sizeof(S) == 2, "16-bit types");
  constexpr int KSTEP = Tr::kStep;
  constexpr int EPF = Tr::kPerFrag;
  constexpr int CW = 128;  // columns per chunk

  const int lane = threadIdx.x & 63, w = wave_id();
  const int c = lane & 15, g = lane >> 4;
  const int a = tile.a, r = tile.r;
  const float sigma = tile.sigma;
  const int nend = nb0 + nblen;
  const int nchunks = (nblen + CW - 1) / CW;
  const int nci = w < nchunks ? (nchunks - w + NW - 1) / NW : 0;  // this wave's chunks

  const S* __restrict__ hbuf = reinterpret_cast<const S*>(p.h);
  const S* __restrict__ wb = reinterpret_cast<const S*>(p.w_b);
  S* __restrict__ y = reinterpret_cast<S*>(p.y);

  Frag<S, ALB> hf[JS];  // over the padded rank; masked by the rank after the ring prologue
  uint4 hv[JS];
  {
    const bool ok = c < tile.mlen;
    const S* hrow = hbuf + int64_t(tile.m0 + (ok ? c : 0)) * p.ldh + s * p.R;
#pragma unroll
    for (int js = 0; js < JS; ++js) {
      const int j = js * KSTEP + g * EPF;
      hf[js].fetch(hrow + j, p.R - j, hrow);
    }
  }
  S* yrow[4];
  bool tok_ok[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    tok_ok[v] = m < tile.mlen;
    const int pos = tile.m0 + (tok_ok[v] ? m : 0);
    yrow[v] = y + int64_t(p.permutation != nullptr ? p.permutation[pos] : pos) * p.ldy;
  }
  const S* bblk = wb + int64_t(a) * p.N * p.ldb;

  Frag<S, true> yr[D][4];
  Frag<S, ALB> br[D][JS][8];
  auto fetch = [&](auto slot, int i) {
    constexpr int d = decltype(slot)::value;
    const int cbase = nb0 + (w + i * NW) * CW;
    const bool in = i < nci;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int col = cbase + 8 * c + q;
      const S* brow = bblk + int64_t((in && col < nend) ? col : nb0) * p.ldb;
#pragma unroll
      for (int js = 0; js < JS; ++js) {
        const int j = js * KSTEP + g * EPF;
        br[d][js][q].fetch(brow + j, in ? p.R - j : 0, brow);
      }
    }
    const int c0 = cbase + 8 * c;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int valid = (in && tok_ok[v]) ? nend - c0 : 0;
      yr[d][v].fetch(yrow[v] + c0, valid, yrow[v] + nb0);
    }
  };
  auto do_chunk = [&](auto slot, int i, auto refill) {
    constexpr int d = decltype(slot)::value;
    f32x4_t acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int js = 0; js < JS; ++js) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        acc[q] = mma_step<DT>(hv[js], br[d][js][q].masked(r - (js * KSTEP + g * EPF)), acc[q]);
    }
    const int c0 = nb0 + (w + i * NW) * CW + 8 * c;
    const int ncols = min(8, nend - c0);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      union {
        uint4 u;
        S e[8];
      } o;
      o.u = yr[d][v].raw();
#pragma unroll
      for (int q = 0; q < 8; ++q)
        o.e[q] = Tr::from_f32(__builtin_fmaf(sigma, acc[q][v], Tr::to_f32(o.e[q])));
      if (tok_ok[v] && ncols > 0) {
        S* dst = yrow[v] + c0;
        if (ncols == 8) {
          *reinterpret_cast<uint4*>(dst) = o.u;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (q < ncols) dst[q] = o.e[q];
        }
      }
    }
    if constexpr (decltype(refill)::value) {
      __builtin_amdgcn_sched_barrier(0);
      fetch(slot, i + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  [&]<int... dd>(std::integer_sequence<int, dd...>) {
    ((fetch(std::integral_constant<int, dd>{}, dd), __builtin_amdgcn_sched_barrier(0)), ...);
  }(std::make_integer_sequence<int, D>{});
  if (r <= 0) return;  // a rank-0 adapter leaves y untouched
#pragma unroll
  for (int js = 0; js < JS; ++js) hv[js] = hf[js].masked(r - (js * KSTEP + g * EPF));
  const int nfull = nci / D;
  for (int gi = 0; gi < nfull; ++gi) {
    [&]<int... dd>(std::integer_sequence<int, dd...>) {
      (do_chunk(std::integral_constant<int, dd>{}, gi * D + dd, std::true_type{}), ...);
    }(std::make_integer_sequence<int, D>{});
  }
  const int rem = nci - nfull * D;
  [&]<int... dd>(std::integer_sequence<int, dd...>) {
    auto one = [&](auto ddc) {
      constexpr int d = decltype(ddc)::value;
      if (d < rem) do_chunk(ddc, nfull * D + d, std::false_type{});
    };
    (one(std::integral_constant<int, dd>{}), ...);
  }(std::make_integer_sequence<int, D>{});
}

// 16-bit types, padded rank <= 16: the 16x16x16 MFMA covers the rank exactly, so h and B
// fragments are 8 bytes (4 ranks) per lane and every lane's B load is useful (the 16x16x32 form
// spends half of each B fragment on rank padding).
__device__ __forceinline__ uint2 mask4(uint2 v, int valid) {
  if (valid >= 4) return v;
  if (valid <= 0) return make_uint2(0u, 0u);
  if (valid == 1) return make_uint2(v.x & 0xffffu, 0u);
  if (valid == 2) return make_uint2(v.x, 0u);
  return make_uint2(v.x, v.y & 0xffffu);
}

template <int DT>
__device__ __forceinline__ f32x4_t mma_k16(uint2 a, uint2 b, f32x4_t acc);

template <>
__device__ __forceinline__ f32x4_t mma_k16<DT_BF16>(uint2 a, uint2 b, f32x4_t acc) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b),
                                                   acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4_t mma_k16<DT_F16>(uint2 a, uint2 b, f32x4_t acc) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, a), __builtin_bit_cast(h4, b),
                                               acc, 0, 0, 0);
}

// The wide body (128-column chunks, 16-byte y pieces) with the 16x16x16 MFMA for ranks <= 16.
// y moves with non-temporal loads and stores: each element is read and written exactly once.
template <int DT, int NW, int D, bool ALB>
__device__ __forceinline__ void expand_body_wide16(const ExpandArgs& p, const Tile& tile, int s,
                                                   int nb0, int nblen) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  static_assert(sizeof(S) == 2, "16-bit types");
  constexpr int CW = 128;

  const int lane = threadIdx.x & 63, w = wave_id();
  const int c = lane & 15, g = lane >> 4;
  const int a = tile.a, r = tile.r;
  const float sigma = tile.sigma;
  const int nend = nb0 + nblen;
  const int nchunks = (nblen + CW - 1) / CW;
  const int nci = w < nchunks ? (nchunks - w + NW - 1) / NW : 0;
  int jv = 0;  // valid ranks of this lane's 4 (set once the first loads are in flight)

  const S* __restrict__ hbuf = reinterpret_cast<const S*>(p.h);
  const S* __restrict__ wb = reinterpret_cast<const S*>(p.w_b);
  S* __restrict__ y = reinterpret_cast<S*>(p.y);

  Frag8<S, ALB> hf;  // over the padded rank; masked by the rank after the ring prologue
  uint2 hv;
  {
    const bool ok = c < tile.mlen;
    const S* hrow = hbuf + int64_t(tile.m0 + (ok ? c : 0)) * p.ldh + s * p.R;
    hf.fetch(hrow + 4 * g, p.R - 4 * g, hrow);
  }
  S* yrow[4];
  bool tok_ok[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    tok_ok[v] = m < tile.mlen;
    const int pos = tile.m0 + (tok_ok[v] ? m : 0);
    yrow[v] = y + int64_t(p.permutation != nullptr ? p.permutation[pos] : pos) * p.ldy;
  }
  const S* bblk = wb + int64_t(a) * p.N * p.ldb;

  uint4 yr[D][4];
  Frag8<S, ALB> br[D][8];
  auto fetch = [&](auto slot, int i) {
    constexpr int d = decltype(slot)::value;
    const int cbase = nb0 + (w + i * NW) * CW;
    const bool in = i < nci;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int col = cbase + 8 * c + q;
      const S* brow = bblk + int64_t((in && col < nend) ? col : nb0) * p.ldb;
      br[d][q].fetch(brow + 4 * g, in ? p.R - 4 * g : 0, brow);
    }
    const int c0 = cbase + 8 * c;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int valid = (in && tok_ok[v]) ? nend - c0 : 0;
      yr[d][v] = gload16_nt(valid > 0 ? yrow[v] + c0 : yrow[v] + nb0);
    }
  };
  auto do_chunk = [&](auto slot, int i, auto refill) {
    constexpr int d = decltype(slot)::value;
    f32x4_t acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      acc[q] = mma_k16<DT>(hv, mask4(br[d][q].raw(), jv), f32x4_t{0.f, 0.f, 0.f, 0.f});
    const int c0 = nb0 + (w + i * NW) * CW + 8 * c;
    const int ncols = min(8, nend - c0);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      union {
        uint4 u;
        S e[8];
      } o;
      o.u = yr[d][v];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        o.e[q] = Tr::from_f32(__builtin_fmaf(sigma, acc[q][v], Tr::to_f32(o.e[q])));
      if (tok_ok[v] && ncols > 0) {
        S* dst = yrow[v] + c0;
        if (ncols == 8) {
          gstore16_nt(dst, o.u);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (q < ncols) dst[q] = o.e[q];
        }
      }
    }
    if constexpr (decltype(refill)::value) {
      __builtin_amdgcn_sched_barrier(0);
      fetch(slot, i + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  [&]<int... dd>(std::integer_sequence<int, dd...>) {
    ((fetch(std::integral_constant<int, dd>{}, dd), __builtin_amdgcn_sched_barrier(0)), ...);
  }(std::make_integer_sequence<int, D>{});
  if (r <= 0) return;  // a rank-0 adapter leaves y untouched
  jv = r - 4 * g;
  hv = mask4(hf.raw(), jv);
  const int nfull = nci / D;
  for (int gi = 0; gi < nfull; ++gi) {
    [&]<int... dd>(std::integer_sequence<int, dd...>) {
      (do_chunk(std::integral_constant<int, dd>{}, gi * D + dd, std::true_type{}), ...);
    }(std::make_integer_sequence<int, D>{});
  }
  const int rem = nci - nfull * D;
  [&]<int... dd>(std::integer_sequence<int, dd...>) {
    auto one = [&](auto ddc) {
      constexpr int d = decltype(ddc)::value;
      if (d < rem) do_chunk(ddc, nfull * D + d, std::false_type{});
    };
    (one(std::integral_constant<int, dd>{}), ...);
  }(std::make_integer_sequence<int, D>{});
}

template <int DT, int NW, int JS, int D, bool ALB, bool ALY, bool WIDE>
__global__ __launch_bounds__(NW * 64) void expand_kernel(ExpandArgs p) {
  constexpr int NT = NW * 64;
  constexpr int BM = 16;

  __shared__ Tile s_tile;
  __shared__ int s_scan[NW];

  // The slice bounds, the tile search and then the rank: each load is issued as early as its
  // address is known, so the operand loads wait for one round trip less (a rank-0 adapter is
  // skipped inside the body, after its first loads, and leaves y untouched).
  const SliceLane sl = slice_lanes(p.slice_offsets, p.S);
  get_tile<NT, false>(p.seg_indptr, p.weight_indices, p.lora_ranks, p.scalings, p.G, BM, p.tiles,
                      p.tile_count, int(blockIdx.x), &s_tile, s_scan);
  Tile tile = s_tile;
  if (tile.g < 0) return;
  tile_rank(p.lora_ranks, p.scalings, &tile);
  int s, nb0, nblen;
  if (!find_nblock_lanes(sl, p.S, p.BN, int(blockIdx.y), &s, &nb0, &nblen)) return;
  if constexpr (WIDE && ALY && DT != DT_F32) {
    // 16-byte pieces when the block starts on a 16-byte boundary (rows are 16-byte aligned)
    if ((nb0 * int(sizeof(typename Traits<DT>::store_t))) % 16 == 0) {
      if constexpr (JS == 1) {
        if (p.R <= 16) {
          expand_body_wide16<DT, NW, D, ALB>(p, tile, s, nb0, nblen);
          return;
        }
      }
      expand_body_wide<DT, NW, JS, D, ALB>(p, tile, s, nb0, nblen);
      return;
    }
  }
  if constexpr (ALY) {
    // whole 8-byte pieces only when the block starts on an 8-byte boundary
    if ((nb0 * int(sizeof(typename Traits<DT>::store_t))) % 8 != 0) {
      expand_body<DT, NW, JS, D, ALB, false>(p, tile, s, nb0, nblen, wave_id());
      return;
    }
  }
  expand_body<DT, NW, JS, D, ALB, ALY>(p, tile, s, nb0, nblen, wave_id());
}

// Expand for slices of rank exactly 16 at large token counts. A workgroup owns up to 64 tokens of
// one segment (16 per wave) and its four waves walk the same 128-column chunks. Each chunk's B
// rows (128 x 16 values, 4 KB) are loaded once for the workgroup, one 16-byte piece per thread,
// and written to LDS in MFMA fragment order (q-th 16x16x16 product, lane), so each wave reads its
// eight B fragments with linear 8-byte LDS reads: one global B load per thread and chunk instead
// of eight per lane. Ranks at or past the adapter's rank are zeroed as the pieces go to LDS. Two
// LDS buffers and one barrier per chunk (chunk i+1 is written while chunk i is read). Lane
// (c, g) of a wave owns columns 8c .. 8c+7 of tokens 4g .. 4g+3 of the wave's 16; y moves as
// non-temporal 16-byte pieces through a D-deep ring per wave. Column blocks whose start is not
// 16-byte aligned run the 8-byte form per wave on that wave's 16 tokens.
template <int DT, int D, bool ALB>
__global__ __launch_bounds__(256) void expand_shared_kernel(ExpandArgs p) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  static_assert(sizeof(S) == 2, "16-bit types");
  constexpr int NW = 4, NT = 256, BM = 64, CW = 128;
  constexpr int PQ = 68;  // 8-byte LDS slots per product: 64 lanes + 4 of padding (bank spread)

  __shared__ Tile s_tile;
  __shared__ int s_scan[NW];
  __shared__ __align__(16) uint2 bsh[2][8 * PQ];

  // loads issued as early as their addresses are known (see expand_kernel)
  const SliceLane sl = slice_lanes(p.slice_offsets, p.S);
  get_tile<NT, false>(p.seg_indptr, p.weight_indices, p.lora_ranks, p.scalings, p.G, BM, p.tiles,
                      p.tile_count, int(blockIdx.x), &s_tile, s_scan);
  Tile tile = s_tile;
  if (tile.g < 0) return;
  tile_rank(p.lora_ranks, p.scalings, &tile);
  int s, nb0, nblen;
  if (!find_nblock_lanes(sl, p.S, p.BN, int(blockIdx.y), &s, &nb0, &nblen)) return;
  const int w = wave_id();
  const int mw = tile.mlen - 16 * w;  // tokens of this wave (uniform over the wave; may be <= 0)
  if ((nb0 * int(sizeof(S))) % 16 != 0) {
    Tile sub = tile;
    sub.m0 = tile.m0 + 16 * w;
    sub.mlen = min(16, mw);
    if (sub.mlen > 0) expand_body<DT, 1, 1, 1, ALB, false>(p, sub, s, nb0, nblen, 0);
    return;
  }

  const int t = int(threadIdx.x), lane = t & 63;
  const int c = lane & 15, g = lane >> 4;
  const int r = tile.r;
  const float sigma = tile.sigma;
  const int nend = nb0 + nblen;
  const int nchunks = (nblen + CW - 1) / CW;

  const S* __restrict__ hbuf = reinterpret_cast<const S*>(p.h);
  const S* __restrict__ wb = reinterpret_cast<const S*>(p.w_b);
  S* __restrict__ y = reinterpret_cast<S*>(p.y);

  // A operand: h row of this wave's token c (ranks 4g .. 4g+3 of the padded rank; the rank
  // masks it after the first y loads are in flight)
  Frag8<S, ALB> hf;
  {
    const bool ok = c < mw;
    const S* hrow = hbuf + int64_t(ok ? tile.m0 + 16 * w + c : tile.m0) * p.ldh + s * p.R;
    hf.fetch(hrow + 4 * g, p.R - 4 * g, hrow);
  }
  S* yrow[4];
  bool tok_ok[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    tok_ok[v] = m < mw;
    const int pos = tok_ok[v] ? tile.m0 + 16 * w + m : tile.m0;
    yrow[v] = y + int64_t(p.permutation != nullptr ? p.permutation[pos] : pos) * p.ldy;
  }

  // B loader: thread t moves ranks 8h .. 8h+7 (h = t & 1) of chunk row t >> 1, which feed
  // fragment groups 2h and 2h+1 of product q = row & 7 for lane c = row >> 3.
  const int lrow = t >> 1, lhalf = t & 1;
  const int slot = (lrow & 7) * PQ + 32 * lhalf + (lrow >> 3);
  int lvalid = 0;  // valid ranks of the piece (set once the first loads are in flight)
  const S* bblk = wb + int64_t(tile.a) * p.N * p.ldb + 8 * lhalf;
  auto bload = [&](int i) -> uint4 {
    const int col = nb0 + i * CW + lrow;
    return gload16(bblk + int64_t((i < nchunks && col < nend) ? col : nb0) * p.ldb);
  };
  auto bput = [&](int buf, uint4 v) {
    v = mask_elems<S>(v, lvalid);
    bsh[buf][slot] = make_uint2(v.x, v.y);
    bsh[buf][slot + 16] = make_uint2(v.z, v.w);
  };

  uint4 yr[D][4];
  auto yfetch = [&](auto slotc, int i) {
    constexpr int d = decltype(slotc)::value;
    const int c0 = nb0 + i * CW + 8 * c;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int valid = (i < nchunks && tok_ok[v]) ? nend - c0 : 0;
      yr[d][v] = gload16_nt(valid > 0 ? yrow[v] + c0 : yrow[v] + nb0);
    }
  };
  const bool active = mw > 0;
  uint4 bnext = bload(0);
  if (active) {
    [&]<int... dd>(std::integer_sequence<int, dd...>) {
      (yfetch(std::integral_constant<int, dd>{}, dd), ...);
    }(std::make_integer_sequence<int, D>{});
  }
  __builtin_amdgcn_sched_barrier(0);
  if (r <= 0) return;  // uniform: a rank-0 adapter leaves y untouched
  lvalid = r - 8 * lhalf;
  const uint2 hv = mask4(hf.raw(), r - 4 * g);
  bput(0, bnext);
  bnext = bload(1);
  __syncthreads();

  auto step = [&](auto slotc, int i) {
    constexpr int d = decltype(slotc)::value;
    const int buf = i & 1;
    if (active) {
      f32x4_t acc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        acc[q] = mma_k16<DT>(hv, bsh[buf][q * PQ + lane], f32x4_t{0.f, 0.f, 0.f, 0.f});
      const int c0 = nb0 + i * CW + 8 * c;
      const int ncols = min(8, nend - c0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        union {
          uint4 u;
          S e[8];
        } o;
        o.u = yr[d][v];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          o.e[q] = Tr::from_f32(__builtin_fmaf(sigma, acc[q][v], Tr::to_f32(o.e[q])));
        if (tok_ok[v] && ncols > 0) {
          S* dst = yrow[v] + c0;
          if (ncols == 8) {
            gstore16_nt(dst, o.u);
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (q < ncols) dst[q] = o.e[q];
          }
        }
      }
      yfetch(slotc, i + D);
    }
    bput(buf ^ 1, bnext);  // chunk i+1 (never read when i+1 == nchunks)
    bnext = bload(i + 2);
    __syncthreads();
  };
  const int ngroups = (nchunks + D - 1) / D;
  for (int gi = 0; gi < ngroups; ++gi) {
    [&]<int... dd>(std::integer_sequence<int, dd...>) {
      auto one = [&](auto ddc) {
        constexpr int d = decltype(ddc)::value;
        if (gi * D + d < nchunks) step(ddc, gi * D + d);  // uniform over the workgroup
      };
      (one(std::integral_constant<int, dd>{}), ...);
    }(std::make_integer_sequence<int, D>{});
  }
}

// ------------------------------------------------------------- single-launch shrink + expand

// Shrink and expand of one call in one launch, for decode sizes (tiles of 16 sorted positions in
// both). Workgroups [0, shrink_wgs) are the register-ring shrink (shape 1x1x8x2: one 16-token
// group, one 16-column block, 8 waves, 2-deep ring) with its (tile, K step) work split into
// pieces, each stored as fp32 partial sums and counted in on the arrival counter of its (tile,
// column block); the last piece of each writes h as in lora_shrink and leaves the counter at the
// piece count. The remaining workgroups are the 64-column expand (8 waves, 2-deep ring) over
// (tile, column block): each primes its ring with y and B, waits until every piece of its
// slice's column blocks has arrived, and adds the partial sums itself -- one element of the
// tile's [16][R] h block per thread, planes added in plane order and rounded once, exactly as
// the last piece adds them for h -- into LDS, where each wave takes its MFMA fragments. So the
// expand does not wait for h to be written and read back, and every output is computed with the
// same operands and instructions as in the separate calls (the column blocking does not enter
// the arithmetic). The host sizes the column blocks so that the whole grid is resident at once.
// A tile's expand workgroups count themselves out on its done counter; the last one waits for
// every column block's pieces (also those of slices no expand workgroup reads) and clears the
// tile's counters, so the workspace is ready for the next call. A rank-0 tile stores no pieces
// and its expand workgroups neither wait nor count.
template <int DT, bool KFULL, bool ALY>
__global__ __launch_bounds__(512) void pair_kernel(ShrinkArgs ps, ExpandArgs pe, PairArgs pp) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  constexpr int KSTEP = Tr::kStep;
  constexpr int EPF = Tr::kPerFrag;
  __shared__ ShrinkSmem<1, 1, 8> sm;
  __shared__ __attribute__((aligned(16))) S s_h[16 * KSTEP];  // the tile's h block of one slice
  const int id = int(blockIdx.x);
  if (id < pp.shrink_wgs) {
    shrink_wg<DT, 1, 1, 8, 2, true, KFULL, true>(ps, id % pp.sgx, id / pp.sgx, pp.sgx, pp.sgy, sm);
    return;
  }
  const int e = id - pp.shrink_wgs;
  const int tx = e % pp.egx, by = e / pp.egx;
  const SliceLane sl = slice_lanes(pe.slice_offsets, pe.S);
  get_tile<512, false>(pe.seg_indptr, pe.weight_indices, pe.lora_ranks, pe.scalings, pe.G, 16,
                       pe.tiles, pe.tile_count, tx, &sm.tile, sm.scan);
  Tile tile = sm.tile;
  if (tile.g < 0) return;
  tile_rank(pe.lora_ranks, pe.scalings, &tile);
  if (tile.r <= 0) return;
  const int R = pe.R, NB = (R + 15) >> 4, gy = pp.sgy;
  const int64_t nsteps = (ps.K + KSTEP - 1) / KSTEP;
  const int np = sk_pieces(tx, nsteps, ps.sk_q);
  // counter of column block b of this tile
  auto ctr = [&](int b) { return ps.counters + ((int64_t(tx) * gy + b) << ps.ctr_shift); };
  int s, nb0, nblen;
  const bool has = find_nblock_lanes(sl, pe.S, pe.BN, by, &s, &nb0, &nblen);
  const int w = wave_id();
  if (has) {
    // h fragments of slice s: wait for the pieces of the slice's column blocks, add them
    auto hfn = [&](uint4 (&fr)[1]) {
      if (w == 0)
        for (int b = 0; b < NB; ++b) wait_count(ctr(s * NB + b), np, pp.err);
      __syncthreads();
      const int el = int(threadIdx.x);
      if (el < 16 * R) {
        const int m = el / R, c = el - (el / R) * R;
        S v = S(0);
        if (m < tile.mlen && c < tile.r) {
          const int64_t plane = int64_t(ps.T) * (ps.S * ps.R);
          const float* src = ps.part + int64_t(tile.m0 + m) * (ps.S * ps.R) + s * R + c;
          float acc = 0.f;
          for (int q0 = 0; q0 < np; q0 += 8) {
            float bq[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) bq[i] = (q0 + i < np) ? part_load(src + (q0 + i) * plane) : 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
              if (q0 + i < np) acc = (q0 + i == 0) ? bq[i] : acc + bq[i];
          }
          v = Tr::from_f32(acc);
        }
        s_h[m * R + c] = v;
      }
      __syncthreads();
      const int lane = threadIdx.x & 63, cl = lane & 15, g = lane >> 4;
      const int j = g * EPF;  // rank offset of this lane's fragment (JS = 1)
      fr[0] = j < R ? *reinterpret_cast<const uint4*>(s_h + cl * R + j) : make_uint4(0, 0, 0, 0);
    };
    // whole 8-byte y pieces only when the block starts on an 8-byte boundary
    if (ALY && (nb0 * int(sizeof(S))) % 8 == 0)
      expand_body<DT, 8, 1, 2, true, ALY>(pe, tile, s, nb0, nblen, w, hfn);
    else
      expand_body<DT, 8, 1, 2, true, false>(pe, tile, s, nb0, nblen, w, hfn);
  }
  __syncthreads();  // every wave of this workgroup is past its wait
  if (threadIdx.x == 0) {
    int* const done = pp.done + tx;
    const int before = __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before == pp.egy - 1) {  // the tile's last expand workgroup: no wave waits on it any more
      for (int b = 0; b < gy; ++b) {
        wait_count(ctr(b), np, pp.err);  // every piece has counted in: no increment follows
        __hip_atomic_store(ctr(b), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __hip_atomic_store(done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------------------------ launchers

// Kernel shapes. Shrink: (token groups of 16 per tile, 16-column blocks per workgroup, waves,
// ring depth of the streamed A and x fragments). Expand: (waves, ring depth of the
// streamed y chunks, 128-column chunks with 16-byte y pieces); expand tiles are 16 tokens. fp32 (small correctness workloads) has one
// shape of each.
#define LMX_SHRINK_VARIANTS(X) \
  X(0, 1, 1, 8, 4)             \
  X(1, 2, 4, 4, 4)             \
  X(2, 1, 1, 8, 2)             \
  X(3, 2, 3, 4, 4)             \
  X(4, 2, 3, 4, 2)
#define LMX_EXPAND_VARIANTS(X) \
  X(0, 4, 3, false)            \
  X(1, 8, 2, false)            \
  X(2, 4, 4, false)            \
  X(3, 4, 2, false)            \
  X(4, 8, 1, false)            \
  X(5, 4, 2, true)             \
  X(6, 4, 1, true)             \
  X(7, 8, 1, true)

template <int DT, int MT, int CB, int NW, int D>
static hipError_t launch_shrink_t(const ShrinkArgs& a, bool aligned, int grid_x, hipStream_t st) {
  const int NB = (a.R + 15) / 16;
  const int nblk = a.S * NB;
  dim3 grid(grid_x, (nblk + CB - 1) / CB);
  if (a.xcd_rows > 0) {  // direct mode, tiles of one tile's grid rows on one XCD (see the kernel)
    if (a.sk_q != 0 || a.xcd_rows != int(grid.y)) return hipErrorInvalidValue;
    grid = dim3(unsigned((grid_x + 7) / 8 * 8 * a.xcd_rows), 1);
  }
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

template <int DT>
hipError_t launch_shrink_sk_reduce_dt(const ShrinkArgs& a, int bm, hipStream_t st) {
  const int gy = int((int64_t(bm) * a.S * a.R + 255) / 256);
  hipLaunchKernelGGL((shrink_sk_reduce_kernel<DT>), dim3(a.sk_tiles, gy), dim3(256), 0, st, a, bm);
  return hipGetLastError();
}

template <int DT, int NW, int JS, int D, bool WIDE>
static void launch_expand_al(const ExpandArgs& a, const ExpandPlan& plan, dim3 grid, hipStream_t st) {
  dim3 block(NW * 64);
  if (plan.aligned_b && plan.aligned_y)
    hipLaunchKernelGGL((expand_kernel<DT, NW, JS, D, true, true, WIDE>), grid, block, 0, st, a);
  else if (plan.aligned_b)
    hipLaunchKernelGGL((expand_kernel<DT, NW, JS, D, true, false, WIDE>), grid, block, 0, st, a);
  else if (plan.aligned_y)
    hipLaunchKernelGGL((expand_kernel<DT, NW, JS, D, false, true, WIDE>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((expand_kernel<DT, NW, JS, D, false, false, WIDE>), grid, block, 0, st, a);
}

template <int DT, int NW, int D, bool WIDE>
static hipError_t launch_expand_t(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st) {
  const int64_t gy = (a.N + a.BN - 1) / a.BN + a.S;
  dim3 grid(plan.grid_x, unsigned(gy));
  constexpr int KS = Traits<DT>::kStep;
  const int js = (a.R + KS - 1) / KS;
  if (js <= 1) launch_expand_al<DT, NW, 1, D, WIDE>(a, plan, grid, st);
  else if (js == 2) launch_expand_al<DT, NW, 2, D, WIDE>(a, plan, grid, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_expand_shared_t(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st) {
  const int64_t gy = (a.N + a.BN - 1) / a.BN + a.S;
  dim3 grid(plan.grid_x, unsigned(gy));
  if (!plan.aligned_b || !plan.aligned_y || a.R != 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL((expand_shared_kernel<DT, D, true>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_pair_dt(const ShrinkArgs& s, const ExpandArgs& e, const PairArgs& pa, bool kfull,
                          bool aligned_y, hipStream_t st) {
  if constexpr (DT == DT_F32) {
    return hipErrorInvalidValue;
  } else {
    if (e.R > Traits<DT>::kStep || pa.shrink_wgs != pa.sgx * pa.sgy) return hipErrorInvalidValue;
    const dim3 grid(unsigned(pa.shrink_wgs + pa.egx * pa.egy));
    if (kfull && aligned_y)
      hipLaunchKernelGGL((pair_kernel<DT, true, true>), grid, dim3(512), 0, st, s, e, pa);
    else if (kfull)
      hipLaunchKernelGGL((pair_kernel<DT, true, false>), grid, dim3(512), 0, st, s, e, pa);
    else if (aligned_y)
      hipLaunchKernelGGL((pair_kernel<DT, false, true>), grid, dim3(512), 0, st, s, e, pa);
    else
      hipLaunchKernelGGL((pair_kernel<DT, false, false>), grid, dim3(512), 0, st, s, e, pa);
    return hipGetLastError();
  }
}

template <int DT>
hipError_t launch_expand_dt(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st) {
  if constexpr (DT == DT_F32) {
    return launch_expand_t<DT, 4, 2, false>(a, plan, st);
  } else {
    if (plan.variant == kExpandSharedD1) return launch_expand_shared_t<DT, 1>(a, plan, st);
    if (plan.variant == kExpandSharedD2) return launch_expand_shared_t<DT, 2>(a, plan, st);
    switch (plan.variant) {
#define X(V, NW, D, WIDE) \
      case V: return launch_expand_t<DT, NW, D, WIDE>(a, plan, st);
      LMX_EXPAND_VARIANTS(X)
#undef X
    }
    return hipErrorInvalidValue;
  }
}

}  // namespace lmx
