#pragma once
// LDS-staged chunked-SGMV shrink for 16-bit types ("Decode LoRA kernels are optimized",
// Summary: gathered-A mainloop, one rank block per output slice).
//
// A workgroup owns a tile of BM = 16 * BMG sorted positions of one segment and NC = 16 * NCB
// rank columns. The reduction runs in stages of 64 indices (128 bytes per row): every stage
// moves the tile's x rows (read through the permutation) and the adapter's A rows straight into
// LDS with direct-to-LDS loads, each instruction covering 8 full 128-byte row chunks, NS stages
// in flight. The chunk index inside a row is XOR-swizzled by the row (on the global side, since
// the load writes LDS lane-linearly), so the MFMA fragment reads (ds_read_b128) are
// bank-conflict free. Each of the 4 waves owns BMG / 4 groups of 16 positions across all NC
// columns: no reduction between waves, and every A chunk loaded is shared by the whole tile.
//
// Rows past the tile and rank columns past the padded rank load a valid row of the same operand
// (their outputs are never stored; rows at or past the adapter's rank are stored as zeros); reduction indices past K load a block of zeros.
// Requires 16-byte aligned x and A rows and K a multiple of 8 (the host checks).
//
// Work split: direct (sk_q == 0, one workgroup per tile over all of K) or shared (the
// (tile, stage) work cut into ranges of sk_q stages per workgroup, partial planes added by the
// tile's last workgroup or by shrink_sk_reduce_kernel), as for the register-ring shrink.
//
// The stage's 1 KiB load instructions are dealt round-robin to the waves with no padding, so
// waves may differ by one instruction; each waits with the immediate for its own count.
#include "sgmv_impl.hpp"  // shrink_tile, the shared reduce kernel

namespace lmx {

static __device__ __align__(16) uint4 g_zero_block[1] = {{0u, 0u, 0u, 0u}};

template <int DT, int BMG, int NCB, int NS, int NW>
__global__ __launch_bounds__(NW * 64) void shrink_lds_kernel(ShrinkArgs p) {
  using Tr = Traits<DT>;
  using S = typename Tr::store_t;
  static_assert(sizeof(S) == 2, "16-bit storage types only");
  constexpr int NT = NW * 64;
  constexpr int BM = 16 * BMG, NC = 16 * NCB;
  constexpr int KB = 64;                    // reduction indices per stage
  constexpr int XI = BM / 8, AI = NC / 8;   // 1 KiB load instructions per stage for x and A
  constexpr int TOT = XI + AI;
  constexpr int PER = (TOT + NW - 1) / NW;  // load instructions of waves w < TOT % NW (or all)
  constexpr int PER_LO = TOT / NW;          // ... of the other waves
  constexpr int ROWS = TOT * 8;             // rows of a stage buffer
  constexpr int GPW = BMG / NW;             // groups of 16 positions per wave
  static_assert(BMG % NW == 0, "row groups must split evenly over the waves");
  static_assert((NS - 2) * PER < 64, "vmcnt range");

  __shared__ __align__(16) S lds[NS][ROWS * KB];
  __shared__ Tile s_tile;
  __shared__ int s_scan[NW];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63, w = wave_id();
  const int li = lane & 15, lg = lane >> 4;
  const int NB = (p.R + 15) >> 4;
  const int nblk = p.S * NB;
  const int K = int(p.K);
  const int64_t nunits = (p.K + KB - 1) / KB;
  const S* __restrict__ x = reinterpret_cast<const S*>(p.x);
  const S* __restrict__ wa = reinterpret_cast<const S*>(p.w_a);
  const void* zero = g_zero_block;

  // this wave's load instructions per stage (uniform: the waits below are immediates)
  const bool hi = (TOT % NW == 0) || w < TOT % NW;

  // One piece: stages [u0, u1) of `tile` for column-block group `by`; the sums go to h
  // (slot == nullptr) or a partial plane.
  auto piece = [&](const Tile& tile, int by, int64_t u0, int64_t u1, float* slot) {
    // DMA sources of this lane: instruction i = w + NW * ii fills stage rows 8 i .. 8 i + 7;
    // this lane writes row rb = 8 i + lane / 8, 16-byte slot lane % 8, which holds chunk
    // (lane % 8) ^ (rb % 8) of the source row. A row past the tile or past the adapter's rank
    // reads a valid row of the same operand instead: its products land in outputs that are
    // never stored.
    const S* src[PER];
    int chunk[PER];
#pragma unroll
    for (int ii = 0; ii < PER; ++ii) {
      const int i = w + NW * ii;
      const int rb = 8 * i + (lane >> 3);
      chunk[ii] = (lane & 7) ^ (rb & 7);
      src[ii] = x;
      if (i < XI) {
        const int m = rb;
        const int pos = tile.m0 + (m < tile.mlen ? m : 0);
        const int tok = p.permutation != nullptr ? p.permutation[pos] : pos;
        src[ii] = x + int64_t(tok) * p.ldx;
      } else if (i < TOT) {
        const int n = rb - BM;
        const int blk = by * NCB + (n >> 4);
        const int s = blk / NB, b = blk - (blk / NB) * NB;
        const int j = 16 * b + (n & 15);
        const bool ok = blk < nblk && j < p.R;
        const int ss = ok ? s : 0;
        src[ii] = wa + (int64_t(tile.a * p.S + ss) * p.R + (ok ? j : 0)) * p.lda;
      }
    }
    // Reduction indices past K read a block of zeros (both operands, so no garbage enters).
    auto issue = [&](int buf, int64_t unit) {
#pragma unroll
      for (int ii = 0; ii < PER; ++ii) {
        if (ii < PER_LO || hi) {
          const int64_t k = unit * KB + 8 * chunk[ii];
          const void* g = k < K ? static_cast<const void*>(src[ii] + k) : zero;
          dma16(g, lds_addr(&lds[buf][(w + NW * ii) * 8 * KB]));
        }
      }
    };
    auto wait_stage = [&]() {  // this wave's loads of the oldest stage in flight have landed
      if (hi) vm_wait<(NS - 2) * PER>();
      else vm_wait<(NS - 2) * PER_LO>();
    };
    f32x4_t acc[GPW][NCB];
#pragma unroll
    for (int g = 0; g < GPW; ++g)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[g][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int buf) {
      const S* L0 = lds[buf];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int c = 4 * kk + lg;
        uint4 av[NCB], xv[GPW];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int row = BM + 16 * cb + li;
          av[cb] = *reinterpret_cast<const uint4*>(L0 + row * KB + ((c ^ (row & 7)) << 3));
        }
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
          const int row = 16 * (w + g * NW) + li;
          xv[g] = *reinterpret_cast<const uint4*>(L0 + row * KB + ((c ^ (row & 7)) << 3));
        }
#pragma unroll
        for (int g = 0; g < GPW; ++g)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) acc[g][cb] = mma_step<DT>(av[cb], xv[g], acc[g][cb]);
      }
    };

    // NS - 1 stages in flight; every stage is issued (past the piece or past K they load data
    // that is never used, or zeros), so every wait has the same count.
    const int n = int(u1 - u0);
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st, u0 + st);
    for (int s = 0; s < n; ++s) {
      wait_stage();     // this wave's loads of stage s have landed
      __syncthreads();  // everyone's have; everyone is done reading stage s - 1
      issue((s + NS - 1) % NS, u0 + s + NS - 1);
      compute(s % NS);
    }
    vm_wait<0>();
    __syncthreads();  // the stage buffers are reused by the next piece

    // epilogue: lane (li, lg) holds D[rank column 4 lg + v][position li] of each 16 x 16 block
#pragma unroll
    for (int g = 0; g < GPW; ++g) {
      const int m = 16 * (w + g * NW) + li;
      if (m >= tile.mlen) continue;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int blk = by * NCB + cb;
        if (blk >= nblk) continue;
        const int s = blk / NB, b = blk - (blk / NB) * NB;
        if (slot != nullptr) {
          float* prow = slot + int64_t(m) * (p.S * p.R) + s * p.R;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int c = 16 * b + 4 * lg + v;
            if (c < tile.r) part_store(prow + c, acc[g][cb][v]);
          }
        } else {
          S* hrow = reinterpret_cast<S*>(p.h) + int64_t(tile.m0 + m) * p.ldh + s * p.R;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int c = 16 * b + 4 * lg + v;
            if (c < p.R) hrow[c] = (c < tile.r) ? Tr::from_f32(acc[g][cb][v]) : S(0);
          }
        }
      }
    }
  };

  if (p.sk_q == 0) {
    // Direct mode; with p.xcd_rows > 0 the grid is one-dimensional and workgroup L (which runs
    // on XCD L % 8) takes tile (L % 8) * tpx + (L / 8) / xcd_rows, grid row (L / 8) % xcd_rows:
    // each XCD a contiguous eighth of the segment-major tiles, so the tiles of one segment
    // (one adapter's A rows) read them from one or two XCDs' L2.
    int tx = int(blockIdx.x), by = int(blockIdx.y);
    if (p.xcd_rows > 0) {
      const int Lw = int(blockIdx.x);
      const int tpx = (int(gridDim.x) / 8) / p.xcd_rows;
      tx = (Lw % 8) * tpx + (Lw / 8) / p.xcd_rows;
      by = (Lw / 8) % p.xcd_rows;
    }
    const Tile tile = shrink_tile<NT>(p, BM, tx, &s_tile, s_scan);
    if (tile.g < 0) return;
    piece(tile, by, 0, nunits, nullptr);
    return;
  }
  const int64_t units = int64_t(p.sk_tiles) * nunits;
  int64_t u = int64_t(blockIdx.x) * p.sk_q;
  const int64_t uend = min(u + p.sk_q, units);
  while (u < uend) {
    const int t = int(u / nunits);
    const int64_t k0 = u - int64_t(t) * nunits;
    const int64_t k1 = min(nunits, k0 + (uend - u));
    const Tile tile = shrink_tile<NT>(p, BM, t, &s_tile, s_scan);
    if (tile.g < 0) break;  // past the last tile (uniform over the workgroup)
    const int j = int(blockIdx.x) - int((int64_t(t) * nunits) / p.sk_q);
    float* slot = p.part + (int64_t(j) * p.T + tile.m0) * (p.S * p.R);
    piece(tile, int(blockIdx.y), k0, k1, slot);  // (a rank-0 tile stores nothing)
    if (p.counters != nullptr)
      sk_finish<DT, NT, 4>(p, tile, t, j, sk_pieces(t, nunits, p.sk_q), NCB, int(blockIdx.y),
                            int(gridDim.y), &s_last);
    u += k1 - k0;
    __syncthreads();  // every wave has read the shared tile record before the next search
  }
}

// Kernel shapes of the LDS-staged shrink: (index, BMG, NCB, NS, NW): 16 BMG positions per tile,
// NCB 16-column blocks per workgroup, NS stages, NW waves.
#define LMX_SHRINK_LDS_VARIANTS(X) \
  X(0, 8, 2, 3, 4)                 \
  X(1, 8, 3, 3, 4)                 \
  X(2, 8, 4, 3, 4)                 \
  X(3, 8, 8, 3, 4)                 \
  X(4, 8, 12, 3, 4)                \
  X(5, 4, 3, 3, 4)                 \
  X(6, 4, 3, 4, 4)                 \
  X(7, 4, 3, 6, 4)                 \
  X(8, 2, 3, 4, 2)                 \
  X(9, 2, 3, 6, 2)                 \
  X(10, 4, 3, 6, 2)                \
  X(11, 3, 3, 4, 3)                \
  X(12, 3, 3, 6, 3)

template <int DT>
hipError_t launch_shrink_lds_dt(const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st) {
  const int NB = (a.R + 15) / 16;
  const int nblk = a.S * NB;
  // direct mode with XCD-contiguous tiles (see the kernel): a one-dimensional grid
  auto grid = [&](int ncb) {
    const int gy = (nblk + ncb - 1) / ncb;
    if (a.xcd_rows > 0) return dim3(unsigned((plan.grid_x + 7) / 8 * 8 * gy), 1);
    return dim3(unsigned(plan.grid_x), unsigned(gy));
  };
  if (a.xcd_rows > 0 && a.sk_q != 0) return hipErrorInvalidValue;
  switch (plan.variant) {
#define X(V, BMG, NCB, NS, NW)                                                               \
    case V:                                                                                  \
      if (a.xcd_rows > 0 && a.xcd_rows != (nblk + NCB - 1) / NCB) return hipErrorInvalidValue; \
      hipLaunchKernelGGL((shrink_lds_kernel<DT, BMG, NCB, NS, NW>), grid(NCB), dim3(NW * 64), 0, \
                         st, a);                                                             \
      return hipGetLastError();
    LMX_SHRINK_LDS_VARIANTS(X)
#undef X
  }
  return hipErrorInvalidValue;
}

}  // namespace lmx
