// Single-adapter LoRA MLP with fused SwiGLU for gfx950 ("Add optional fast lora path for
// qwen2/qwen3 on npu", What this PR does: the Qwen MLP forward with LoRA on the gate, up and down
// projections and a fused SwiGLU; Compatibility checks: dropout 0, one adapter, no bias).
//
// out = round(hmid W_d^T + s * xa_d B_d^T),   hmid = round(silu(g) * u),
// g = x W_g^T + s * xa_g B_g^T,  u = x W_u^T + s * xa_u B_u^T,  xa_* = round(x A_*^T)
//
// Launches on the caller's stream:
//   1. the scaled LoRA-B operands s*B_g, s*B_u, s*B_d in bf16, zero padded (small; exact when s
//      is a power of two, as alpha / rank usually is);
//   2. LoRA-A products of x for gate and up (the dense mode of the shrink kernel, both slices in
//      one pass over x) -> xa_gu [M][2*rp] = [xa_g | xa_u] (rp = rank rounded up to 32);
//   3. gate/up GEMM over K = H + 2*rp: the last 2*rp reduction columns are [xa_g | xa_u] against
//      [s*B_g | 0] for gate rows and [0 | s*B_u] for up rows, so the LoRA term accumulates with
//      the base product. One workgroup computes 256 rows x 128 output columns of BOTH
//      projections (its B tile holds the 128 gate rows then the 128 up rows), so every lane
//      holds g and u of the same outputs and the epilogue stores hmid = silu(g) * u in bf16;
//   4. LoRA-A product of hmid for down -> xa_d [M][rp];
//   5. down GEMM over K = I + rp -> out.
//
// GEMM main loop: 256x256x32 block stages, 4 waves of 128x128, v_mfma_f32_32x32x16_bf16, both
// operands K-contiguous ([rows][K] row-major, as nn.Linear stores them) loaded straight into
// LDS (global_load_lds_dwordx4) three stages deep, with XOR-swizzled 64-byte rows so 16-byte
// fragment reads are bank-conflict free; fragment reads of the next k slice overlap the MFMAs.
#include "device_common.hpp"
#include "mlp_kernels.hpp"
#include "sgmv_kernels.hpp"

#include <type_traits>
#include <utility>

namespace lmx {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int kBM = 256;  // rows of A per block
constexpr int kBR = 256;  // rows of W per block (B operand)
constexpr int kBK = 32;   // K per stage (64 bytes per row)
constexpr int kStages = 3;  // LDS buffers (more in flight per compute unit measured slower)
constexpr int kStageElems = (kBM + kBR) * kBK;  // elements per stage (32 KiB)

__device__ __forceinline__ f32x16_t mma32(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// bf16 round to nearest even with gfx950's conversion instruction (v_cvt_pk_bf16_f32, paired by
// the compiler). Same values as the integer form of Traits<DT_BF16>::from_f32 for every non-NaN
// input; measured faster in these GEMM epilogues (and slower in the SGMV expand, which keeps the
// integer form).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// LDS tiles hold rows of 64 bytes (4 chunks of 16 bytes) with the chunk index XOR-swizzled by
// (row / 4) % 4, so that the 16 lanes of each 16-byte read phase hit 16 distinct bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

}  // namespace

template <int MODE>
__global__ __launch_bounds__(256) void gemm_lora_kernel(GemmArgs p) {
  constexpr bool SWIGLU = MODE == kGemmSwiglu || MODE == kGemmSwigluSave;
  // One LDS array per pipeline stage.
  __shared__ __attribute__((aligned(1024))) uint16_t stg[kStages][kStageElems];
  auto stage = [&](auto sc) -> uint16_t* {
    constexpr int s = decltype(sc)::value;
    return stg[s];
  };

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int wi = w >> 1, wj = w & 1;  // wave row / column in the 2x2 wave grid
  // Block coordinates. Workgroup i runs on XCD i % 8. When the block grid tiles into 16 x 16
  // super-tiles, the 32 workgroups an XCD runs together form a 4 x 8 sub-grid of one
  // super-tile, so each K slice of an A tile is read by 8 of its CUs and each slice of a W tile
  // by 4 out of the XCD's L2. Otherwise column blocks walk fastest inside groups of 8 row blocks.
  const bool grouped = MODE == kGemmPlain && p.ngroups > 1;  // uniform
  const int nbn = SWIGLU ? (p.N + 127) / 128 : (grouped ? p.gblk[p.ngroups] : (p.N + 255) / 256);
  const int nbm = (p.M + kBM - 1) / kBM;
  int bm, bn;
  if (nbm % 16 == 0 && nbn % 16 == 0) {
    const int id = int(blockIdx.x);
    const int super = id >> 8, xcd = id & 7, slot = (id >> 3) & 31;
    const int nsn = nbn / 16;  // super-tiles per row of super-tiles
    bm = (super / nsn) * 16 + 4 * (xcd >> 1) + (slot & 3);
    bn = (super % nsn) * 16 + 8 * (xcd & 1) + (slot >> 2);
  } else {
    const int group = int(blockIdx.x) / (8 * nbn);
    const int first_m = group * 8;
    const int gsize = min(nbm - first_m, 8);
    const int local = int(blockIdx.x) - group * 8 * nbn;
    bm = first_m + local % gsize;
    bn = local / gsize;
  }
  // column group of this block (constant-index selection keeps the tables out of scratch)
  const uint16_t* gW0 = p.W0;
  const uint16_t* gB2 = p.B2;
  const uint16_t* gA2 = p.A2;
  uint16_t* gC = p.C;
  int64_t gldc = p.ldc;
  int gN = p.N;
  if constexpr (MODE == kGemmPlain) {
    if (grouped) {
      int sel = 0;
#pragma unroll
      for (int g = 1; g < 3; ++g)
        if (g < p.ngroups && bn >= p.gblk[g]) sel = g;
#pragma unroll
      for (int g = 0; g < 3; ++g) {
        if (sel == g) {
          gW0 = p.gW[g]; gB2 = p.gB2[g]; gA2 = p.A2 + p.ga2[g]; gC = p.gC[g]; gldc = p.gldc[g];
          gN = p.gN[g]; bn -= p.gblk[g];
        }
      }
    }
  }
  const int m0 = bm * kBM;
  const int n0 = SWIGLU ? bn * 128 : bn * 256;

  // DMA mapping: wave w fills tile rows [64 w, 64 w + 64) of A and of W, 16 rows per
  // instruction; lane L covers row 16 i + L / 4 and LDS slot L % 4, which holds global chunk
  // swz(row, slot). Stages past K read the LoRA columns (A2, B2).
  const int drow = lane >> 2, dslot = lane & 3;
  const int nk1 = p.K / kBK;
  const int nk = nk1 + p.K2 / kBK;
  // kernel arguments as values (selecting between argument fields per lane would load them
  // through vector memory)
  const uint16_t* const pA = p.A;
  const uint16_t* const pA2 = gA2;
  const uint16_t* const pW0 = gW0;
  const uint16_t* const pW1 = p.W1;
  const uint16_t* const pB2 = gB2;
  const int64_t plda = p.lda, plda2 = p.lda2, pldw = p.ldw, pldb2 = p.ldb2;
  const int pM = p.M, pN = gN;
  // Tiles inside M and N (all of them when M is a multiple of 256 and N of the column tile)
  // address each 16-row load group as a wave-uniform base plus one loop-invariant per-lane byte
  // offset: the lane's row inside the group (drow) and its swizzled chunk, which do not depend
  // on the group (row % 16 == drow and swz(row, c) only reads bits 2..3 of the row).
  const bool full = m0 + kBM <= pM && n0 + (SWIGLU ? 128 : 256) <= pN;  // uniform
  const int swb = swz(drow, dslot) * 16;
  const uint32_t voA = uint32_t(drow * plda * 2 + swb), voW = uint32_t(drow * pldw * 2 + swb);
  const uint32_t voA2 = uint32_t(drow * plda2 * 2 + swb), voB2 = uint32_t(drow * pldb2 * 2 + swb);
  auto issue = [&](auto sc, int kt) {
    uint16_t* sa = stage(sc);
    uint16_t* sb = sa + kBM * kBK;
    const bool lora = kt >= nk1;
    const int koff = (lora ? kt - nk1 : kt) * kBK;
    if (full) {
      const char* abase = reinterpret_cast<const char*>(lora ? pA2 : pA) + int64_t(koff) * 2;
      const int64_t lda = lora ? plda2 : plda;
      const uint32_t voa = lora ? voA2 : voA, vow = lora ? voB2 : voW;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = w * 64 + i * 16;  // first row of the load group in the tile
        dma16_saddr(abase + int64_t(m0 + g) * lda * 2, voa, lds_addr(sa + g * kBK));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = w * 64 + i * 16;
        const char* wrow;
        if (SWIGLU) {
          const int n = n0 + (g & 127);
          const bool up = g >= 128;
          wrow = lora ? reinterpret_cast<const char*>(pB2) + (int64_t(up ? pN + n : n) * pldb2 + koff) * 2
                      : reinterpret_cast<const char*>(up ? pW1 : pW0) + (int64_t(n) * pldw + koff) * 2;
        } else {
          const int n = n0 + g;
          wrow = lora ? reinterpret_cast<const char*>(pB2) + (int64_t(n) * pldb2 + koff) * 2
                      : reinterpret_cast<const char*>(pW0) + (int64_t(n) * pldw + koff) * 2;
        }
        dma16_saddr(wrow, vow, lds_addr(sb + g * kBK));
      }
      return;
    }
    const uint16_t* abase = lora ? pA2 : pA;
    const int64_t lda = lora ? plda2 : plda;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = w * 64 + i * 16 + drow;
      const int kk = koff + swz(row, dslot) * 8;
      dma16(abase + int64_t(min(m0 + row, pM - 1)) * lda + kk,
            lds_addr(sa + (w * 64 + i * 16) * kBK));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = w * 64 + i * 16 + drow;
      const int kk = koff + swz(row, dslot) * 8;
      const uint16_t* wsrc;
      if (SWIGLU) {
        const int n = min(n0 + (row & 127), pN - 1);
        const bool up = row >= 128;  // uniform per instruction: 16 rows never straddle 128
        wsrc = lora ? pB2 + int64_t(up ? pN + n : n) * pldb2 + kk
                    : (up ? pW1 : pW0) + int64_t(n) * pldw + kk;
      } else {
        const int n = min(n0 + row, pN - 1);
        wsrc = lora ? pB2 + int64_t(n) * pldb2 + kk : pW0 + int64_t(n) * pldw + kk;
      }
      dma16(wsrc, lds_addr(sb + (w * 64 + i * 16) * kBK));
    }
  };

  // this wave's B rows inside the block tile, per 32-row column block
  int brow0[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
    brow0[cb] = SWIGLU ? (cb < 2 ? wj * 64 + cb * 32 : 128 + wj * 64 + (cb - 2) * 32)
                       : wj * 128 + cb * 32;
  const int lr = lane & 31, lc = lane >> 5;  // MFMA operand row and chunk-in-slice

  f32x16_t acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x16_t{};

  // Software pipeline. Stage kt lives in buffer kt % kStages. Step kt: read the fragments of its
  // second 16-wide k slice while the MFMAs of the first run; then wait for stage kt+1's loads and
  // meet at the barrier (which also certifies every wave is done reading stage kt), refill stage
  // kt's buffer with stage kt+kStages, read stage kt+1's first slice and run the MFMAs of the second.
  uint4 fa0[4], fb0[4], fa1[4], fb1[4];
  auto read = [&](const uint16_t* sbase, int ks, uint4* fa, uint4* fb) {
    const uint16_t* sa = sbase;
    const uint16_t* sb = sbase + kBM * kBK;
    const int chunk = ks * 2 + lc;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int row = wi * 128 + rb * 32 + lr;
      fa[rb] = *reinterpret_cast<const uint4*>(sa + row * kBK + swz(row, chunk) * 8);
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int row = brow0[cb] + lr;
      fb[cb] = *reinterpret_cast<const uint4*>(sb + row * kBK + swz(row, chunk) * 8);
    }
  };
  auto mma_all = [&](const uint4* fa, const uint4* fb) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mma32(fa[rb], fb[cb], acc[rb][cb]);
  };
  // wait until at most `younger` stages of this wave's loads are outstanding (8 loads per stage).
  // s_waitcnt immediate: vmcnt bits 3:0 (low) and 15:14 (high), expcnt 6:4 and lgkmcnt 11:8
  // left at their maxima.
  auto wait_stages = [&](int younger) {
    static_assert(kStages <= 5, "wait table");
    if (younger >= 4) vm_wait<32>();
    else if (younger == 3) vm_wait<24>();
    else if (younger == 2) vm_wait<16>();
    else if (younger == 1) vm_wait<8>();
    else vm_wait<0>();
  };

  // prologue: all stages in flight, stage 0 published, its first slice read
  [&]<int... ss>(std::integer_sequence<int, ss...>) {
    ((ss < nk ? issue(std::integral_constant<int, ss>{}, ss) : void()), ...);
  }(std::make_integer_sequence<int, kStages>{});
  wait_stages(min(nk - 1, kStages - 1));
  __syncthreads();
  read(stg[0], 0, fa0, fb0);

  auto step = [&](auto sc, int kt) {
    constexpr int s = decltype(sc)::value;
    read(stage(sc), 1, fa1, fb1);
    mma_all(fa0, fb0);
    if (kt + 1 < nk) {
      wait_stages(min(nk - 2 - kt, kStages - 2));
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage kt are done
      __syncthreads();
      if (kt + kStages < nk) issue(sc, kt + kStages);
      read(stage(std::integral_constant<int, (s + 1) % kStages>{}), 0, fa0, fb0);
    }
    mma_all(fa1, fb1);
  };
  for (int kt = 0; kt < nk; kt += kStages) {
    [&]<int... ss>(std::integer_sequence<int, ss...>) {
      ((kt + ss < nk ? step(std::integral_constant<int, ss>{}, kt + ss) : void()), ...);
    }(std::make_integer_sequence<int, kStages>{});
  }

  // epilogue. Output layout of a 32x32 block: lane l holds column l % 32 and rows
  // 8 * (v / 4) + 4 * (l / 32) + v % 4 for registers v = 0..15.
  const int rq = lc * 4;
  const int col_base = SWIGLU ? n0 + wj * 64 : n0 + wj * 128;
  if constexpr (SWIGLU) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int rbase = m0 + wi * 128 + rb * 32;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int n = col_base + cb * 32 + lr;
        if (n >= p.N) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = rbase + 8 * (v >> 2) + rq + (v & 3);
          const float g = acc[rb][cb][v], u = acc[rb][cb + 2][v];
          if (row < p.M) {
            p.C[int64_t(row) * p.ldc + n] = bf16_rne(silu(g) * u);
            if constexpr (MODE == kGemmSwigluSave) {
              p.E[int64_t(row) * p.lde + n] = bf16_rne(g);
              p.V[int64_t(row) * p.lde + n] = bf16_rne(u);
            }
          }
        }
      }
    }
  } else if constexpr (MODE == kGemmSwigluBwd) {
    // acc = dhmid; e, v = saved pre-activations; f = silu(e) = e sigmoid(e),
    // silu'(e) = sigmoid(e) (1 + e (1 - sigmoid(e))). The tile goes through LDS (the stage
    // buffers, free after the main loop) in four passes of 64 rows, so e and v are read and hmid,
    // de, dv written as 16-byte vectors of 8 adjacent columns (E, V, C, D rows 16-byte aligned,
    // N a multiple of 8; the host checks). The register side is expanded at compile time (a
    // runtime index would move acc to scratch).
    constexpr int kPitch = 260;  // floats per LDS row: 256 + 4 against bank conflicts
    float* tl = reinterpret_cast<float*>(&stg[0][0]);
    static_assert(64 * kPitch * 4 <= int(sizeof(stg)), "LDS tile");
    __syncthreads();  // every wave is done reading the last stage
    auto pass = [&](auto pc) {
      constexpr int ps = decltype(pc)::value;
      if (wi == ps / 2) {  // the two waves holding rows [64 ps, 64 ps + 64) of the tile
        [&]<int... ii>(std::integer_sequence<int, ii...>) {
          auto put = [&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int rbl = i / 64, cb = (i / 16) % 4, v = i % 16;  // rbl: row block in pass
            constexpr int rb = 2 * (ps % 2) + rbl;
            const int row = rbl * 32 + 8 * (v >> 2) + rq + (v & 3);
            tl[row * kPitch + wj * 128 + cb * 32 + lr] = acc[rb][cb][v];
          };
          (put(std::integral_constant<int, ii>{}), ...);
        }(std::make_integer_sequence<int, 128>{});
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int q = tid + 256 * k;  // 8-column vector q of the pass: row q / 32
        const int rl = q >> 5, c8 = (q & 31) * 8;
        const int row = m0 + 64 * ps + rl, n = n0 + c8;
        if (row < p.M && n < p.N) {
          const float4 d0 = *reinterpret_cast<const float4*>(tl + rl * kPitch + c8);
          const float4 d1 = *reinterpret_cast<const float4*>(tl + rl * kPitch + c8 + 4);
          const float dh[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
          const uint4 ev = *reinterpret_cast<const uint4*>(p.E + int64_t(row) * p.lde + n);
          const uint4 vv = *reinterpret_cast<const uint4*>(p.V + int64_t(row) * p.lde + n);
          const uint32_t ew[4] = {ev.x, ev.y, ev.z, ev.w}, vw[4] = {vv.x, vv.y, vv.z, vv.w};
          typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
          uint32_t hw[4], dw[4], uw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float h2[2], d2[2], u2[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const float z = __uint_as_float(t ? (ew[j] & 0xffff0000u) : (ew[j] << 16));
              const float u = __uint_as_float(t ? (vw[j] & 0xffff0000u) : (vw[j] << 16));
              const float g = dh[2 * j + t];
              const float ex = __expf(-z);
              const float sg = 1.0f / (1.0f + ex);
              const float f = z / (1.0f + ex);
              h2[t] = f * u;
              d2[t] = g * u * (sg * (1.0f + z * (1.0f - sg)));
              u2[t] = g * f;
            }
            // two roundings to bf16 (nearest even) per packed word
            hw[j] = __builtin_bit_cast(uint32_t, bf2_t{static_cast<__bf16>(h2[0]), static_cast<__bf16>(h2[1])});
            dw[j] = __builtin_bit_cast(uint32_t, bf2_t{static_cast<__bf16>(d2[0]), static_cast<__bf16>(d2[1])});
            uw[j] = __builtin_bit_cast(uint32_t, bf2_t{static_cast<__bf16>(u2[0]), static_cast<__bf16>(u2[1])});
          }
          *reinterpret_cast<uint4*>(p.C + int64_t(row) * p.ldc + n) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
          *reinterpret_cast<uint4*>(p.D + int64_t(row) * p.ldd + n) = make_uint4(dw[0], dw[1], dw[2], dw[3]);
          *reinterpret_cast<uint4*>(p.D + int64_t(row) * p.ldd + p.N + n) =
              make_uint4(uw[0], uw[1], uw[2], uw[3]);
        }
      }
      __syncthreads();  // the next pass overwrites the LDS tile
    };
    [&]<int... pp>(std::integer_sequence<int, pp...>) {
      (pass(std::integral_constant<int, pp>{}), ...);
    }(std::make_integer_sequence<int, 4>{});
  } else {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int rbase = m0 + wi * 128 + rb * 32;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int n = col_base + cb * 32 + lr;
        if (n >= gN) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = rbase + 8 * (v >> 2) + rq + (v & 3);
          if (row < p.M) gC[int64_t(row) * gldc + n] = bf16_rne(acc[rb][cb][v]);
        }
      }
    }
  }
}

// The scaled LoRA-B operands of all three projections in one launch: job q writes
// dst_q[row][c] = round(scale * src_q[row][c - col0_q]) for col0_q <= c < col0_q + r and 0
// elsewhere in its [n_q][ld_dst_q] block; the grid covers the three blocks back to back.
__global__ void scale_lora_b_kernel(ScaleJobs jobs, float scale, int r) {
  // (every block has fewer than 2^31 elements: 32-bit index arithmetic)
  int i = int(blockIdx.x) * int(blockDim.x) + int(threadIdx.x);
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const ScaleJob& jb = jobs.job[q];
    const int ld = int(jb.ld_dst);
    const int total = jb.n * ld;
    if (i < total) {
      const int row = i / ld, j = i - row * ld - jb.col0;
      uint16_t v = 0;
      if (j >= 0 && j < r)
        v = bf16_rne(Traits<DT_BF16>::to_f32(jb.src[int64_t(row) * jb.ld_src + j]) * scale);
      jb.dst[i] = v;
      return;
    }
    i -= total;
  }
}

hipError_t launch_scale_lora_b(const ScaleJobs& jobs, float scale, int r, hipStream_t st) {
  int64_t total = 0;
  for (int q = 0; q < 3; ++q) total += int64_t(jobs.job[q].n) * jobs.job[q].ld_dst;
  hipLaunchKernelGGL(scale_lora_b_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, st,
                     jobs, scale, r);
  return hipGetLastError();
}

hipError_t launch_gemm_lora(const GemmArgs& a, int mode, hipStream_t st) {
  const bool swiglu = mode == kGemmSwiglu || mode == kGemmSwigluSave;
  const int nbm = (a.M + kBM - 1) / kBM;
  const int nbn = swiglu ? (a.N + 127) / 128
                         : (mode == kGemmPlain && a.ngroups > 1 ? a.gblk[a.ngroups] : (a.N + 255) / 256);
  dim3 grid(nbm * nbn);
  switch (mode) {
    case kGemmPlain: hipLaunchKernelGGL(gemm_lora_kernel<kGemmPlain>, grid, dim3(256), 0, st, a); break;
    case kGemmSwiglu: hipLaunchKernelGGL(gemm_lora_kernel<kGemmSwiglu>, grid, dim3(256), 0, st, a); break;
    case kGemmSwigluSave:
      hipLaunchKernelGGL(gemm_lora_kernel<kGemmSwigluSave>, grid, dim3(256), 0, st, a);
      break;
    case kGemmSwigluBwd:
      hipLaunchKernelGGL(gemm_lora_kernel<kGemmSwigluBwd>, grid, dim3(256), 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lmx
