// C ABI of the library: argument validation, kernel-shape selection and launches.
// Every check here runs on the host before anything is enqueued; nothing reads device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <initializer_list>
#include <cstdint>
#include <mutex>

#include "../../include/lora_mi355x.h"
#include "embedding.hpp"
#include "metadata_check.hpp"
#include "mlp_kernels.hpp"
#include "sgmv_kernels.hpp"

// Device scratch of lora_shrink_noalloc, for callers that cannot allocate: file-scope device
// storage, one copy per GPU the library runs on, held until the process ends. In host code this
// name is only a host-side stand-in: kernels and copies take the device address that
// hipGetSymbolAddress returns for the current device (scratch_address below), never the name.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// The scratch array's device address, taken once per device (with that device current) and kept
// per device; thread-safe.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

constexpr int kInlineMaxSegments = 1024;  // above this the standalone scheduler builds the list
constexpr int kMaxSlices = 64;
constexpr int kMaxRank = 1024;

// Arrival counters of the in-launch stream-K completion: the first kCounterBytes of every
// nonzero shrink workspace, zero before the call and zero after it.
constexpr size_t kCounterBytes = 32768;
constexpr int64_t kMaxCounters = int64_t(kCounterBytes / 4);

// The caller's kernel-shape choices (lora_plan; -1 = the library's own choice). A plain value
// passed down the planning functions: the library keeps no state between calls.
struct Knobs {
  int family = -1, shape = -1, split = -1, finish = -1, eshape = -1, ebn = -1;
};

Knobs knobs_of(const lora_plan* p) {
  Knobs k;
  if (p == nullptr) return k;
  k.family = p->shrink_kernel;
  k.shape = p->shrink_shape;
  k.split = p->shrink_split;
  k.finish = p->shrink_finish;
  k.eshape = p->expand_shape;
  k.ebn = p->expand_block_n;
  return k;
}

// Plan fields outside their documented ranges are argument errors.
bool knobs_valid(const Knobs& k) {
  return k.family >= -1 && k.family <= 2 && k.shape >= -1 &&
         k.shape < std::max(lmx::num_shrink_variants(), lmx::num_shrink_lds_variants()) &&
         !(k.family == 1 && k.shape >= lmx::num_shrink_lds_variants()) &&
         !(k.family == 0 && k.shape >= lmx::num_shrink_variants()) && k.split >= -1 &&
         k.split <= 65535 && k.finish >= -1 && k.finish <= 1 && k.eshape >= -1 &&
         k.eshape < lmx::num_expand_variants() && (k.ebn == -1 || (k.ebn >= 1 && k.ebn <= 65536));
}

bool valid_dtype(int d) { return d == LORA_F32 || d == LORA_BF16 || d == LORA_F16; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int esize(int dtype) { return dtype == LORA_F32 ? 4 : 2; }

// Columns per expand workgroup, in multiples of the 64-column chunks the waves walk: the widest
// blocks (up to 4096 columns) that still give about 400 workgroups. Longer column runs per wave
// measured faster than more workgroups once the chip is covered (rocprofv3 sweeps on MI355X).
// The shared-B kernel takes the narrowest power-of-two multiple of its 128-column unit whose
// grid (tiles x (column blocks + slices)) stays within 1200 workgroups. Power-of-two widths
// divide the usual slice widths evenly (the host cannot read the slice offsets), and blocks
// that end part-way into a slice left some workgroups with far less work than others. Event
// timings after a 512 MiB write on the decode sweep (q/k/v slices 4096/1024/1024): 8192 tokens
// 1024 columns (1188 workgroups) 53.6 us against 55.7 us for 1536 (924) and 54.9 us for 512
// (1980); 6144 tokens 1024 columns 40.8 us against 42.4 for 768 and 46.7 for 512 (1500);
// 4096: 512 columns 31.0 against 31.4 for 768; 2048: 256 columns 19.3 against 20.4 for 384
// and 21.3 for 128 (1836); 1024: 128 columns 13.3 against 14.0 for 256.
int expand_bn(const Knobs& kn, int64_t T, int32_t G, int32_t S, int64_t N, int bm, int waves,
              int chunk, bool shared) {
  const int unit = chunk * waves;
  if (kn.ebn > 0) return int(cdiv(kn.ebn, unit) * unit);
  const int64_t tiles = cdiv(T, bm) + G;
  if (shared) {
    int64_t bn = unit;
    while (bn < 4096 && tiles * (cdiv(N, bn) + S) > 1200) bn *= 2;
    return int(std::min<int64_t>(bn, 4096));
  }
  const int64_t blocks = std::max<int64_t>(1, cdiv(400, tiles));
  int64_t bn = cdiv(cdiv(N, blocks), unit) * unit;
  bn = std::min<int64_t>(std::max<int64_t>(bn, unit), 4096);
  return int(bn);
}

// Kernel shape for a shrink call, from host-known sizes only (event timings and rocprofv3 sweeps
// on MI355X over the decode sweep, prefill and irregular workloads). One compute unit streams
// about 25 GB/s through the register ring, so the time of a call is set by the bytes each
// workgroup streams (x rows of its tile and A rows of its column blocks over all of K) as long as
// the grid fits on the chip. One token group of 16 and one 16-column block per workgroup, 8
// waves splitting K, while that grid stays within two workgroups per compute unit; beyond that
// two token groups sharing each A fragment over 3 column blocks (x read once per tile), or 4
// when the slices have 4 or fewer blocks that 3 does not divide. The 2-deep operand ring
// measured faster than 4-deep.
int shrink_variant(const Knobs& kn, int64_t T, int32_t S, int32_t R, int32_t G) {
  if (kn.shape >= 0 && kn.shape < lmx::num_shrink_variants()) return kn.shape;
  const int64_t nblk = int64_t(S) * ((R + 15) / 16);
  if (nblk % 3 == 0) return (cdiv(T, 16) + G) * nblk <= 512 ? 2 : 4;
  return nblk <= 4 ? 1 : 4;
}

// Shrink launch plan and workspace: [0, sched) the standalone scheduler's tile list (only for
// many segments), then the stream-K partial planes. Stream-K gives every compute unit an equal
// share of the (tile, reduction step) work, about one workgroup per compute unit.
struct ShrinkWs {
  bool lds;          // LDS-staged kernel (else the register-ring kernel)
  bool gemv;         // wave-reduction kernel (direct only)
  bool in_launch;    // stream-K pieces added by each tile's last workgroup (arrival counters)
  int variant, bm, grid_x, gy, mp, unit;
  int64_t bound, q;  // tile bound; stream-K units per workgroup (0 = direct mode)
  size_t sched, part, total;  // byte offsets: schedule list at kCounterBytes, partial planes
};

// Expand kernel shape (rocprofv3 sweeps and event timings on MI355X). From 512 tokens, slices of
// rank exactly 16 with 16-bit types and 16-byte aligned h, B and y rows take the shared-B kernel
// (8192 tokens: 62 -> 56 us; 1024: 17.6 -> 16.7 us; 512, after a 512 MiB write: 12.2 -> 11.0 us;
// at 256 tokens and below it is no faster). Otherwise 4 waves with a 2-deep ring of y
// and B chunks up to 1024 tokens, and from 2048 tokens 128-column chunks with 16-byte y pieces
// and a 1-deep ring (fewer bytes in flight per compute unit measured faster than deeper rings;
// the wide chunks saved 3-12% at 2048..6144 tokens). Blocks whose y rows or start are not
// 16-byte aligned take the 8-byte form inside the same launch.
int expand_variant(const Knobs& kn, int64_t T, bool shared_ok) {
  if (kn.eshape >= 0) {
    const bool shared = kn.eshape == lmx::kExpandSharedD1 || kn.eshape == lmx::kExpandSharedD2;
    return (shared && !shared_ok) ? 6 : kn.eshape;
  }
  if (shared_ok && T >= 512) return lmx::kExpandSharedD1;
  return T >= 2048 ? 6 : 3;
}

size_t schedule_bytes(int64_t T, int32_t G, int bm) {
  if (G <= kInlineMaxSegments) return 0;
  return size_t(cdiv(T, bm) + G) * 16 + 256;
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// The LDS-staged shrink covers the 16-bit types whose x and A rows are 16-byte aligned and
// whose K is a multiple of 8; its shape is the smallest column-block count that holds every
// block of the slices (or 12 blocks per workgroup beyond that).
int shrink_lds_variant(const Knobs& kn, int64_t T, int32_t S, int32_t R, int32_t G) {
  if (kn.shape >= 0 && kn.shape < lmx::num_shrink_lds_variants()) return kn.shape;
  const int64_t nblk = int64_t(S) * ((R + 15) / 16);
  if (nblk == 3) {
    // Three column blocks (rank 16 over three slices, the decode projections): the shortest
    // tiles whose grid fits in one round of 256 workgroups. Kernel durations on the decode
    // sweep (rocprofv3, each call after a 512 MiB device write, so the caches hold dirty lines
    // as after the expand that precedes a shrink): 32-position tiles, 2 waves, 6 stages
    // 22.6 / 23.5 / 26.4 us at 2048 / 4096 / 6144 tokens (4 stages: 24.1 / 26.2 / 28.1; 8
    // stages no better); at 8192 (260 such tiles) 48-position tiles, 3 waves, 6 stages 32.1 us,
    // against 35.9 us for 64-position tiles (after a 512 MiB read instead: 23.5 and 26.1 us,
    // 39 us for 128-position tiles). Shorter tiles re-read the A rows from the L2 more often
    // but keep more compute units streaming x.
    for (int v : {9, 12, 7})
      if (cdiv(T, lmx::shrink_lds_bm(v)) + G <= 256) return v;
    return 1;
  }
  int widest = 0;
  for (int v = 0; v < lmx::num_shrink_lds_variants(); ++v) {
    if (lmx::shrink_lds_bm(v) != 128) continue;
    if (lmx::shrink_lds_ncb(v) >= nblk) return v;
    if (lmx::shrink_lds_ncb(v) > lmx::shrink_lds_ncb(widest)) widest = v;
  }
  return widest;
}

// Which shrink kernel to run when the LDS-staged one is eligible (event timings and rocprofv3
// sweeps on MI355X). The LDS-staged kernel's direct-to-LDS loads fetch whole 128-byte row
// chunks (the register ring's MFMA-layout loads take 64 bytes from each of 16 rows, and its
// address path stalls on the L1), and each A chunk is shared by the whole tile: with three
// column blocks from 8 Mi elements (the short-tile shapes, see shrink_lds_variant); otherwise
// when even the register ring's wider shape would need a second round of workgroups and T * K
// is large.
bool prefer_lds(const Knobs& kn, int dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                    int32_t G) {
  if (kn.family >= 0) return kn.family == 1;
  const int64_t nblk = int64_t(S) * ((R + 15) / 16);
  // three column blocks: the short-tile LDS shapes from 8 Mi elements of x (2048 tokens at
  // K = 4096: 21.3 us against 22.9 us for the register ring; at 1024 tokens the ring's 13.6 us
  // against 21.0 us)
  if (nblk == 3) return T * K >= (int64_t(8) << 20);
  if (T * K < (int64_t(16) << 20) || nblk > 4) return false;
  const int v = shrink_variant(kn, T, S, R, G);
  const int64_t ring_wgs = (cdiv(T, lmx::shrink_plan_bm(dtype, v)) + G) *
                           cdiv(nblk, lmx::shrink_plan_cb(dtype, v));
  return ring_wgs > 256;
}

ShrinkWs shrink_ws(const Knobs& kn, int dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                   int32_t G, bool lds, bool gemv = false) {
  ShrinkWs w{};
  w.lds = lds;
  w.gemv = gemv;
  const int64_t nblk = int64_t(S) * ((R + 15) / 16);
  int64_t gy, frags;
  if (gemv) {  // one workgroup per 16-token tile and 16-column block, over all of K
    w.variant = 0;
    w.bm = 16;
    w.unit = 32;
    w.gy = int(nblk);
    w.bound = cdiv(T, 16) + G;
    w.grid_x = int(w.bound);
    w.sched = schedule_bytes(T, G, w.bm);
    w.part = align256(kCounterBytes + w.sched);
    w.total = w.sched > 0 ? kCounterBytes + w.sched : 0;
    return w;
  }
  if (lds) {
    w.variant = shrink_lds_variant(kn, T, S, R, G);
    w.bm = lmx::shrink_lds_bm(w.variant);
    w.unit = lmx::kShrinkLdsUnit;
    gy = cdiv(nblk, lmx::shrink_lds_ncb(w.variant));
    frags = (w.bm + 16 * lmx::shrink_lds_ncb(w.variant)) / 8;  // 1 KiB loads per stage
  } else {
    w.variant = shrink_variant(kn, T, S, R, G);
    w.bm = lmx::shrink_plan_bm(dtype, w.variant);
    w.unit = dtype == LORA_F32 ? 16 : 32;
    gy = cdiv(nblk, lmx::shrink_plan_cb(dtype, w.variant));
    frags = w.bm / 16 + lmx::shrink_plan_cb(dtype, w.variant);  // 1 KiB loads per step
  }
  w.gy = int(gy);
  w.bound = cdiv(T, w.bm) + G;
  const int64_t nsteps = cdiv(K, w.unit);
  // Shared (tile, step) work pays when one workgroup per tile leaves most compute units idle and
  // each workgroup would stream a lot. With the in-launch completion (arrival counters) it costs
  // three dependent memory round trips instead of a second launch: measured on the decode sweep
  // it pays only below about 48 direct workgroups (50 tokens: 24 workgroups 14.9 us, 192 sharing
  // 12.0 us, cold calls), with 64 workgroups per grid row; the LDS-staged kernel runs direct
  // there (8192 tokens: 52 us against 55 us shared). An explicit plan may ask for the second
  // launch instead (finish 0) or for a split the counters cannot cover.
  const int64_t direct_wgs = w.bound * gy;
  const bool counters_fit = w.bound * gy <= kMaxCounters;
  w.in_launch = kn.finish >= 0 ? (kn.finish == 1 && counters_fit) : counters_fit;
  bool shared;
  int64_t pdef;
  if (w.in_launch) {
    // k = 2, 4 or 8 pieces per tile (every piece inside one tile when the step count divides by
    // k: pieces that straddle two tiles pay two searches and two completions), the largest with
    // at most about 320 workgroups; direct below 2. rocprofv3, each call after a 512 MiB write
    // (decode sweep, 3 column blocks): 50 tokens k = 8, 192 workgroups 9.9 us; 128 tokens k = 8,
    // 288 workgroups 10.9 us (64 per grid row, straddling: 13.0 us); 256 tokens k = 4, 240
    // workgroups 10.1 us (direct 12.9 us, k = 8 11.3 us); 512 tokens k = 2, 216 workgroups
    // 12.2 us (direct 13.3 us); 1024 tokens direct 13.5 us (k = 2: 17.3 us).
    int64_t k = 1;
    if (!lds)
      while (k < 8 && direct_wgs * k * 2 <= 320) k *= 2;
    shared = k > 1;
    pdef = w.bound * k;
  } else {
    shared = lds ? direct_wgs < 256
                 : direct_wgs < 128 && nsteps * frags * 1024 >= (int64_t(512) << 10);
    pdef = std::max<int64_t>(1, 256 / gy);
  }
  const int64_t P = kn.split >= 0 ? kn.split : (shared ? pdef : 0);
  w.sched = schedule_bytes(T, G, w.bm);
  const size_t base = kCounterBytes;  // the counter region leads every nonzero workspace
  w.part = align256(base + w.sched);
  if (P == 0) {
    w.q = 0;
    w.in_launch = false;
    w.grid_x = int(w.bound);
    w.total = w.sched > 0 ? base + w.sched : 0;
  } else {
    const int64_t units = w.bound * nsteps;
    w.q = cdiv(units, P);
    w.grid_x = int(cdiv(units, w.q));
    w.mp = int((nsteps - 1) / w.q + 2);
    w.total = w.part + size_t(w.mp) * size_t(T) * size_t(S) * size_t(R) * 4;
  }
  return w;
}

lora_status hip_status(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_EHIP; }

// Workspace of the fused MLP: byte offsets of its six sections (256-byte aligned).
// Workgroups of the sums kernel launches (two fit per compute unit): about 512 where the
// partials are a small part of the bytes moved; 256 for the sums over tokens of x and dout
// alone, whose row chunks each add nh x 64 bytes of partials per column.
#ifndef LMX_SUMS_COLS_TARGET
#define LMX_SUMS_COLS_TARGET 256
#endif
#ifndef LMX_SUMS_ROWS_TARGET
#define LMX_SUMS_ROWS_TARGET 512
#endif

struct MlpLayout {
  int64_t rp;           // rank rounded up to 32
  lmx::SumJobs gu, dn;  // the LoRA-A products of x (gate, up) and of hmid (down)
  size_t xa_gu, lb_gu, hmid, xa_d, lb_d, apad, rowpart, total;
};

// LoRA-A products h = round(P A^T) through the sums kernel's row side read 16 * ceil(r / 16) rows
// of each A: the caller's A when its rank is a multiple of 16 and its rows are 16-byte aligned,
// else a zero-padded copy in the workspace.
bool lora_a_in_place(int32_t r, std::initializer_list<const void*> as) {
  if (r % 16 != 0) return false;
  for (const void* a : as)
    if (!al16(a)) return false;
  return true;
}

MlpLayout mlp_layout(int64_t M, int64_t H, int64_t I, int32_t r) {
  MlpLayout L{};
  L.rp = cdiv(r, 32) * 32;
  const int JB = int(cdiv(r, 16));
  int64_t rf1 = 0, cf1 = 0, rf2 = 0, cf2 = 0;
  L.gu.n = 1; L.gu.M = int(M); L.gu.JB = JB;
  L.gu.job[0].C = int(H); L.gu.job[0].nr = 2; L.gu.job[0].nh = 0;
  lmx::plan_sums(L.gu, LMX_SUMS_ROWS_TARGET, &rf1, &cf1);
  L.dn.n = 1; L.dn.M = int(M); L.dn.JB = JB;
  L.dn.job[0].C = int(I); L.dn.job[0].nr = 1; L.dn.job[0].nh = 0;
  lmx::plan_sums(L.dn, 512, &rf2, &cf2);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += align256(bytes); return at; };
  L.xa_gu = take(size_t(M) * 2 * L.rp * 2);
  L.lb_gu = take(size_t(2 * I) * 2 * L.rp * 2);
  L.hmid = take(size_t(M) * I * 2);
  L.xa_d = take(size_t(M) * L.rp * 2);
  L.lb_d = take(size_t(H) * L.rp * 2);
  L.apad = take(size_t(16 * JB) * (2 * H + I) * 2);  // [A_g | A_u | A_d] padded copies
  L.rowpart = take(size_t(std::max(rf1, rf2)) * 4);
  L.total = off;
  return L;
}

// Workspace of the LoRA linear projections (P = 1 or 3 projections of one x): byte offsets of
// [xa [M][P rp]], the scaled LoRA-B copies [N_p][rp] and the shrink partials.
struct LinearLayout {
  int64_t rp;
  int P;
  lmx::SumJobs xs;  // the LoRA-A products of x, one row-side operand per projection
  size_t xa, lb[3], apad, rowpart, total;
};

LinearLayout linear_layout(int64_t M, int64_t K, const int64_t* N, int P, int32_t r) {
  LinearLayout L{};
  L.rp = cdiv(r, 32) * 32;
  L.P = P;
  const int JB = int(cdiv(r, 16));
  int64_t rf = 0, cf = 0;
  L.xs.n = 1; L.xs.M = int(M); L.xs.JB = JB;
  L.xs.job[0].C = int(K); L.xs.job[0].nr = P; L.xs.job[0].nh = 0;
  lmx::plan_sums(L.xs, LMX_SUMS_ROWS_TARGET, &rf, &cf);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += align256(bytes); return at; };
  L.xa = take(size_t(M) * P * L.rp * 2);
  for (int p = 0; p < P; ++p) L.lb[p] = take(size_t(N[p]) * L.rp * 2);
  L.apad = take(size_t(16 * JB) * K * P * 2);
  L.rowpart = take(size_t(rf) * 4);
  L.total = off;
  return L;
}

lora_status mlp_forward(lora_dtype dtype, int64_t M, int64_t H, int64_t I, int32_t r, float scale,
                        const void* x, int64_t ldx, const void* w_gate, const void* w_up,
                        const void* w_down, const void* a_gate, const void* b_gate,
                        const void* a_up, const void* b_up, const void* a_down,
                        const void* b_down, void* out, int64_t ldo, void* e_save, void* v_save,
                        int64_t lde, void* workspace, size_t workspace_bytes, void* stream);

// Workspace of the LoRA MLP backward: byte offsets of the scaled / padded / transposed LoRA
// operands, the LoRA-A products and their gradients, the gradient intermediates and the partial
// sums.
struct MlpBwdLayout {
  int64_t rp;
  lmx::SumJobs in;     // LoRA-A products of x and dout (sums over columns; pointers set per call)
  lmx::SumJobs both;   // one pass over de, dv, hmid: sums over columns and over tokens
  lmx::SumJobs cols;   // sums over tokens of x and dout
  size_t sbdt, sbgt, sbut, adt, adp, agp, aup, agut, xa_gu, dxa_d, xa_d, dxa_gu, hmid, dedv,
      rowpart, colpart, total;
};

MlpBwdLayout mlp_bwd_layout(int64_t M, int64_t H, int64_t I, int32_t r) {
  MlpBwdLayout L{};
  L.rp = cdiv(r, 32) * 32;
  const int rp = int(L.rp);
  const int JB = int(cdiv(r, 16));
  int64_t rf[3] = {0, 0, 0}, cf[3] = {0, 0, 0};
  auto init = [&](lmx::SumJobs& j, int n) { j.n = n; j.M = int(M); j.JB = JB; };
  auto job = [](lmx::SumJob& j, int64_t C, int nr, int nh) { j.C = int(C); j.nr = nr; j.nh = nh; };
  // Two workgroups per compute unit (their LDS allows two) where the partials are a small part
  // of the bytes read; one per compute unit for the sums over tokens of x and dout alone, whose
  // row chunks each add nh x 64 bytes of partials per column, so the chunks stay long.
  init(L.in, 2);
  job(L.in.job[0], H, 2, 0);  // x: xa_g, xa_u
  job(L.in.job[1], H, 1, 0);  // dout: dxa_d
  lmx::plan_sums(L.in, LMX_SUMS_ROWS_TARGET, &rf[0], &cf[0]);
  init(L.both, 3);
  for (int q = 0; q < 3; ++q) job(L.both.job[q], I, 1, 1);  // de, dv, hmid
  lmx::plan_sums(L.both, 512, &rf[1], &cf[1]);
  init(L.cols, 2);
  job(L.cols.job[0], H, 0, 2);  // x: dA_g, dA_u
  job(L.cols.job[1], H, 0, 1);  // dout: dB_d
  lmx::plan_sums(L.cols, LMX_SUMS_COLS_TARGET, &rf[2], &cf[2]);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += align256(bytes); return at; };
  L.sbdt = take(size_t(rp) * H * 2);
  L.sbgt = take(size_t(rp) * I * 2);
  L.sbut = take(size_t(rp) * I * 2);
  L.adt = take(size_t(I) * rp * 2);
  L.adp = take(size_t(rp) * I * 2);
  L.agp = take(size_t(rp) * H * 2);
  L.aup = take(size_t(rp) * H * 2);
  L.agut = take(size_t(H) * 2 * rp * 2);
  L.xa_gu = take(size_t(M) * 2 * rp * 2);
  L.dxa_d = take(size_t(M) * rp * 2);
  L.xa_d = take(size_t(M) * rp * 2);
  L.dxa_gu = take(size_t(M) * 2 * rp * 2);
  L.hmid = take(size_t(M) * I * 2);
  L.dedv = take(size_t(M) * 2 * I * 2);
  L.rowpart = take(size_t(std::max({rf[0], rf[1], rf[2]})) * 4);
  L.colpart = take(size_t(std::max({cf[0], cf[1], cf[2]})) * 4);
  L.total = off;
  return L;
}

// The shared body of lora_linear_fused (P = 1) and lora_qkv_fused (P = 3).
lora_status linear_fused(lora_dtype dtype, int64_t M, int64_t K, const int64_t* N, int P,
                         int32_t r, float scale, const void* x, int64_t ldx, const void* const* w,
                         const void* const* a, const void* const* b, void* const* out,
                         const int64_t* ldo, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (dtype != LORA_BF16) return LORA_EUNSUPPORTED;
  if (M < 0 || K < 1 || r < 1) return LORA_EINVAL;
  for (int p = 0; p < P; ++p)
    if (N[p] < 1) return LORA_EINVAL;
  if (r > 64 || K % 32 != 0) return LORA_EUNSUPPORTED;
  if (M >= INT_MAX || K >= INT_MAX / 4) return LORA_EUNSUPPORTED;
  for (int p = 0; p < P; ++p)
    if (N[p] >= INT_MAX / 4) return LORA_EUNSUPPORTED;
  if (M == 0) return LORA_OK;
  if (!x) return LORA_EINVAL;
  for (int p = 0; p < P; ++p)
    if (!w[p] || !a[p] || !b[p] || !out[p]) return LORA_EINVAL;
  if (ldx < K) return LORA_EINVAL;
  for (int p = 0; p < P; ++p)
    if (ldo[p] < N[p]) return LORA_EINVAL;
  if (!al16(x) || (ldx * 2) % 16 != 0) return LORA_EUNSUPPORTED;
  for (int p = 0; p < P; ++p)
    if (!al16(w[p])) return LORA_EUNSUPPORTED;
  int64_t ntot = 0;
  for (int p = 0; p < P; ++p) ntot += N[p];
  if (ntot * 64 >= int64_t(INT_MAX)) return LORA_EUNSUPPORTED;  // the scaled-B copies
  const LinearLayout L = linear_layout(M, K, N, P, r);
  if (workspace == nullptr || workspace_bytes < L.total || !al16(workspace)) return LORA_EWORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  uint16_t* xa = reinterpret_cast<uint16_t*>(ws + L.xa);
  const int64_t rp = L.rp;
  auto u16 = [](const void* q) { return static_cast<const uint16_t*>(q); };
  // 1. scaled LoRA-B operands s * B_p, zero padded to rp columns
  {
    lmx::ScaleJobs jobs{};
    for (int p = 0; p < P; ++p)
      jobs.job[p] = {u16(b[p]), r, reinterpret_cast<uint16_t*>(ws + L.lb[p]), rp, int(N[p]), 0};
    if (lmx::launch_scale_lora_b(jobs, scale, r, st) != hipSuccess) return LORA_EHIP;
  }
  // 2. [xa_0 | .. | xa_{P-1}] = round(x [A_0; ..]^T) in one pass over x: the sums kernel's row
  //    side with one operand per projection, then the fixed-order reduction (rank padding zeroed)
  {
    const int JB = L.xs.JB;
    const uint16_t* ap[3] = {nullptr, nullptr, nullptr};
    const bool in_place = P == 1 ? lora_a_in_place(r, {a[0]}) : lora_a_in_place(r, {a[0], a[1], a[2]});
    if (in_place) {
      for (int p = 0; p < P; ++p) ap[p] = u16(a[p]);
    } else {
      lmx::TJobs t{};
      t.n = P;
      for (int p = 0; p < P; ++p) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(ws + L.apad) + int64_t(p) * 16 * JB * K;
        t.job[p] = {u16(a[p]), K, dst, K, 16 * JB, int(K), 0, int(K), r, 1.0f, true};
        ap[p] = dst;
      }
      if (lmx::launch_small_transposes(t, st) != hipSuccess) return LORA_EHIP;
    }
    lmx::SumJobs j = L.xs;
    j.job[0].P = u16(x); j.job[0].ldp = ldx; j.job[0].ldr = K;
    for (int p = 0; p < 3; ++p) j.job[0].R[p] = ap[p];
    float* rowpart = reinterpret_cast<float*>(ws + L.rowpart);
    if (lmx::launch_sums(j, rowpart, rowpart, st) != hipSuccess) return LORA_EHIP;
    const int64_t rs = M * JB * 16;
    const int nc = j.blk0[1] - j.blk0[0];
    lmx::RedJobs rj{};
    rj.n = P;
    rj.JB = JB;
    for (int p = 0; p < P; ++p) {
      lmx::RedJob& q = rj.job[p];
      q.src = rowpart + j.job[0].rp0 + p * nc * rs; q.pstride = rs; q.np = nc;
      q.out = xa + p * rp; q.osa = P * rp; q.osj = 1; q.A = int(M); q.J = int(rp); q.r = r;
      q.scale = 1.0f;
    }
    if (lmx::launch_reduce_sums(rj, st) != hipSuccess) return LORA_EHIP;
  }
  // 3. out_p = round(x W_p^T + s xa_p B_p^T) with LoRA in K: one launch over the P column
  //    groups (query, key and value share the pass over x and fill the chip together), or the
  //    first group alone and then the others when that finishes sooner (at M = 4096 the query
  //    fills exactly one round of 256-row tiles and key + value one round of 128-row tiles,
  //    where the single launch would leave a half-empty second round)
  int first = 0;  // groups [0, first) go in a launch of their own
  if (P > 1) {
    int nb[3], all = 0, rest = 0;
    for (int p = 0; p < P; ++p) { nb[p] = int(cdiv(N[p], 256)); all += nb[p]; }
    rest = all - nb[0];
    const double one = lmx::gemm_plain_cost(int(M), all, nullptr);
    const double split = lmx::gemm_plain_cost(int(M), nb[0], nullptr) + lmx::gemm_plain_cost(int(M), rest, nullptr);
    if (split + 0.05 < one) first = 1;
  }
  const int bounds[3] = {0, first, P};  // launch i covers groups [bounds[i], bounds[i + 1])
  for (int li = first > 0 ? 0 : 1; li < 2; ++li) {
    const int g0 = bounds[li], g1 = bounds[li + 1];
    lmx::GemmArgs g{};
    g.A = u16(x); g.lda = ldx; g.W0 = u16(w[g0]); g.W1 = u16(w[g0]); g.ldw = K;
    g.A2 = xa + g0 * rp; g.lda2 = P * rp;
    g.B2 = reinterpret_cast<const uint16_t*>(ws + L.lb[g0]); g.ldb2 = rp;
    g.C = static_cast<uint16_t*>(out[g0]); g.ldc = ldo[g0];
    g.M = int(M); g.N = int(N[g0]); g.K = int(K); g.K2 = int(rp);
    if (g1 - g0 > 1) {
      g.A2 = xa;
      g.ngroups = g1 - g0;
      g.gblk[0] = 0;
      for (int q = 0; q < g1 - g0; ++q) {
        const int p = g0 + q;
        g.gW[q] = u16(w[p]);
        g.gB2[q] = reinterpret_cast<const uint16_t*>(ws + L.lb[p]);
        g.ga2[q] = p * rp;
        g.gC[q] = static_cast<uint16_t*>(out[p]);
        g.gldc[q] = ldo[p];
        g.gN[q] = int(N[p]);
        g.gblk[q + 1] = g.gblk[q] + int(cdiv(N[p], 256));
      }
    }
    if (lmx::launch_gemm_lora(g, lmx::kGemmPlain, st) != hipSuccess) return LORA_EHIP;
  }
  return LORA_OK;
}

// The shrink entry points' shared body. `in_scratch`: the workspace is the library's device
// scratch array (lora_shrink_noalloc): a plan needing more is refused, and the arrival counters
// a call uses are cleared first by a small fill kernel (the array keeps the last call's
// contents).
lora_status shrink_impl(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R, int32_t L,
                        int32_t G, const void* x, int64_t ldx, const void* w_a, int64_t lda,
                        const int32_t* seg_indptr, const int32_t* weight_indices,
                        const int32_t* permutation, const int32_t* lora_ranks, void* h,
                        int64_t ldh, const Knobs& kn, void* workspace, size_t workspace_bytes,
                        void* stream, bool in_scratch) {
  if (!valid_dtype(dtype)) return LORA_EUNSUPPORTED;
  if (T < 0 || G < 0 || S < 1 || R < 1) return LORA_EINVAL;
  if (S > kMaxSlices || R > kMaxRank) return LORA_EUNSUPPORTED;
  if (T == 0 || G == 0) return LORA_OK;
  if (K < 1 || L < 1) return LORA_EINVAL;
  if (T >= INT_MAX || K >= INT_MAX || G >= INT_MAX / 2) return LORA_EUNSUPPORTED;
  if (!x || !w_a || !seg_indptr || !weight_indices || !lora_ranks || !h)
    return LORA_EINVAL;
  if (ldx < K || lda < K || ldh < int64_t(S) * R) return LORA_EINVAL;
  if (int64_t(S) * R * T * 16 >= int64_t(1) << 62) return LORA_EUNSUPPORTED;
  const int e = esize(dtype);
  const bool aligned = al16(x) && al16(w_a) && (ldx * e) % 16 == 0 && (lda * e) % 16 == 0;
  const bool gemv = kn.family == 2 && dtype != LORA_F32 && aligned && K % 8 == 0;
  const bool lds = !gemv && dtype != LORA_F32 && aligned && K % 8 == 0 &&
                   prefer_lds(kn, int(dtype), T, K, S, R, G);
  const ShrinkWs ws = shrink_ws(kn, int(dtype), T, K, S, R, G, lds, gemv);
  const int variant = ws.variant;
  const int bm = ws.bm;
  if (ws.total > 0 && (workspace == nullptr || workspace_bytes < ws.total)) return LORA_EWORKSPACE;
  if (ws.total > 0 && !al16(workspace)) return LORA_EWORKSPACE;
  const int64_t bound = ws.bound;
  if (bound >= INT_MAX) return LORA_EUNSUPPORTED;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(workspace);
  if (in_scratch && ws.q > 0 && ws.in_launch &&
      lmx::launch_zero_ints(reinterpret_cast<int*>(wsb), int(bound) * ws.gy, st) != hipSuccess)
    return LORA_EHIP;
  lmx::ShrinkArgs a{};
  a.x = x; a.w_a = w_a; a.seg_indptr = seg_indptr; a.weight_indices = weight_indices;
  a.permutation = permutation; a.lora_ranks = lora_ranks; a.h = h;
  a.K = K; a.ldx = ldx; a.lda = lda; a.ldh = ldh; a.S = S; a.R = R; a.G = G; a.T = int(T);
  if (ws.sched > 0) {
    int4* tiles = reinterpret_cast<int4*>(wsb + kCounterBytes + 256);
    int* count = reinterpret_cast<int*>(wsb + kCounterBytes);
    hipError_t err = lmx::launch_schedule(seg_indptr, weight_indices, G, bm, tiles, count, st);
    if (err != hipSuccess) return LORA_EHIP;
    a.tiles = tiles; a.tile_count = count;
  }
  a.sk_q = ws.q; a.sk_tiles = int(bound); a.sk_mp = ws.mp; a.sk_unit = ws.unit;
  if (ws.q > 0) a.part = reinterpret_cast<float*>(wsb + ws.part);
  if (ws.q > 0 && ws.in_launch) a.counters = reinterpret_cast<int*>(wsb);
#ifndef LMX_NO_XCD_ROWS
  if (!ws.gemv && ws.q == 0 && (ws.lds || ws.gy > 1)) a.xcd_rows = ws.gy;
#endif
  lmx::ShrinkPlan splan{variant, ws.grid_x, aligned, ws.lds, ws.gemv};
  if (lmx::launch_shrink(int(dtype), a, splan, st) != hipSuccess) return LORA_EHIP;
  if (ws.q > 0 && !ws.in_launch)
    return hip_status(lmx::launch_shrink_sk_reduce(int(dtype), a, bm, st));
  return LORA_OK;
}

// Workspace of the projection backward (P = 1, or 3 projections of one x): byte offsets of its
// sections (256-byte aligned). Token-side sums need P + 2 jobs (x carries at most two Q
// operands per job) and a sums launch takes four, so P = 3 makes two launches (cols, cols2).
struct LinBwdLayout {
  int64_t rp;
  int P, ncols;           // projections; sums launches on the token side (1 or 2)
  lmx::SumJobs in, cols, cols2;
  size_t sbt[3], ap[3], at, xa, dxa, dcat, rowpart, colpart, total;
};

LinBwdLayout lin_bwd_layout(int64_t M, int64_t K, const int64_t* N, int P, int32_t r) {
  LinBwdLayout L{};
  L.rp = cdiv(r, 32) * 32;
  L.P = P;
  const int JB = int(cdiv(r, 16));
  int64_t rf[3] = {0, 0, 0}, cf[3] = {0, 0, 0};
  auto init = [&](lmx::SumJobs& j, int n) { j.n = n; j.M = int(M); j.JB = JB; };
  auto job = [](lmx::SumJob& j, int64_t C, int nr, int nh) { j.C = int(C); j.nr = nr; j.nh = nh; };
  init(L.in, P + 1);
  job(L.in.job[0], K, P, 0);                                 // x: xa of every projection
  for (int p = 0; p < P; ++p) job(L.in.job[1 + p], N[p], 1, 0);  // dout_p: dxa_p
  lmx::plan_sums(L.in, LMX_SUMS_ROWS_TARGET, &rf[0], &cf[0]);
  if (P == 1) {
    L.ncols = 1;
    init(L.cols, 2);
    job(L.cols.job[0], K, 0, 1);     // x: dA
    job(L.cols.job[1], N[0], 0, 1);  // dout: dB
    lmx::plan_sums(L.cols, LMX_SUMS_COLS_TARGET, &rf[1], &cf[1]);
  } else {
    L.ncols = 2;
    init(L.cols, 4);
    job(L.cols.job[0], K, 0, 2);     // x: dA_q, dA_k
    job(L.cols.job[1], K, 0, 1);     // x: dA_v
    job(L.cols.job[2], N[0], 0, 1);  // dq: dB_q
    job(L.cols.job[3], N[1], 0, 1);  // dk: dB_k
    lmx::plan_sums(L.cols, LMX_SUMS_COLS_TARGET, &rf[1], &cf[1]);
    init(L.cols2, 1);
    job(L.cols2.job[0], N[2], 0, 1);  // dv: dB_v
    lmx::plan_sums(L.cols2, LMX_SUMS_COLS_TARGET, &rf[2], &cf[2]);
  }
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += align256(bytes); return at; };
  const size_t rp = size_t(L.rp);
  int64_t ntot = 0;
  for (int p = 0; p < P; ++p) {
    L.sbt[p] = take(rp * N[p] * 2);
    L.ap[p] = take(rp * K * 2);
    ntot += N[p];
  }
  L.at = take(size_t(K) * P * rp * 2);
  L.xa = take(size_t(M) * P * rp * 2);
  L.dxa = take(size_t(M) * P * rp * 2);
  L.dcat = P > 1 ? take(size_t(M) * ntot * 2) : 0;
  L.rowpart = take(size_t(std::max({rf[0], rf[1], rf[2]})) * 4);
  L.colpart = take(size_t(std::max({cf[0], cf[1], cf[2]})) * 4);
  L.total = off;
  return L;
}

// Workspace of lora_shrink_expand. Single launch: every counter sits in the leading 32 KiB that
// every call leaves zero, at offsets that do not depend on the sizes, so calls of any size can
// share one workspace: the shrink's arrival counters in [0, 16 KiB), the per-tile done counters
// from 28 KiB, the wait-bound flag in the last int; the shrink's partial planes follow as in
// lora_shrink's own layout. Two launches: the shrink's workspace, then the expand's at
// expand_off. The query covers both, since the choice depends on pointer alignment.
constexpr size_t kPairFlagOffset = kCounterBytes - 4;
static_assert(kPairFlagOffset == LORA_SHRINK_EXPAND_FLAG_OFFSET, "flag offset of the header");
constexpr int64_t kPairArrivalInts = 4096;
// Each arrival counter of the single launch on a 64-byte line of its own: expand waves poll them
// while shrink pieces count in on them.
constexpr int kPairCounterShift = 4;
constexpr size_t kPairDoneOffset = 28672;
constexpr int64_t kPairMaxTiles = 192;
static_assert(kPairArrivalInts * 4 <= kPairDoneOffset &&
              kPairDoneOffset + kPairMaxTiles * 4 <= kPairFlagOffset, "pair counter layout");

struct PairWs {
  ShrinkWs sw;           // the single launch's shrink plan
  bool shape_ok;         // sizes allow the single launch (alignment is checked per call)
  size_t single_total;
  size_t expand_off, two_total;
};

PairWs pair_ws(int dtype, int64_t T, int64_t K, int32_t S, int32_t R, int32_t G) {
  PairWs w{};
  const Knobs kn;
  // Single launch: 16-bit types at decode sizes, where lora_shrink takes the 1x1x8x2 register
  // ring (K % 8 == 0 with aligned rows: the LDS-staged family is not preferred there) from the
  // inline search, and lora_expand the 64-column, 4-wave, 2-deep form over 16-token tiles.
  w.shape_ok = (dtype == LORA_BF16 || dtype == LORA_F16) && T < 1024 && K % 8 == 0 &&
               G <= kInlineMaxSegments && R <= 32 &&
               !prefer_lds(kn, dtype, T, K, S, R, G);
  if (w.shape_ok) {
    w.sw = shrink_ws(kn, dtype, T, K, S, R, G, false);
    w.shape_ok = w.sw.variant == 2 && w.sw.sched == 0 && w.sw.bound <= kPairMaxTiles &&
                 (w.sw.bound * w.sw.gy << kPairCounterShift) <= kPairArrivalInts && w.sw.q > 0 &&
                 w.sw.in_launch;
  }
  if (w.shape_ok) w.single_total = std::max(w.sw.total, kCounterBytes);
  const size_t st = lora_shrink_workspace_size_ex(lora_dtype(dtype), T, K, S, R, G, nullptr);
  w.expand_off = align256(st);
  w.two_total = w.expand_off + schedule_bytes(T, G, 16);
  return w;
}

// The projection backward for P = 1 or 3 projections of one x (the query, key and value
// projections; their dx terms summed and rounded once). w_t = [W_0^T | .. | W_{P-1}^T] [K][Ntot].
lora_status linear_backward(lora_dtype dtype, int64_t M, int64_t K, const int64_t* N, int P,
                            int32_t r, float scale, const void* x, int64_t ldx,
                            const void* const* dout, const int64_t* lddo, const void* w_t,
                            const void* const* a, const void* const* b, void* dx, int64_t lddx,
                            void* const* da, void* const* db, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (dtype != LORA_BF16) return LORA_EUNSUPPORTED;
  if (M < 0 || K < 1 || r < 1) return LORA_EINVAL;
  int64_t ntot = 0;
  for (int p = 0; p < P; ++p) {
    if (N[p] < 1) return LORA_EINVAL;
    if (N[p] % 32 != 0 || N[p] >= INT_MAX / 8) return LORA_EUNSUPPORTED;
    ntot += N[p];
  }
  if (r > 64 || K % 32 != 0) return LORA_EUNSUPPORTED;
  if (M >= INT_MAX || K >= INT_MAX / 8 || ntot >= INT_MAX / 8) return LORA_EUNSUPPORTED;
  if (M == 0) return LORA_OK;
  if (!x || !w_t || !dx) return LORA_EINVAL;
  for (int p = 0; p < P; ++p)
    if (!dout[p] || !a[p] || !b[p] || !da[p] || !db[p]) return LORA_EINVAL;
  if (ldx < K || lddx < K) return LORA_EINVAL;
  for (int p = 0; p < P; ++p) {
    if (lddo[p] < N[p]) return LORA_EINVAL;
    if (dx == dout[p]) return LORA_EINVAL;
  }
  if (dx == x) return LORA_EINVAL;  // the saved input is never overwritten
  if (!al16(x) || (ldx * 2) % 16 != 0 || !al16(w_t)) return LORA_EUNSUPPORTED;
  for (int p = 0; p < P; ++p)
    if (!al16(dout[p]) || (lddo[p] * 2) % 16 != 0) return LORA_EUNSUPPORTED;
  const LinBwdLayout L = lin_bwd_layout(M, K, N, P, r);
  if (workspace == nullptr || workspace_bytes < L.total || !al16(workspace)) return LORA_EWORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  auto W = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  auto u16 = [](const void* q) { return static_cast<const uint16_t*>(q); };
  const int rp = int(L.rp), prp = P * rp;
  uint16_t *at = W(L.at), *xa = W(L.xa), *dxa = W(L.dxa);
  float* rowpart = reinterpret_cast<float*>(ws + L.rowpart);
  float* colpart = reinterpret_cast<float*>(ws + L.colpart);
  const int JB = L.in.JB;
  auto ncb = [](const lmx::SumJobs& j, int q) { return j.blk0[q + 1] - j.blk0[q]; };
  // 1. operands, rank rows past r zero: s B_p^T [rp][N_p], A_p [rp][K], and
  //    [A_0^T | .. | A_{P-1}^T] [K][P rp]
  {
    lmx::TJobs t{};
    t.n = 3 * P;
    for (int p = 0; p < P; ++p) {
      t.job[3 * p] = {u16(b[p]), r, W(L.sbt[p]), N[p], rp, int(N[p]), 0, int(N[p]), r, scale, false};
      t.job[3 * p + 1] = {u16(a[p]), K, W(L.ap[p]), K, rp, int(K), 0, int(K), r, 1.0f, true};
      t.job[3 * p + 2] = {u16(a[p]), K, at + p * rp, prp, int(K), rp, 0, r, int(K), 1.0f, false};
    }
    if (lmx::launch_small_transposes(t, st) != hipSuccess) return LORA_EHIP;
  }
  // 2. xa_p = round(x A_p^T) in one pass over x and dxa_p = round(dout_p (s B_p)): the sums
  //    kernel's row side in one launch, then the fixed-order reduction (rank padding zeroed)
  {
    lmx::SumJobs j = L.in;
    j.job[0].P = u16(x); j.job[0].ldp = ldx; j.job[0].ldr = K;
    for (int p = 0; p < P; ++p) {
      j.job[0].R[p] = W(L.ap[p]);
      j.job[1 + p].P = u16(dout[p]); j.job[1 + p].ldp = lddo[p];
      j.job[1 + p].R[0] = W(L.sbt[p]); j.job[1 + p].ldr = N[p];
    }
    if (lmx::launch_sums(j, rowpart, colpart, st) != hipSuccess) return LORA_EHIP;
    const int64_t rs = M * JB * 16;
    const int nx = ncb(j, 0);
    lmx::RedJobs rj{};
    rj.n = 2 * P;
    rj.JB = JB;
    for (int p = 0; p < P; ++p) {
      rj.job[p] = {rowpart + j.job[0].rp0 + p * nx * rs, rs, xa + p * rp, prp, 1, int(M), rp, r,
                   nx, 1.0f};
      rj.job[P + p] = {rowpart + j.job[1 + p].rp0, rs, dxa + p * rp, prp, 1, int(M), rp, r,
                       ncb(j, 1 + p), 1.0f};
    }
    if (lmx::launch_reduce_sums(rj, st) != hipSuccess) return LORA_EHIP;
  }
  // 3. sums over tokens: dA_p = dxa_p^T x [r][K], dB_p = s dout_p^T xa_p [N_p][r]
  auto out16 = [](void* q) { return static_cast<uint16_t*>(q); };
  auto da_job = [&](lmx::RedJob& rj, const float* src, void* out) {
    rj = {src, K * JB * 16, out16(out), 1, K, int(K), r, r, 0, 1.0f};
  };
  auto db_job = [&](lmx::RedJob& rj, const float* src, int p) {
    rj = {src, N[p] * JB * 16, out16(db[p]), r, 1, int(N[p]), r, r, 0, scale};
  };
  if (P == 1) {
    lmx::SumJobs j = L.cols;
    j.job[0].P = u16(x); j.job[0].ldp = ldx; j.job[0].Q[0] = dxa; j.job[0].ldq = prp;
    j.job[1].P = u16(dout[0]); j.job[1].ldp = lddo[0]; j.job[1].Q[0] = xa; j.job[1].ldq = prp;
    if (lmx::launch_sums(j, rowpart, colpart, st) != hipSuccess) return LORA_EHIP;
    lmx::RedJobs rj{};
    rj.n = 2;
    rj.JB = JB;
    da_job(rj.job[0], colpart + j.job[0].cp0, da[0]);
    db_job(rj.job[1], colpart + j.job[1].cp0, 0);
    for (int q = 0; q < 2; ++q) rj.job[q].np = j.chunks;
    if (lmx::launch_reduce_sums(rj, st) != hipSuccess) return LORA_EHIP;
  } else {
    {
      lmx::SumJobs j = L.cols;
      j.job[0].P = u16(x); j.job[0].ldp = ldx; j.job[0].ldq = prp;
      j.job[0].Q[0] = dxa; j.job[0].Q[1] = dxa + rp;
      j.job[1].P = u16(x); j.job[1].ldp = ldx; j.job[1].Q[0] = dxa + 2 * rp; j.job[1].ldq = prp;
      for (int p = 0; p < 2; ++p) {
        j.job[2 + p].P = u16(dout[p]); j.job[2 + p].ldp = lddo[p];
        j.job[2 + p].Q[0] = xa + p * rp; j.job[2 + p].ldq = prp;
      }
      if (lmx::launch_sums(j, rowpart, colpart, st) != hipSuccess) return LORA_EHIP;
      const int64_t hstride = int64_t(j.chunks) * K * JB * 16;
      lmx::RedJobs rj{};
      rj.n = 5;
      rj.JB = JB;
      da_job(rj.job[0], colpart + j.job[0].cp0, da[0]);
      da_job(rj.job[1], colpart + j.job[0].cp0 + hstride, da[1]);
      da_job(rj.job[2], colpart + j.job[1].cp0, da[2]);
      db_job(rj.job[3], colpart + j.job[2].cp0, 0);
      db_job(rj.job[4], colpart + j.job[3].cp0, 1);
      for (int q = 0; q < 5; ++q) rj.job[q].np = j.chunks;
      if (lmx::launch_reduce_sums(rj, st) != hipSuccess) return LORA_EHIP;
    }
    {
      lmx::SumJobs j = L.cols2;
      j.job[0].P = u16(dout[2]); j.job[0].ldp = lddo[2];
      j.job[0].Q[0] = xa + 2 * rp; j.job[0].ldq = prp;
      if (lmx::launch_sums(j, rowpart, colpart, st) != hipSuccess) return LORA_EHIP;
      lmx::RedJobs rj{};
      rj.n = 1;
      rj.JB = JB;
      db_job(rj.job[0], colpart + j.job[0].cp0, 2);
      rj.job[0].np = j.chunks;
      if (lmx::launch_reduce_sums(rj, st) != hipSuccess) return LORA_EHIP;
    }
  }
  // 4. dx = round(sum_p dout_p W_p + dxa_p A_p): the plain GEMM over the reduction Ntot with the
  //    LoRA terms in K ([dout_0 | ..] copied side by side first when P > 1, unless it already is)
  const uint16_t* dA = u16(dout[0]);
  int64_t ldA = lddo[0];
  // already side by side (views of one [M][>= Ntot] gradient of a fused projection): read in place
  bool adjacent = true;
  for (int p = 1; p < P; ++p)
    adjacent = adjacent && lddo[p] == lddo[0] && u16(dout[p]) == u16(dout[p - 1]) + N[p - 1];
  if (P > 1 && !adjacent) {
    uint16_t* dcat = W(L.dcat);
    int64_t c0 = 0;
    for (int p = 0; p < P; ++p) {
      if (lmx::launch_copy2d(u16(dout[p]), lddo[p], dcat + c0, ntot, int(M), int(N[p]), st) !=
          hipSuccess)
        return LORA_EHIP;
      c0 += N[p];
    }
    dA = dcat;
    ldA = ntot;
  }
  {
    lmx::GemmArgs g{};
    g.A = dA; g.lda = ldA; g.W0 = u16(w_t); g.W1 = u16(w_t); g.ldw = ntot;
    g.A2 = dxa; g.lda2 = prp; g.B2 = at; g.ldb2 = prp;
    g.C = static_cast<uint16_t*>(dx); g.ldc = lddx;
    g.M = int(M); g.N = int(K); g.K = int(ntot); g.K2 = prp;
    if (lmx::launch_gemm_lora(g, lmx::kGemmPlain, st) != hipSuccess) return LORA_EHIP;
  }
  return LORA_OK;
}

}  // namespace

extern "C" {

const char* lora_status_str(lora_status s) {
  switch (s) {
    case LORA_OK: return "LORA_OK";
    case LORA_EINVAL: return "LORA_EINVAL: invalid argument";
    case LORA_EUNSUPPORTED: return "LORA_EUNSUPPORTED: unsupported dtype or size";
    case LORA_EWORKSPACE: return "LORA_EWORKSPACE: workspace too small";
    case LORA_EHIP: return "LORA_EHIP: HIP runtime error";
    case LORA_EVALUE: return "LORA_EVALUE: invalid metadata values";
  }
  return "LORA_?: unknown status";
}

const char* lora_version(void) { return "lora_mi355x 0.1 gfx950"; }

size_t lora_shrink_workspace_size_ex(lora_dtype dtype, int64_t T, int64_t K, int32_t S,
                                     int32_t R, int32_t G, const lora_plan* plan) {
  if (T <= 0 || G <= 0 || K <= 0 || S <= 0 || R <= 0 || !valid_dtype(dtype)) return 0;
  const Knobs kn = knobs_of(plan);
  if (!knobs_valid(kn)) return 0;
  // the kernel family depends on pointer alignment, which the query does not see: cover each
  // family the call may take
  const size_t reg = shrink_ws(kn, int(dtype), T, K, S, R, G, false).total;
  if (dtype == LORA_F32 || K % 8 != 0 || kn.family == 0) return reg;
  if (kn.family == 2) return std::max(reg, shrink_ws(kn, int(dtype), T, K, S, R, G, false, true).total);
  return std::max(reg, shrink_ws(kn, int(dtype), T, K, S, R, G, true).total);
}

size_t lora_shrink_workspace_size(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                                  int32_t G) {
  return lora_shrink_workspace_size_ex(dtype, T, K, S, R, G, nullptr);
}

size_t lora_expand_workspace_size(lora_dtype dtype, int64_t T, int32_t S, int32_t R, int32_t G,
                                  int64_t N) {
  (void)dtype; (void)S; (void)R; (void)N;
  if (T <= 0 || G <= 0) return 0;
  return schedule_bytes(T, G, 16);  // the smallest tile of any expand shape: the longest list
}

lora_status lora_shrink_ex(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                           int32_t L, int32_t G, const void* x, int64_t ldx, const void* w_a,
                           int64_t lda, const int32_t* seg_indptr, const int32_t* weight_indices,
                           const int32_t* permutation, const int32_t* lora_ranks, void* h,
                           int64_t ldh, const lora_plan* plan, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const Knobs kn = knobs_of(plan);
  if (!knobs_valid(kn)) return LORA_EINVAL;
  return shrink_impl(dtype, T, K, S, R, L, G, x, ldx, w_a, lda, seg_indptr, weight_indices,
                     permutation, lora_ranks, h, ldh, kn, workspace, workspace_bytes, stream,
                     false);
}

lora_status lora_shrink_noalloc(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                                int32_t L, int32_t G, const void* x, int64_t ldx,
                                const void* w_a, int64_t lda, const int32_t* seg_indptr,
                                const int32_t* weight_indices, const int32_t* permutation,
                                const int32_t* lora_ranks, void* h, int64_t ldh, void* stream) {
  const Knobs kn;
  if (T > 0 && G > 0 && K > 0 && S > 0 && R > 0 && valid_dtype(dtype) &&
      lora_shrink_workspace_size_ex(dtype, T, K, S, R, G, nullptr) > kScratchBytes)
    return LORA_EWORKSPACE;  // needs more than the fixed scratch array
  void* ptr = nullptr;
  if (scratch_address(&ptr) != hipSuccess || ptr == nullptr) return LORA_EHIP;
  return shrink_impl(dtype, T, K, S, R, L, G, x, ldx, w_a, lda, seg_indptr, weight_indices,
                     permutation, lora_ranks, h, ldh, kn, ptr, kScratchBytes, stream, true);
}

size_t lora_shrink_noalloc_max_workspace(void) { return kScratchBytes; }

lora_status lora_shrink(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R, int32_t L,
                        int32_t G, const void* x, int64_t ldx, const void* w_a, int64_t lda,
                        const int32_t* seg_indptr, const int32_t* weight_indices,
                        const int32_t* permutation, const int32_t* lora_ranks, void* h,
                        int64_t ldh, void* workspace, size_t workspace_bytes, void* stream) {
  return lora_shrink_ex(dtype, T, K, S, R, L, G, x, ldx, w_a, lda, seg_indptr, weight_indices,
                        permutation, lora_ranks, h, ldh, nullptr, workspace, workspace_bytes,
                        stream);
}

lora_status lora_expand_ex(lora_dtype dtype, int64_t T, int32_t S, int32_t R, int32_t L,
                           int32_t G, int64_t N, const void* h, int64_t ldh, const void* w_b,
                           int64_t ldb, const int32_t* slice_offsets, const int32_t* seg_indptr,
                           const int32_t* weight_indices, const int32_t* permutation,
                           const int32_t* lora_ranks, const float* scalings, void* y,
                           int64_t ldy, const lora_plan* plan, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return LORA_EUNSUPPORTED;
  const Knobs kn = knobs_of(plan);
  if (!knobs_valid(kn)) return LORA_EINVAL;
  if (T < 0 || G < 0 || S < 1 || R < 1 || N < 0) return LORA_EINVAL;
  if (S > kMaxSlices || R > kMaxRank) return LORA_EUNSUPPORTED;
  if (T == 0 || G == 0 || N == 0) return LORA_OK;
  if (L < 1) return LORA_EINVAL;
  if (T >= INT_MAX || N >= INT_MAX / 2 || G >= INT_MAX / 2) return LORA_EUNSUPPORTED;
  if (!h || !w_b || !slice_offsets || !seg_indptr || !weight_indices ||
      !lora_ranks || !scalings || !y)
    return LORA_EINVAL;
  if (ldh < int64_t(S) * R || ldb < R || ldy < N) return LORA_EINVAL;
  if (R > lmx::expand_max_rank(int(dtype))) return LORA_EUNSUPPORTED;
  const int e = esize(dtype);
  const bool aligned_b = al16(h) && al16(w_b) && (ldh * e) % 16 == 0 && (ldb * e) % 16 == 0 &&
                         (int64_t(R) * e) % 16 == 0;
  const bool aligned_y = al16(y) && (ldy * e) % 16 == 0;
  const int variant = expand_variant(kn, T, dtype != LORA_F32 && R == 16 && aligned_b && aligned_y);
  const int bm = lmx::expand_plan_bm(int(dtype), variant);
  const bool shared = dtype != LORA_F32 && (variant == lmx::kExpandSharedD1 ||
                                            variant == lmx::kExpandSharedD2);
  const int bn = expand_bn(kn, T, G, S, N, bm, lmx::expand_plan_waves(int(dtype), variant),
                           lmx::expand_plan_chunk(int(dtype), variant), shared);
  if (cdiv(N, bn) + S > 65535) return LORA_EUNSUPPORTED;
  const size_t need = schedule_bytes(T, G, bm);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LORA_EWORKSPACE;
  const int64_t bound = cdiv(T, bm) + G;
  if (bound >= INT_MAX) return LORA_EUNSUPPORTED;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  lmx::ExpandArgs a{};
  a.h = h; a.w_b = w_b; a.slice_offsets = slice_offsets; a.seg_indptr = seg_indptr;
  a.weight_indices = weight_indices; a.permutation = permutation; a.lora_ranks = lora_ranks;
  a.scalings = scalings; a.y = y;
  a.N = N; a.ldh = ldh; a.ldb = ldb; a.ldy = ldy; a.S = S; a.R = R; a.G = G; a.BN = bn;
  if (need > 0) {
    int4* tiles = reinterpret_cast<int4*>(static_cast<char*>(workspace) + 256);
    int* count = static_cast<int*>(workspace);
    hipError_t err = lmx::launch_schedule(seg_indptr, weight_indices, G, bm, tiles, count, st);
    if (err != hipSuccess) return LORA_EHIP;
    a.tiles = tiles; a.tile_count = count;
  }
  lmx::ExpandPlan eplan{variant, int(bound), aligned_b, aligned_y};
  return hip_status(lmx::launch_expand(int(dtype), a, eplan, st));
}

lora_status lora_expand(lora_dtype dtype, int64_t T, int32_t S, int32_t R, int32_t L, int32_t G,
                        int64_t N, const void* h, int64_t ldh, const void* w_b, int64_t ldb,
                        const int32_t* slice_offsets, const int32_t* seg_indptr,
                        const int32_t* weight_indices, const int32_t* permutation,
                        const int32_t* lora_ranks, const float* scalings, void* y, int64_t ldy,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return lora_expand_ex(dtype, T, S, R, L, G, N, h, ldh, w_b, ldb, slice_offsets, seg_indptr,
                        weight_indices, permutation, lora_ranks, scalings, y, ldy, nullptr,
                        workspace, workspace_bytes, stream);
}

size_t lora_shrink_expand_workspace_size(lora_dtype dtype, int64_t T, int64_t K, int32_t S,
                                         int32_t R, int32_t G, int64_t N) {
  (void)N;
  if (T <= 0 || G <= 0 || K <= 0 || S <= 0 || R <= 0 || !valid_dtype(dtype)) return 0;
  const PairWs w = pair_ws(int(dtype), T, K, S, R, G);
  return std::max(std::max(w.single_total, w.two_total), kCounterBytes);
}

lora_status lora_shrink_expand(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                               int32_t L, int32_t G, int64_t N, const void* x, int64_t ldx,
                               const void* w_a, int64_t lda, const void* w_b, int64_t ldb,
                               const int32_t* slice_offsets, const int32_t* seg_indptr,
                               const int32_t* weight_indices, const int32_t* permutation,
                               const int32_t* lora_ranks, const float* scalings, void* h,
                               int64_t ldh, void* y, int64_t ldy, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return LORA_EUNSUPPORTED;
  if (T < 0 || G < 0 || S < 1 || R < 1 || N < 0) return LORA_EINVAL;
  if (T == 0 || G == 0) return LORA_OK;
  if (K < 1 || L < 1) return LORA_EINVAL;
  const size_t need = lora_shrink_expand_workspace_size(dtype, T, K, S, R, G, N);
  if (workspace == nullptr || workspace_bytes < need || !al16(workspace)) return LORA_EWORKSPACE;
  const PairWs w = pair_ws(int(dtype), T, K, S, R, G);
  const int e = esize(dtype);
  const bool aligned_x = al16(x) && al16(w_a) && (ldx * e) % 16 == 0 && (lda * e) % 16 == 0;
  const bool aligned_b = al16(h) && al16(w_b) && (ldh * e) % 16 == 0 && (ldb * e) % 16 == 0 &&
                         (int64_t(R) * e) % 16 == 0;
  const bool aligned_y = al16(y) && (ldy * e) % 16 == 0;
  char* wsb = static_cast<char*>(workspace);
  // Column blocks of the single launch's expand workgroups (8 waves of 64-column chunks): the
  // library's usual width, widened until the shrink and expand grids are resident together (two
  // 512-thread workgroups per compute unit). Where even the widest blocks leave workgroups for a
  // second round, those would start their loads only after the shrink (1000 tokens: 34.6 us
  // against 29.3 us for two launches, cold calls), so the call makes two launches instead.
  const ShrinkWs& ws = w.sw;
  int bn = 0;
  bool single = w.shape_ok && aligned_x && aligned_b && N > 0;
  if (single) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return LORA_EHIP;
    const int64_t swgs = int64_t(ws.grid_x) * ws.gy;
    bn = expand_bn(Knobs{}, T, G, S, N, 16, 8, 64, false);
    while (bn < 4096 && swgs + ws.bound * (cdiv(N, bn) + S) > 2 * int64_t(cus)) bn += 512;
    single = swgs + ws.bound * (cdiv(N, bn) + S) <= 2 * int64_t(cus);
  }
  if (!single) {
    // two launches, exactly lora_shrink then lora_expand
    const lora_status st = lora_shrink(dtype, T, K, S, R, L, G, x, ldx, w_a, lda, seg_indptr,
                                       weight_indices, permutation, lora_ranks, h, ldh, workspace,
                                       w.expand_off, stream);
    if (st != LORA_OK) return st;
    return lora_expand(dtype, T, S, R, L, G, N, h, ldh, w_b, ldb, slice_offsets, seg_indptr,
                       weight_indices, permutation, lora_ranks, scalings, y, ldy,
                       wsb + w.expand_off, workspace_bytes - w.expand_off, stream);
  }
  // the argument checks of both calls
  if (S > kMaxSlices || R > kMaxRank) return LORA_EUNSUPPORTED;
  if (T >= INT_MAX || K >= INT_MAX || N >= INT_MAX / 2 || G >= INT_MAX / 2)
    return LORA_EUNSUPPORTED;
  if (!x || !w_a || !w_b || !slice_offsets || !seg_indptr || !weight_indices || !lora_ranks ||
      !scalings || !h || !y)
    return LORA_EINVAL;
  if (ldx < K || lda < K || ldh < int64_t(S) * R || ldb < R || ldy < N) return LORA_EINVAL;
  if (int64_t(S) * R * T * 16 >= int64_t(1) << 62) return LORA_EUNSUPPORTED;
  if (cdiv(N, bn) + S > 65535) return LORA_EUNSUPPORTED;

  lmx::ShrinkArgs a{};
  a.x = x; a.w_a = w_a; a.seg_indptr = seg_indptr; a.weight_indices = weight_indices;
  a.permutation = permutation; a.lora_ranks = lora_ranks; a.h = h;
  a.K = K; a.ldx = ldx; a.lda = lda; a.ldh = ldh; a.S = S; a.R = R; a.G = G; a.T = int(T);
  a.sk_q = ws.q; a.sk_tiles = int(ws.bound); a.sk_mp = ws.mp; a.sk_unit = ws.unit;
  a.part = reinterpret_cast<float*>(wsb + ws.part);
  a.counters = reinterpret_cast<int*>(wsb);
  a.ctr_shift = kPairCounterShift;
  lmx::ExpandArgs b{};
  b.h = h; b.w_b = w_b; b.slice_offsets = slice_offsets; b.seg_indptr = seg_indptr;
  b.weight_indices = weight_indices; b.permutation = permutation; b.lora_ranks = lora_ranks;
  b.scalings = scalings; b.y = y;
  b.N = N; b.ldh = ldh; b.ldb = ldb; b.ldy = ldy; b.S = S; b.R = R; b.G = G; b.BN = bn;
  lmx::PairArgs pa{};
  pa.sgx = ws.grid_x;
  pa.sgy = ws.gy;
  pa.shrink_wgs = pa.sgx * pa.sgy;
  pa.egx = int(ws.bound);
  pa.egy = int(cdiv(N, bn) + S);
  pa.done = reinterpret_cast<int*>(wsb + kPairDoneOffset);
  pa.err = reinterpret_cast<int*>(wsb + kPairFlagOffset);
  return hip_status(lmx::launch_pair(int(dtype), a, b, pa, K % 32 == 0, aligned_y,
                                     reinterpret_cast<hipStream_t>(stream)));
}

size_t lora_mlp_workspace_size(lora_dtype dtype, int64_t M, int64_t H, int64_t I, int32_t r) {
  (void)dtype;
  if (M <= 0 || H <= 0 || I <= 0 || r <= 0) return 0;
  return mlp_layout(M, H, I, r).total;
}

lora_status lora_mlp_fused(lora_dtype dtype, int64_t M, int64_t H, int64_t I, int32_t r,
                           float scale, const void* x, int64_t ldx, const void* w_gate,
                           const void* w_up, const void* w_down, const void* a_gate,
                           const void* b_gate, const void* a_up, const void* b_up,
                           const void* a_down, const void* b_down, void* out, int64_t ldo,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return mlp_forward(dtype, M, H, I, r, scale, x, ldx, w_gate, w_up, w_down, a_gate, b_gate, a_up,
                     b_up, a_down, b_down, out, ldo, nullptr, nullptr, 0, workspace,
                     workspace_bytes, stream);
}

lora_status lora_mlp_fused_train(lora_dtype dtype, int64_t M, int64_t H, int64_t I, int32_t r,
                                 float scale, const void* x, int64_t ldx, const void* w_gate,
                                 const void* w_up, const void* w_down, const void* a_gate,
                                 const void* b_gate, const void* a_up, const void* b_up,
                                 const void* a_down, const void* b_down, void* out, int64_t ldo,
                                 void* e, void* v, int64_t lde, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (M > 0 && (!e || !v)) return LORA_EINVAL;
  if (M > 0 && lde < I) return LORA_EINVAL;
  return mlp_forward(dtype, M, H, I, r, scale, x, ldx, w_gate, w_up, w_down, a_gate, b_gate, a_up,
                     b_up, a_down, b_down, out, ldo, e, v, lde, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

lora_status mlp_forward(lora_dtype dtype, int64_t M, int64_t H, int64_t I, int32_t r, float scale,
                        const void* x, int64_t ldx, const void* w_gate, const void* w_up,
                        const void* w_down, const void* a_gate, const void* b_gate,
                        const void* a_up, const void* b_up, const void* a_down,
                        const void* b_down, void* out, int64_t ldo, void* e_save, void* v_save,
                        int64_t lde, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != LORA_BF16) return LORA_EUNSUPPORTED;
  if (M < 0 || H < 1 || I < 1 || r < 1) return LORA_EINVAL;
  if (r > 64 || H % 32 != 0 || I % 32 != 0) return LORA_EUNSUPPORTED;
  if (M >= INT_MAX || H >= INT_MAX / 4 || I >= INT_MAX / 4) return LORA_EUNSUPPORTED;
  // the scaled LoRA-B copies ([2I][2 rp] and [H][rp], rp <= 64) are indexed with 32 bits
  if (int64_t(2 * I) * 128 + int64_t(H) * 64 >= int64_t(INT_MAX)) return LORA_EUNSUPPORTED;
  if (M == 0) return LORA_OK;
  if (!x || !w_gate || !w_up || !w_down || !a_gate || !b_gate || !a_up || !b_up || !a_down ||
      !b_down || !out)
    return LORA_EINVAL;
  if (ldx < H || ldo < H) return LORA_EINVAL;
  if (!al16(x) || (ldx * 2) % 16 != 0 || !al16(w_gate) || !al16(w_up) || !al16(w_down))
    return LORA_EUNSUPPORTED;
  const MlpLayout L = mlp_layout(M, H, I, r);
  if (workspace == nullptr || workspace_bytes < L.total || !al16(workspace)) return LORA_EWORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  uint16_t* xa_gu = reinterpret_cast<uint16_t*>(ws + L.xa_gu);
  uint16_t* lb_gu = reinterpret_cast<uint16_t*>(ws + L.lb_gu);
  uint16_t* hmid = reinterpret_cast<uint16_t*>(ws + L.hmid);
  uint16_t* xa_d = reinterpret_cast<uint16_t*>(ws + L.xa_d);
  uint16_t* lb_d = reinterpret_cast<uint16_t*>(ws + L.lb_d);
  const int64_t rp = L.rp;
  auto u16 = [](const void* p) { return static_cast<const uint16_t*>(p); };
  hipError_t e;
  // 1. scaled LoRA-B operands: [s B_g | 0] and [0 | s B_u] stacked, and s B_d
  {
    lmx::ScaleJobs jobs{};
    jobs.job[0] = {u16(b_gate), r, lb_gu, 2 * rp, int(I), 0};
    jobs.job[1] = {u16(b_up), r, lb_gu + I * 2 * rp, 2 * rp, int(I), int(rp)};
    jobs.job[2] = {u16(b_down), r, lb_d, rp, int(H), 0};
    if ((e = lmx::launch_scale_lora_b(jobs, scale, r, st)) != hipSuccess) return LORA_EHIP;
  }
  // LoRA-A operands for the sums kernel: in place, or zero-padded copies (rank rows past r)
  const int JB = L.gu.JB;
  const uint16_t *ag = u16(a_gate), *au = u16(a_up), *ad = u16(a_down);
  if (!lora_a_in_place(r, {a_gate, a_up, a_down})) {
    uint16_t* pad = reinterpret_cast<uint16_t*>(ws + L.apad);
    uint16_t *pg = pad, *pu = pad + int64_t(16 * JB) * H, *pd = pad + int64_t(16 * JB) * 2 * H;
    lmx::TJobs t{};
    t.n = 3;
    t.job[0] = {ag, H, pg, H, 16 * JB, int(H), 0, int(H), r, 1.0f, true};
    t.job[1] = {au, H, pu, H, 16 * JB, int(H), 0, int(H), r, 1.0f, true};
    t.job[2] = {ad, I, pd, I, 16 * JB, int(I), 0, int(I), r, 1.0f, true};
    if ((e = lmx::launch_small_transposes(t, st)) != hipSuccess) return LORA_EHIP;
    ag = pg; au = pu; ad = pd;
  }
  float* rowpart = reinterpret_cast<float*>(ws + L.rowpart);
  // h = round(P A^T) of rp padded columns (zeros past r) from the sums kernel's row side
  auto lora_a = [&](const lmx::SumJobs& plan, const uint16_t* P, int64_t ldp, int64_t C,
                    const uint16_t* A0, const uint16_t* A1, uint16_t* h, int64_t ldh) -> bool {
    lmx::SumJobs j = plan;
    j.job[0].P = P; j.job[0].ldp = ldp; j.job[0].ldr = C;
    j.job[0].R[0] = A0; j.job[0].R[1] = A1; j.job[0].R[2] = nullptr;
    if (lmx::launch_sums(j, rowpart, rowpart, st) != hipSuccess) return false;
    const int64_t rs = M * JB * 16;
    const int nc = j.blk0[1] - j.blk0[0];
    lmx::RedJobs rj{};
    rj.n = j.job[0].nr;
    rj.JB = JB;
    for (int q = 0; q < rj.n; ++q) {
      lmx::RedJob& o = rj.job[q];
      o.src = rowpart + j.job[0].rp0 + q * nc * rs; o.pstride = rs; o.np = nc;
      o.out = h + q * rp; o.osa = ldh; o.osj = 1; o.A = int(M); o.J = int(rp); o.r = r;
      o.scale = 1.0f;
    }
    return lmx::launch_reduce_sums(rj, st) == hipSuccess;
  };
  // 2. [xa_g | xa_u] = round(x [A_g; A_u]^T), ranks padded with zeros to rp (one pass over x)
  if (!lora_a(L.gu, u16(x), ldx, H, ag, au, xa_gu, 2 * rp)) return LORA_EHIP;
  // 3. hmid = round(silu(x W_g^T + s xa_g B_g^T) * (x W_u^T + s xa_u B_u^T))
  {
    lmx::GemmArgs g{};
    g.A = u16(x); g.lda = ldx; g.W0 = u16(w_gate); g.W1 = u16(w_up); g.ldw = H;
    g.A2 = xa_gu; g.lda2 = 2 * rp; g.B2 = lb_gu; g.ldb2 = 2 * rp;
    g.C = hmid; g.ldc = I; g.M = int(M); g.N = int(I); g.K = int(H); g.K2 = int(2 * rp);
    g.E = static_cast<uint16_t*>(e_save); g.V = static_cast<uint16_t*>(v_save); g.lde = lde;
    const int mode = e_save != nullptr ? lmx::kGemmSwigluSave : lmx::kGemmSwiglu;
    if ((e = lmx::launch_gemm_lora(g, mode, st)) != hipSuccess) return LORA_EHIP;
  }
  // 4. xa_d = round(hmid A_d^T)
  if (!lora_a(L.dn, hmid, I, I, ad, nullptr, xa_d, rp)) return LORA_EHIP;
  // 5. out = round(hmid W_d^T + s xa_d B_d^T)
  {
    lmx::GemmArgs g{};
    g.A = hmid; g.lda = I; g.W0 = u16(w_down); g.W1 = u16(w_down); g.ldw = I;
    g.A2 = xa_d; g.lda2 = rp; g.B2 = lb_d; g.ldb2 = rp;
    g.C = static_cast<uint16_t*>(out); g.ldc = ldo; g.M = int(M); g.N = int(H); g.K = int(I);
    g.K2 = int(rp);
    if ((e = lmx::launch_gemm_lora(g, lmx::kGemmPlain, st)) != hipSuccess) return LORA_EHIP;
  }
  return LORA_OK;
}

}  // namespace

extern "C" {

lora_status lora_mlp_prepare_backward(lora_dtype dtype, int64_t H, int64_t I, const void* w_gate,
                                      const void* w_up, const void* w_down, void* w_gu_t,
                                      void* w_down_t, void* stream) {
  if (dtype != LORA_BF16) return LORA_EUNSUPPORTED;
  if (H < 1 || I < 1) return LORA_EINVAL;
  if (H >= INT_MAX / 4 || I >= INT_MAX / 4) return LORA_EUNSUPPORTED;
  if (H > 65535 * 64 || I > 65535 * 64) return LORA_EUNSUPPORTED;  // transpose grid rows
  if (!w_gate || !w_up || !w_down || !w_gu_t || !w_down_t) return LORA_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  auto u16 = [](const void* p) { return static_cast<const uint16_t*>(p); };
  uint16_t* gu = static_cast<uint16_t*>(w_gu_t);
  // [W_g^T | W_u^T] as [H][2I], and W_d^T as [I][H]
  if (lmx::launch_transpose(u16(w_gate), H, gu, 2 * I, int(I), int(H), st) != hipSuccess ||
      lmx::launch_transpose(u16(w_up), H, gu + I, 2 * I, int(I), int(H), st) != hipSuccess ||
      lmx::launch_transpose(u16(w_down), I, static_cast<uint16_t*>(w_down_t), H, int(H), int(I),
                            st) != hipSuccess)
    return LORA_EHIP;
  return LORA_OK;
}

int32_t lora_mlp_backward_intermediates(int64_t M, int64_t H, int64_t I, int32_t r,
                                        size_t* offsets) {
  if (M <= 0 || H <= 0 || I <= 0 || r <= 0 || r > 64 || offsets == nullptr) return 0;
  const MlpBwdLayout L = mlp_bwd_layout(M, H, I, r);
  offsets[0] = L.hmid;
  offsets[1] = L.dedv;
  offsets[2] = L.xa_gu;
  offsets[3] = L.xa_d;
  offsets[4] = L.dxa_d;
  offsets[5] = L.dxa_gu;
  return int32_t(L.rp);
}

size_t lora_mlp_backward_workspace_size(lora_dtype dtype, int64_t M, int64_t H, int64_t I,
                                        int32_t r) {
  (void)dtype;
  if (M <= 0 || H <= 0 || I <= 0 || r <= 0 || r > 64) return 0;
  return mlp_bwd_layout(M, H, I, r).total;
}

lora_status lora_mlp_backward(lora_dtype dtype, int64_t M, int64_t H, int64_t I, int32_t r,
                              float scale, const void* x, int64_t ldx, const void* e_saved,
                              const void* v_saved, int64_t lde, const void* dout, int64_t lddo,
                              const void* w_gu_t, const void* w_down_t, const void* a_gate,
                              const void* b_gate, const void* a_up, const void* b_up,
                              const void* a_down, const void* b_down, void* dx, int64_t lddx,
                              void* da_gate, void* db_gate, void* da_up, void* db_up,
                              void* da_down, void* db_down, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (dtype != LORA_BF16) return LORA_EUNSUPPORTED;
  if (M < 0 || H < 1 || I < 1 || r < 1) return LORA_EINVAL;
  if (r > 64 || H % 32 != 0 || I % 32 != 0) return LORA_EUNSUPPORTED;
  if (M >= INT_MAX || H >= INT_MAX / 8 || I >= INT_MAX / 8) return LORA_EUNSUPPORTED;
  if (M == 0) return LORA_OK;
  if (!x || !e_saved || !v_saved || !dout || !w_gu_t || !w_down_t || !a_gate || !b_gate || !a_up ||
      !b_up || !a_down || !b_down || !dx || !da_gate || !db_gate || !da_up || !db_up || !da_down ||
      !db_down)
    return LORA_EINVAL;
  if (ldx < H || lde < I || lddo < H || lddx < H) return LORA_EINVAL;
  if (dx == x || dx == dout) return LORA_EINVAL;  // the saved input is never overwritten
  if (!al16(x) || (ldx * 2) % 16 != 0 || !al16(dout) || (lddo * 2) % 16 != 0 || !al16(w_gu_t) ||
      !al16(w_down_t) || !al16(e_saved) || !al16(v_saved) || (lde * 2) % 16 != 0)
    return LORA_EUNSUPPORTED;
  const MlpBwdLayout L = mlp_bwd_layout(M, H, I, r);
  if (workspace == nullptr || workspace_bytes < L.total || !al16(workspace)) return LORA_EWORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  auto W = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  auto u16 = [](const void* p) { return static_cast<const uint16_t*>(p); };
  const int rp = int(L.rp);
  uint16_t *sbdt = W(L.sbdt), *sbgt = W(L.sbgt), *sbut = W(L.sbut), *adt = W(L.adt);
  uint16_t *agut = W(L.agut), *xa_gu = W(L.xa_gu), *dxa_d = W(L.dxa_d), *xa_d = W(L.xa_d);
  uint16_t *dxa_gu = W(L.dxa_gu), *hmid = W(L.hmid), *dedv = W(L.dedv), *adp = W(L.adp);
  uint16_t *agp = W(L.agp), *aup = W(L.aup);
  float* rowpart = reinterpret_cast<float*>(ws + L.rowpart);
  float* colpart = reinterpret_cast<float*>(ws + L.colpart);
  auto sum_job = [](lmx::SumJob& j, const uint16_t* P, int64_t ldp, const uint16_t* R0,
                    const uint16_t* R1, const uint16_t* Q0, const uint16_t* Q1, int64_t ldq) {
    j.P = P; j.ldp = ldp; j.R[0] = R0; j.R[1] = R1; j.R[2] = nullptr; j.ldr = j.C;
    j.Q[0] = Q0; j.Q[1] = Q1; j.ldq = ldq;
  };
  auto red_job = [](lmx::RedJob& j, const float* src, int64_t pstride, int np, void* out,
                    int64_t osa, int64_t osj, int A, int J, int r, float sc) {
    j.src = src; j.pstride = pstride; j.np = np; j.out = static_cast<uint16_t*>(out);
    j.osa = osa; j.osj = osj; j.A = A; j.J = J; j.r = r; j.scale = sc;
  };
  const int JB = L.both.JB;
  auto ncb = [](const lmx::SumJobs& j, int q) { return j.blk0[q + 1] - j.blk0[q]; };
  // 1. operands, rank rows past r zero: s B_d^T [rp][H]; s B_g^T, s B_u^T, A_d [rp][I];
  //    A_g, A_u [rp][H]; A_d^T [I][rp]; [A_g^T | A_u^T] [H][2 rp]
  {
    lmx::TJobs t{};
    t.n = 9;
    t.job[0] = {u16(b_down), r, sbdt, H, rp, int(H), 0, int(H), r, scale, false};
    t.job[1] = {u16(b_gate), r, sbgt, I, rp, int(I), 0, int(I), r, scale, false};
    t.job[2] = {u16(b_up), r, sbut, I, rp, int(I), 0, int(I), r, scale, false};
    t.job[3] = {u16(a_down), I, adt, rp, int(I), rp, 0, r, int(I), 1.0f, false};
    t.job[4] = {u16(a_gate), H, agut, 2 * rp, int(H), rp, 0, r, int(H), 1.0f, false};
    t.job[5] = {u16(a_up), H, agut + rp, 2 * rp, int(H), rp, 0, r, int(H), 1.0f, false};
    t.job[6] = {u16(a_down), I, adp, I, rp, int(I), 0, int(I), r, 1.0f, true};
    t.job[7] = {u16(a_gate), H, agp, H, rp, int(H), 0, int(H), r, 1.0f, true};
    t.job[8] = {u16(a_up), H, aup, H, rp, int(H), 0, int(H), r, 1.0f, true};
    if (lmx::launch_small_transposes(t, st) != hipSuccess) return LORA_EHIP;
  }
  // 2. [xa_g | xa_u] = round(x [A_g; A_u]^T) and dxa_d = round(dout (s B_d)): sums over the
  //    columns of x and dout, then their fixed-order reduction (with the rank padding zeroed)
  {
    lmx::SumJobs j = L.in;
    sum_job(j.job[0], u16(x), ldx, agp, aup, nullptr, nullptr, 0);
    sum_job(j.job[1], u16(dout), lddo, sbdt, nullptr, nullptr, nullptr, 0);
    if (lmx::launch_sums(j, rowpart, colpart, st) != hipSuccess) return LORA_EHIP;
    const int64_t rs = M * JB * 16;
    const int nx = ncb(j, 0), nd = ncb(j, 1);
    lmx::RedJobs rj{};
    rj.n = 3;
    rj.JB = JB;
    red_job(rj.job[0], rowpart + j.job[0].rp0, rs, nx, xa_gu, 2 * rp, 1, int(M), rp, r, 1.0f);
    red_job(rj.job[1], rowpart + j.job[0].rp0 + nx * rs, rs, nx, xa_gu + rp, 2 * rp, 1, int(M), rp, r, 1.0f);
    red_job(rj.job[2], rowpart + j.job[1].rp0, rs, nd, dxa_d, rp, 1, int(M), rp, r, 1.0f);
    if (lmx::launch_reduce_sums(rj, st) != hipSuccess) return LORA_EHIP;
  }
  // 3. dhmid = dout W_d + dxa_d A_d with the SwiGLU backward in the epilogue:
  //    hmid = round(silu(e) v), de = round(dhmid v silu'(e)), dv = round(dhmid silu(e))
  {
    lmx::GemmArgs g{};
    g.A = u16(dout); g.lda = lddo; g.W0 = u16(w_down_t); g.W1 = u16(w_down_t); g.ldw = H;
    g.A2 = dxa_d; g.lda2 = rp; g.B2 = adt; g.ldb2 = rp;
    g.C = hmid; g.ldc = I;
    g.E = const_cast<uint16_t*>(u16(e_saved)); g.V = const_cast<uint16_t*>(u16(v_saved)); g.lde = lde;
    g.D = dedv; g.ldd = 2 * I;
    g.M = int(M); g.N = int(I); g.K = int(H); g.K2 = rp;
    if (lmx::launch_gemm_lora(g, lmx::kGemmSwigluBwd, st) != hipSuccess) return LORA_EHIP;
  }
  // 4. one pass over de, dv and hmid: the LoRA-A products of the next layer down the chain
  //    (dxa_g = de (s B_g), dxa_u = dv (s B_u), xa_d = hmid A_d^T: sums over columns) and the
  //    weight-gradient sums over tokens (dB_g = s de^T xa_g, dB_u = s dv^T xa_u,
  //    dA_d = dxa_d^T hmid), then their fixed-order reduction
  {
    lmx::SumJobs j = L.both;
    sum_job(j.job[0], dedv, 2 * I, sbgt, nullptr, xa_gu, nullptr, 2 * rp);
    sum_job(j.job[1], dedv + I, 2 * I, sbut, nullptr, xa_gu + rp, nullptr, 2 * rp);
    sum_job(j.job[2], hmid, I, adp, nullptr, dxa_d, nullptr, rp);
    if (lmx::launch_sums(j, rowpart, colpart, st) != hipSuccess) return LORA_EHIP;
    const int nc = ncb(j, 0);
    const int64_t rstride = M * JB * 16, cstride = I * JB * 16;
    lmx::RedJobs rj{};
    rj.n = 6;
    rj.JB = JB;
    red_job(rj.job[0], rowpart + j.job[0].rp0, rstride, nc, dxa_gu, 2 * rp, 1, int(M), rp, r, 1.0f);
    red_job(rj.job[1], rowpart + j.job[1].rp0, rstride, nc, dxa_gu + rp, 2 * rp, 1, int(M), rp, r, 1.0f);
    red_job(rj.job[2], rowpart + j.job[2].rp0, rstride, nc, xa_d, rp, 1, int(M), rp, r, 1.0f);
    red_job(rj.job[3], colpart + j.job[0].cp0, cstride, j.chunks, db_gate, r, 1, int(I), r, r, scale);
    red_job(rj.job[4], colpart + j.job[1].cp0, cstride, j.chunks, db_up, r, 1, int(I), r, r, scale);
    red_job(rj.job[5], colpart + j.job[2].cp0, cstride, j.chunks, da_down, 1, I, int(I), r, r, 1.0f);
    if (lmx::launch_reduce_sums(rj, st) != hipSuccess) return LORA_EHIP;
  }
  // 5. sums over tokens of x and dout: dA_g = dxa_g^T x, dA_u = dxa_u^T x, dB_d = s dout^T xa_d
  {
    lmx::SumJobs j = L.cols;
    sum_job(j.job[0], u16(x), ldx, nullptr, nullptr, dxa_gu, dxa_gu + rp, 2 * rp);
    sum_job(j.job[1], u16(dout), lddo, nullptr, nullptr, xa_d, nullptr, rp);
    if (lmx::launch_sums(j, rowpart, colpart, st) != hipSuccess) return LORA_EHIP;
    const int64_t cstride = H * JB * 16, hstride = int64_t(j.chunks) * cstride;
    lmx::RedJobs rj{};
    rj.n = 3;
    rj.JB = JB;
    red_job(rj.job[0], colpart + j.job[0].cp0, cstride, j.chunks, da_gate, 1, H, int(H), r, r, 1.0f);
    red_job(rj.job[1], colpart + j.job[0].cp0 + hstride, cstride, j.chunks, da_up, 1, H, int(H), r, r, 1.0f);
    red_job(rj.job[2], colpart + j.job[1].cp0, cstride, j.chunks, db_down, r, 1, int(H), r, r, scale);
    if (lmx::launch_reduce_sums(rj, st) != hipSuccess) return LORA_EHIP;
  }
  // 6. dx = round(de W_g + dv W_u + dxa_g A_g + dxa_u A_u)
  {
    lmx::GemmArgs g{};
    g.A = dedv; g.lda = 2 * I; g.W0 = u16(w_gu_t); g.W1 = u16(w_gu_t); g.ldw = 2 * I;
    g.A2 = dxa_gu; g.lda2 = 2 * rp; g.B2 = agut; g.ldb2 = 2 * rp;
    g.C = static_cast<uint16_t*>(dx); g.ldc = lddx;
    g.M = int(M); g.N = int(H); g.K = int(2 * I); g.K2 = 2 * rp;
    if (lmx::launch_gemm_lora(g, lmx::kGemmPlain, st) != hipSuccess) return LORA_EHIP;
  }
  return LORA_OK;
}

lora_status lora_linear_prepare_backward(lora_dtype dtype, int64_t K, int64_t N, const void* w,
                                         void* w_t, void* stream) {
  if (dtype != LORA_BF16) return LORA_EUNSUPPORTED;
  if (K < 1 || N < 1) return LORA_EINVAL;
  if (K >= INT_MAX / 4 || N >= INT_MAX / 4) return LORA_EUNSUPPORTED;
  if (K > 65535 * 64 || N > 65535 * 64) return LORA_EUNSUPPORTED;  // transpose grid rows
  if (!w || !w_t) return LORA_EINVAL;
  // W^T as [K][N]
  return hip_status(lmx::launch_transpose(static_cast<const uint16_t*>(w), K,
                                          static_cast<uint16_t*>(w_t), N, int(N), int(K),
                                          reinterpret_cast<hipStream_t>(stream)));
}

size_t lora_linear_backward_workspace_size(lora_dtype dtype, int64_t M, int64_t K, int64_t N,
                                           int32_t r) {
  if (dtype != LORA_BF16 || M <= 0 || K <= 0 || N <= 0 || r <= 0 || r > 64) return 0;
  return lin_bwd_layout(M, K, &N, 1, r).total;
}

lora_status lora_linear_backward(lora_dtype dtype, int64_t M, int64_t K, int64_t N, int32_t r,
                                 float scale, const void* x, int64_t ldx, const void* dout,
                                 int64_t lddo, const void* w_t, const void* a, const void* b,
                                 void* dx, int64_t lddx, void* da, void* db, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const void* d[1] = {dout};
  const int64_t ld[1] = {lddo};
  const void* aa[1] = {a};
  const void* bb[1] = {b};
  void* dda[1] = {da};
  void* ddb[1] = {db};
  return linear_backward(dtype, M, K, &N, 1, r, scale, x, ldx, d, ld, w_t, aa, bb, dx, lddx, dda,
                         ddb, workspace, workspace_bytes, stream);
}

lora_status lora_qkv_prepare_backward(lora_dtype dtype, int64_t K, int64_t Nq, int64_t Nkv,
                                      const void* w_q, const void* w_k, const void* w_v,
                                      void* w_qkv_t, void* stream) {
  if (dtype != LORA_BF16) return LORA_EUNSUPPORTED;
  if (K < 1 || Nq < 1 || Nkv < 1) return LORA_EINVAL;
  if (K >= INT_MAX / 4 || Nq >= INT_MAX / 8 || Nkv >= INT_MAX / 8) return LORA_EUNSUPPORTED;
  if (K > 65535 * 64 || Nq > 65535 * 64 || Nkv > 65535 * 64) return LORA_EUNSUPPORTED;
  if (!w_q || !w_k || !w_v || !w_qkv_t) return LORA_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  auto u16 = [](const void* q) { return static_cast<const uint16_t*>(q); };
  uint16_t* t = static_cast<uint16_t*>(w_qkv_t);
  const int64_t ntot = Nq + 2 * Nkv;
  // [W_q^T | W_k^T | W_v^T] as [K][Nq + 2 Nkv]
  if (lmx::launch_transpose(u16(w_q), K, t, ntot, int(Nq), int(K), st) != hipSuccess ||
      lmx::launch_transpose(u16(w_k), K, t + Nq, ntot, int(Nkv), int(K), st) != hipSuccess ||
      lmx::launch_transpose(u16(w_v), K, t + Nq + Nkv, ntot, int(Nkv), int(K), st) != hipSuccess)
    return LORA_EHIP;
  return LORA_OK;
}

size_t lora_qkv_backward_workspace_size(lora_dtype dtype, int64_t M, int64_t K, int64_t Nq,
                                        int64_t Nkv, int32_t r) {
  if (dtype != LORA_BF16 || M <= 0 || K <= 0 || Nq <= 0 || Nkv <= 0 || r <= 0 || r > 64) return 0;
  const int64_t N[3] = {Nq, Nkv, Nkv};
  return lin_bwd_layout(M, K, N, 3, r).total;
}

lora_status lora_qkv_backward(lora_dtype dtype, int64_t M, int64_t K, int64_t Nq, int64_t Nkv,
                              int32_t r, float scale, const void* x, int64_t ldx, const void* dq,
                              int64_t lddq, const void* dk, int64_t lddk, const void* dv,
                              int64_t lddv, const void* w_qkv_t, const void* a_q, const void* b_q,
                              const void* a_k, const void* b_k, const void* a_v, const void* b_v,
                              void* dx, int64_t lddx, void* da_q, void* db_q, void* da_k,
                              void* db_k, void* da_v, void* db_v, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const int64_t N[3] = {Nq, Nkv, Nkv};
  const void* d[3] = {dq, dk, dv};
  const int64_t ld[3] = {lddq, lddk, lddv};
  const void* aa[3] = {a_q, a_k, a_v};
  const void* bb[3] = {b_q, b_k, b_v};
  void* dda[3] = {da_q, da_k, da_v};
  void* ddb[3] = {db_q, db_k, db_v};
  return linear_backward(dtype, M, K, N, 3, r, scale, x, ldx, d, ld, w_qkv_t, aa, bb, dx, lddx,
                         dda, ddb, workspace, workspace_bytes, stream);
}

size_t lora_linear_workspace_size(lora_dtype dtype, int64_t M, int64_t K, int64_t N, int32_t r) {
  (void)dtype;
  if (M <= 0 || K <= 0 || N <= 0 || r <= 0) return 0;
  const int64_t n[1] = {N};
  return linear_layout(M, K, n, 1, r).total;
}

lora_status lora_linear_fused(lora_dtype dtype, int64_t M, int64_t K, int64_t N, int32_t r,
                              float scale, const void* x, int64_t ldx, const void* w,
                              const void* a, const void* b, void* out, int64_t ldo,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const int64_t n[1] = {N}, ld[1] = {ldo};
  const void* ws[1] = {w};
  const void* as[1] = {a};
  const void* bs[1] = {b};
  void* os[1] = {out};
  return linear_fused(dtype, M, K, n, 1, r, scale, x, ldx, ws, as, bs, os, ld, workspace,
                      workspace_bytes, stream);
}

size_t lora_qkv_workspace_size(lora_dtype dtype, int64_t M, int64_t K, int64_t Nq, int64_t Nkv,
                               int32_t r) {
  (void)dtype;
  if (M <= 0 || K <= 0 || Nq <= 0 || Nkv <= 0 || r <= 0) return 0;
  const int64_t n[3] = {Nq, Nkv, Nkv};
  return linear_layout(M, K, n, 3, r).total;
}

lora_status lora_qkv_fused(lora_dtype dtype, int64_t M, int64_t K, int64_t Nq, int64_t Nkv,
                           int32_t r, float scale, const void* x, int64_t ldx, const void* w_q,
                           const void* w_k, const void* w_v, const void* a_q, const void* b_q,
                           const void* a_k, const void* b_k, const void* a_v, const void* b_v,
                           void* q, int64_t ldq, void* k, int64_t ldk, void* v, int64_t ldv,
                           void* workspace, size_t workspace_bytes, void* stream) {
  const int64_t n[3] = {Nq, Nkv, Nkv}, ld[3] = {ldq, ldk, ldv};
  const void* ws[3] = {w_q, w_k, w_v};
  const void* as[3] = {a_q, a_k, a_v};
  const void* bs[3] = {b_q, b_k, b_v};
  void* os[3] = {q, k, v};
  return linear_fused(dtype, M, K, n, 3, r, scale, x, ldx, ws, as, bs, os, ld, workspace,
                      workspace_bytes, stream);
}

lora_status lora_embedding_a(lora_dtype dtype, int64_t T, int64_t V, int32_t R, int32_t L,
                             int32_t G, const int32_t* input_ids, const void* w_a,
                             int64_t stride_l, int64_t stride_r, int64_t stride_v,
                             const int32_t* seg_indptr, const int32_t* weight_indices,
                             const int32_t* permutation, const int32_t* lora_ranks, void* h,
                             int64_t ldh, void* stream) {
  if (!valid_dtype(dtype)) return LORA_EUNSUPPORTED;
  if (T < 0 || G < 0 || R < 1 || V < 1) return LORA_EINVAL;
  if (R > kMaxRank) return LORA_EUNSUPPORTED;
  if (T == 0 || G == 0) return LORA_OK;
  if (L < 1) return LORA_EINVAL;
  if (T > INT_MAX - 512 || G >= INT_MAX || V >= INT_MAX) return LORA_EUNSUPPORTED;
  if (!input_ids || !w_a || !seg_indptr || !weight_indices || !lora_ranks || !h) return LORA_EINVAL;
  if (stride_l < 0 || stride_r < 1 || stride_v < 1 || ldh < R) return LORA_EINVAL;
  lmx::EmbeddingArgs a{};
  a.input_ids = input_ids; a.w_a = w_a; a.seg_indptr = seg_indptr; a.weight_indices = weight_indices;
  a.permutation = permutation; a.lora_ranks = lora_ranks; a.h = h;
  a.stride_l = stride_l; a.stride_r = stride_r; a.stride_v = stride_v; a.ldh = ldh;
  a.T = int(T); a.R = R; a.G = G; a.L = L; a.V = int(V);
  const int es = esize(dtype), ve = 16 / es;
  const bool vec = stride_r == 1 && R % ve == 0 && ldh % ve == 0 && stride_v % ve == 0 &&
                   stride_l % ve == 0 && al16(w_a) && al16(h);
  return hip_status(lmx::launch_embedding_a(a, es, vec, reinterpret_cast<hipStream_t>(stream)));
}

size_t lora_check_metadata_workspace_size(int64_t T) {
  return T < 0 ? 0 : 256 + size_t(T) * 4;
}

lora_status lora_check_metadata(int64_t T, int32_t G, int32_t L, int32_t R, int32_t S, int64_t N,
                                const int32_t* seg_indptr, const int32_t* weight_indices,
                                const int32_t* permutation, const int32_t* lora_ranks,
                                const int32_t* slice_offsets, int32_t* rule, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (rule != nullptr) *rule = 0;
  if (T < 0 || G < 0 || L < 0 || R < 0 || S < 0 || N < 0) return LORA_EINVAL;
  if (T >= INT_MAX || G >= INT_MAX - 1 || S >= INT_MAX - 1 || N >= INT_MAX) return LORA_EUNSUPPORTED;
  if (!seg_indptr || (G > 0 && !weight_indices) || (L > 0 && !lora_ranks)) return LORA_EINVAL;
  if (workspace == nullptr || workspace_bytes < lora_check_metadata_workspace_size(T) ||
      !al16(workspace))
    return LORA_EWORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  lmx::MetaArgs a{};
  a.seg_indptr = seg_indptr; a.weight_indices = weight_indices; a.permutation = permutation;
  a.lora_ranks = lora_ranks; a.slice_offsets = slice_offsets; a.N = N;
  a.T = int(T); a.G = G; a.L = L; a.R = R; a.S = S;
  int* flag = static_cast<int*>(workspace);
  int* counts = reinterpret_cast<int*>(static_cast<char*>(workspace) + 256);
  if (lmx::launch_metadata_check(a, flag, counts, st) != hipSuccess) return LORA_EHIP;
  int bits = 0;
  if (hipMemcpyAsync(&bits, flag, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return LORA_EHIP;
  for (int k = 1; k <= 5; ++k) {
    if (bits & (1 << k)) {
      if (rule != nullptr) *rule = k;
      return LORA_EVALUE;
    }
  }
  return LORA_OK;
}

lora_status lora_schedule_tiles(int64_t T, int32_t G, int32_t BM, int32_t method,
                                const int32_t* seg_indptr, const int32_t* weight_indices,
                                const int32_t* lora_ranks, int32_t* tiles, int64_t max_tiles,
                                int32_t* count, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (T < 0 || G < 0 || BM < 1 || BM > 4096 || (method != 0 && method != 1)) return LORA_EINVAL;
  if (!count || !tiles || !seg_indptr || !weight_indices || !lora_ranks) return LORA_EINVAL;
  if (T >= INT_MAX || G >= INT_MAX / 2) return LORA_EUNSUPPORTED;
  const int64_t bound = cdiv(T, BM) + G;
  if (max_tiles < bound) return LORA_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t need = size_t(bound) * 16 + 256;
  if (method == 1 && (workspace == nullptr || workspace_bytes < need)) return LORA_EWORKSPACE;
  if (bound == 0 || G == 0) {
    return hip_status(lmx::launch_zero_int(count, st));
  }
  int4* ws_tiles = method == 1 ? reinterpret_cast<int4*>(static_cast<char*>(workspace) + 256) : nullptr;
  int* ws_count = method == 1 ? static_cast<int*>(workspace) : nullptr;
  return hip_status(lmx::launch_export_tiles(method, seg_indptr, weight_indices, lora_ranks, G, BM,
                                             int(bound), tiles, count, ws_tiles, ws_count, st));
}

}  // extern "C"
