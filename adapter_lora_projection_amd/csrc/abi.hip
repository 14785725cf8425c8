// C ABI of the library: argument validation, kernel-shape selection and launches.
// Every check here runs on the host before anything is enqueued; nothing reads device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>

#include "../../include/lora_mi355x.h"
#include "embedding.hpp"
#include "metadata_check.hpp"
#include "mlp_kernels.hpp"
#include "sgmv_kernels.hpp"

namespace {

constexpr int kInlineMaxSegments = 1024;  // above this the standalone scheduler builds the list
constexpr int kMaxSlices = 64;
constexpr int kMaxRank = 1024;

int g_shrink_override = -1;
int g_lds_override = -1;  // shrink kernel family: 0 = register ring, 1 = LDS-staged where eligible
int g_sk_override = -1;  // shrink workgroups along x in stream-K mode; 0 = direct mode
int g_expand_override = -1;
int g_expand_bn_override = -1;

bool valid_dtype(int d) { return d == LORA_F32 || d == LORA_BF16 || d == LORA_F16; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int esize(int dtype) { return dtype == LORA_F32 ? 4 : 2; }

// Columns per expand workgroup, in multiples of the 64-column chunks the waves walk: the widest
// blocks (up to 4096 columns) that still give about 400 workgroups. Longer column runs per wave
// measured faster than more workgroups once the chip is covered (rocprofv3 sweeps on MI355X).
// The shared-B kernel (three 256-thread workgroups resident per compute unit, 768 on the chip)
// also takes at least 600 / tiles blocks: more blocks than that leave a second round of
// workgroups (8192 tokens: 660 workgroups 55.7 us, 792 workgroups 63.6 us), fewer leave the
// chip half idle (6144 tokens: 500 workgroups 44.0 us, 600 workgroups 40.6 us).
int expand_bn(int64_t T, int32_t G, int64_t N, int bm, int waves, int chunk, bool shared) {
  const int unit = chunk * waves;
  if (g_expand_bn_override > 0) return int(cdiv(g_expand_bn_override, unit) * unit);
  const int64_t tiles = cdiv(T, bm) + G;
  int64_t blocks = std::max<int64_t>(1, cdiv(400, tiles));
  if (shared) blocks = std::max<int64_t>(blocks, 600 / tiles);
  int64_t bn = cdiv(cdiv(N, blocks), unit) * unit;
  bn = std::min<int64_t>(std::max<int64_t>(bn, unit), 4096);
  return int(bn);
}

// Kernel shape for a shrink call, from host-known sizes only (rocprofv3 sweeps on MI355X over
// the decode sweep, prefill and irregular workloads). Small token counts: one token group and
// one 16-column block per workgroup, 8 waves splitting K. Otherwise two token groups per
// workgroup sharing each A fragment, over 3 column blocks, or 4 when the slices have 4 or fewer
// blocks that 3 does not divide. The 2-deep operand ring measured faster than 4-deep.
int shrink_variant(int64_t T, int32_t S, int32_t R) {
  if (g_shrink_override >= 0) return g_shrink_override;
  const int64_t nblk = int64_t(S) * ((R + 15) / 16);
  if (nblk % 3 == 0) return T <= 2048 ? 2 : 4;
  return nblk <= 4 ? 1 : 4;
}

// Shrink launch plan and workspace: [0, sched) the standalone scheduler's tile list (only for
// many segments), then the stream-K partial planes. Stream-K gives every compute unit an equal
// share of the (tile, reduction step) work, about one workgroup per compute unit.
struct ShrinkWs {
  bool lds;          // LDS-staged kernel (else the register-ring kernel)
  int variant, bm, grid_x, mp, unit;
  int64_t bound, q;  // tile bound; stream-K units per workgroup (0 = direct mode)
  size_t sched, part, total;
};

// Expand kernel shape (rocprofv3 sweeps and event timings on MI355X). From 1024 tokens, slices of
// rank exactly 16 with 16-bit types and 16-byte aligned h, B and y rows take the shared-B kernel
// (8192 tokens: 62 -> 56 us; 1024: 17.6 -> 16.7 us). Otherwise 4 waves with a 2-deep ring of y
// and B chunks up to 1024 tokens, and from 2048 tokens 128-column chunks with 16-byte y pieces
// and a 1-deep ring (fewer bytes in flight per compute unit measured faster than deeper rings;
// the wide chunks saved 3-12% at 2048..6144 tokens). Blocks whose y rows or start are not
// 16-byte aligned take the 8-byte form inside the same launch.
int expand_variant(int64_t T, bool shared_ok) {
  if (g_expand_override >= 0) {
    const bool shared = g_expand_override == lmx::kExpandSharedD1 ||
                        g_expand_override == lmx::kExpandSharedD2;
    return (shared && !shared_ok) ? 6 : g_expand_override;
  }
  if (shared_ok && T >= 1024) return lmx::kExpandSharedD1;
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
int shrink_lds_variant(int32_t S, int32_t R) {
  if (g_shrink_override >= 0 && g_shrink_override < lmx::num_shrink_lds_variants())
    return g_shrink_override;
  const int64_t nblk = int64_t(S) * ((R + 15) / 16);
  for (int v = 0; v < lmx::num_shrink_lds_variants(); ++v)
    if (lmx::shrink_lds_ncb(v) >= nblk) return v;
  return lmx::num_shrink_lds_variants() - 1;
}

// Which shrink kernel to run when the LDS-staged one is eligible (rocprofv3 sweeps on MI355X):
// it pays for its shared-work second launch when every compute unit streams a lot of x
// (T * K at least 16 Mi elements: decode tok >= 4096, prefill down-proj, the MLP's LoRA-A)
// and the slices have few column blocks; the register-ring kernel is faster below that.
bool prefer_lds(int64_t T, int64_t K, int32_t S, int32_t R) {
  if (g_lds_override >= 0) return g_lds_override == 1;
  const int64_t nblk = int64_t(S) * ((R + 15) / 16);
  return T * K >= (int64_t(16) << 20) && nblk <= 4;
}

ShrinkWs shrink_ws(int dtype, int64_t T, int64_t K, int32_t S, int32_t R, int32_t G, bool lds) {
  ShrinkWs w{};
  w.lds = lds;
  const int64_t nblk = int64_t(S) * ((R + 15) / 16);
  int64_t gy, frags;
  if (lds) {
    w.variant = shrink_lds_variant(S, R);
    w.bm = lmx::kShrinkLdsBM;
    w.unit = lmx::kShrinkLdsUnit;
    gy = cdiv(nblk, lmx::shrink_lds_ncb(w.variant));
    frags = (w.bm + 16 * lmx::shrink_lds_ncb(w.variant)) / 8;  // 1 KiB loads per stage
  } else {
    w.variant = shrink_variant(T, S, R);
    w.bm = lmx::shrink_plan_bm(dtype, w.variant);
    w.unit = dtype == LORA_F32 ? 16 : 32;
    gy = cdiv(nblk, lmx::shrink_plan_cb(dtype, w.variant));
    frags = w.bm / 16 + lmx::shrink_plan_cb(dtype, w.variant);  // 1 KiB loads per step
  }
  w.bound = cdiv(T, w.bm) + G;
  const int64_t nsteps = cdiv(K, w.unit);
  // Shared (tile, step) work pays for its second launch only when one workgroup per tile leaves
  // half the compute units idle and each workgroup would stream a lot.
  // (The LDS-staged kernel is chosen only for such problems: it always shares when its tiles
  // leave compute units idle.)
  const int64_t direct_wgs = w.bound * gy;
  const bool shared = lds ? direct_wgs < 256
                          : direct_wgs < 128 && nsteps * frags * 1024 >= (int64_t(512) << 10);
  const int64_t P = g_sk_override >= 0 ? g_sk_override : (shared ? std::max<int64_t>(1, 256 / gy) : 0);
  w.sched = schedule_bytes(T, G, w.bm);
  w.part = align256(w.sched);
  if (P == 0) {
    w.q = 0;
    w.grid_x = int(w.bound);
    w.total = w.sched;
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
struct MlpLayout {
  int64_t rp;           // rank rounded up to 32
  ShrinkWs s_gu, s_d;   // plans of the two LoRA-A products (dense mode, one segment)
  ShrinkWs r_gu, r_d;   // the same with the register-ring kernel (unaligned A pointers)
  size_t xa_gu, lb_gu, hmid, xa_d, lb_d, part, total;
};

MlpLayout mlp_layout(int64_t M, int64_t H, int64_t I, int32_t r) {
  MlpLayout L{};
  L.rp = cdiv(r, 32) * 32;
  // dense mode has no segments: the tile bound is ceil(M / BM)
  // plans for both shrink families (the LDS-staged one needs aligned A pointers, known only
  // at call time); the partials section fits either
  L.s_gu = shrink_ws(LORA_BF16, M, H, 2, int(L.rp), 0, prefer_lds(M, H, 2, int(L.rp)));
  L.s_d = shrink_ws(LORA_BF16, M, I, 1, int(L.rp), 0, prefer_lds(M, I, 1, int(L.rp)));
  L.r_gu = shrink_ws(LORA_BF16, M, H, 2, int(L.rp), 0, false);
  L.r_d = shrink_ws(LORA_BF16, M, I, 1, int(L.rp), 0, false);
  size_t off = 0;
  L.xa_gu = off; off += align256(size_t(M) * 2 * L.rp * 2);
  L.lb_gu = off; off += align256(size_t(2 * I) * 2 * L.rp * 2);
  L.hmid = off; off += align256(size_t(M) * I * 2);
  L.xa_d = off; off += align256(size_t(M) * L.rp * 2);
  L.lb_d = off; off += align256(size_t(H) * L.rp * 2);
  L.part = off;
  off += align256(std::max(std::max(L.s_gu.total - L.s_gu.part, L.s_d.total - L.s_d.part),
                           std::max(L.r_gu.total - L.r_gu.part, L.r_d.total - L.r_d.part)));
  L.total = off;
  return L;
}

// Workspace of the LoRA linear projections (P = 1 or 3 projections of one x): byte offsets of
// [xa [M][P rp]], the scaled LoRA-B copies [N_p][rp] and the shrink partials.
struct LinearLayout {
  int64_t rp;
  int P;
  ShrinkWs s, r;  // LoRA-A product plans: LDS-staged / register-ring (unaligned A pointers)
  size_t xa, lb[3], part, total;
};

LinearLayout linear_layout(int64_t M, int64_t K, const int64_t* N, int P, int32_t r) {
  LinearLayout L{};
  L.rp = cdiv(r, 32) * 32;
  L.P = P;
  L.s = shrink_ws(LORA_BF16, M, K, P, int(L.rp), 0, prefer_lds(M, K, P, int(L.rp)));
  L.r = shrink_ws(LORA_BF16, M, K, P, int(L.rp), 0, false);
  size_t off = 0;
  L.xa = off; off += align256(size_t(M) * P * L.rp * 2);
  for (int p = 0; p < P; ++p) { L.lb[p] = off; off += align256(size_t(N[p]) * L.rp * 2); }
  L.part = off;
  off += align256(std::max(L.s.total - L.s.part, L.r.total - L.r.part));
  L.total = off;
  return L;
}

lora_status mlp_forward(lora_dtype dtype, int64_t M, int64_t H, int64_t I, int32_t r, float scale,
                        const void* x, int64_t ldx, const void* w_gate, const void* w_up,
                        const void* w_down, const void* a_gate, const void* b_gate,
                        const void* a_up, const void* b_up, const void* a_down,
                        const void* b_down, void* out, int64_t ldo, void* e_save, void* v_save,
                        int64_t lde, void* workspace, size_t workspace_bytes, void* stream);

// Workspace of the LoRA MLP backward: byte offsets of the transposed / scaled LoRA operands, the
// recomputed LoRA-A products, the gradient intermediates and the partial sums.
struct MlpBwdLayout {
  int64_t rp;
  ShrinkWs s_x, r_x;   // [xa_g | xa_u] from x (plans for aligned / unaligned A)
  ShrinkWs s_w;        // products against operands in the workspace (always aligned): K = H
  ShrinkWs s_i, r_i;   // products over K = I (xa_d from hmid; dxa_g, dxa_u from de, dv)
  lmx::ColJobs cj;     // geometry of the sums over tokens (pointers set at call time)
  size_t sbdt, sbgt, sbut, adt, agut, xa_gu, dxa_d, xa_d, dxa_gu, hmid, dedv, part, colpart, total;
};

lmx::ColJobs mlp_bwd_coljobs(int64_t M, int64_t H, int64_t I, int32_t r) {
  lmx::ColJobs j{};
  j.n = 6;
  j.M = int(M);
  const int64_t C[6] = {H, H, I, I, I, H};
  int64_t blocks = 0;
  for (int q = 0; q < 6; ++q) {
    j.job[q].C = int(C[q]);
    j.job[q].nq = r;
    blocks += cdiv(C[q], 1024);
  }
  const int64_t jb = cdiv(r, 16);
  // about 512 workgroups, chunks of at least 64 rows
  j.chunks = int(std::max<int64_t>(1, std::min<int64_t>(cdiv(512, blocks * jb), M / 64)));
  return j;
}

MlpBwdLayout mlp_bwd_layout(int64_t M, int64_t H, int64_t I, int32_t r) {
  MlpBwdLayout L{};
  L.rp = cdiv(r, 32) * 32;
  const int rp = int(L.rp);
  L.s_x = shrink_ws(LORA_BF16, M, H, 2, rp, 0, prefer_lds(M, H, 2, rp));
  L.r_x = shrink_ws(LORA_BF16, M, H, 2, rp, 0, false);
  L.s_w = shrink_ws(LORA_BF16, M, H, 1, rp, 0, prefer_lds(M, H, 1, rp));
  L.s_i = shrink_ws(LORA_BF16, M, I, 1, rp, 0, prefer_lds(M, I, 1, rp));
  L.r_i = shrink_ws(LORA_BF16, M, I, 1, rp, 0, false);
  L.cj = mlp_bwd_coljobs(M, H, I, r);
  size_t off = 0;
  L.sbdt = off; off += align256(size_t(r) * H * 2);
  L.sbgt = off; off += align256(size_t(r) * I * 2);
  L.sbut = off; off += align256(size_t(r) * I * 2);
  L.adt = off; off += align256(size_t(I) * L.rp * 2);
  L.agut = off; off += align256(size_t(H) * 2 * L.rp * 2);
  L.xa_gu = off; off += align256(size_t(M) * 2 * L.rp * 2);
  L.dxa_d = off; off += align256(size_t(M) * L.rp * 2);
  L.xa_d = off; off += align256(size_t(M) * L.rp * 2);
  L.dxa_gu = off; off += align256(size_t(M) * 2 * L.rp * 2);
  L.hmid = off; off += align256(size_t(M) * I * 2);
  L.dedv = off; off += align256(size_t(M) * 2 * I * 2);
  size_t sp = 0;
  for (const ShrinkWs* w : {&L.s_x, &L.r_x, &L.s_w, &L.s_i, &L.r_i}) sp = std::max(sp, w->total - w->part);
  L.part = off; off += align256(sp);
  L.colpart = off; off += align256(lmx::colred_partial_floats(L.cj) * 4);
  L.total = off;
  return L;
}

// One dense LoRA-A product h = round(x A^T) (one segment; S slices of padded rank rp, true rank
// r): the LDS-staged plan when A is aligned, else the register-ring plan.
hipError_t dense_shrink(const void* x, int64_t ldx, int64_t K, int S, const void* const* A,
                        int64_t lda, int64_t M, int rp, int r, void* h, int64_t ldh,
                        const ShrinkWs& s_al, const ShrinkWs& s_un, void* part, hipStream_t st) {
  bool al = true;
  for (int q = 0; q < S; ++q) al = al && al16(A[q]);
  const ShrinkWs& sp = al ? s_al : s_un;
  lmx::ShrinkArgs a{};
  a.x = x; a.ldx = ldx; a.K = K; a.S = S; a.R = rp; a.G = 1; a.T = int(M);
  a.dense_rank = r; a.w_a = A[0]; a.lda = lda;
  for (int q = 0; q < S; ++q) a.w_a_slice[q] = A[q];
  a.h = h; a.ldh = ldh;
  a.sk_q = sp.q; a.sk_tiles = int(sp.bound); a.sk_mp = sp.mp; a.sk_unit = sp.unit;
  a.part = static_cast<float*>(part);
  lmx::ShrinkPlan plan{sp.variant, sp.grid_x, al, sp.lds};
  hipError_t e = lmx::launch_shrink(LORA_BF16, a, plan, st);
  if (e == hipSuccess && sp.q > 0) e = lmx::launch_shrink_sk_reduce(LORA_BF16, a, sp.bm, st);
  return e;
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
  // 2. [xa_0 | .. | xa_{P-1}] = round(x [A_0; ..]^T) in one pass over x (dense shrink, P slices)
  {
    bool al = true;
    for (int p = 0; p < P; ++p) al = al && al16(a[p]);
    const ShrinkWs& sp = al ? L.s : L.r;
    lmx::ShrinkArgs sa{};
    sa.x = x; sa.ldx = ldx; sa.K = K; sa.S = P; sa.R = int(rp); sa.G = 1; sa.T = int(M);
    sa.dense_rank = r; sa.w_a = a[0]; sa.lda = K;
    for (int p = 0; p < P; ++p) sa.w_a_slice[p] = a[p];
    sa.h = xa; sa.ldh = P * rp;
    sa.sk_q = sp.q; sa.sk_tiles = int(sp.bound); sa.sk_mp = sp.mp; sa.sk_unit = sp.unit;
    sa.part = reinterpret_cast<float*>(ws + L.part);
    lmx::ShrinkPlan plan{sp.variant, sp.grid_x, al, sp.lds};
    if (lmx::launch_shrink(LORA_BF16, sa, plan, st) != hipSuccess) return LORA_EHIP;
    if (sp.q > 0 && lmx::launch_shrink_sk_reduce(LORA_BF16, sa, sp.bm, st) != hipSuccess)
      return LORA_EHIP;
  }
  // 3. out_p = round(x W_p^T + s xa_p B_p^T) with LoRA in K: one launch over the P column
  //    groups (query, key and value share the pass over x and fill the chip together)
  {
    lmx::GemmArgs g{};
    g.A = u16(x); g.lda = ldx; g.W0 = u16(w[0]); g.W1 = u16(w[0]); g.ldw = K;
    g.A2 = xa; g.lda2 = P * rp;
    g.B2 = reinterpret_cast<const uint16_t*>(ws + L.lb[0]); g.ldb2 = rp;
    g.C = static_cast<uint16_t*>(out[0]); g.ldc = ldo[0];
    g.M = int(M); g.N = int(N[0]); g.K = int(K); g.K2 = int(rp);
    if (P > 1) {
      g.ngroups = P;
      g.gblk[0] = 0;
      for (int p = 0; p < P; ++p) {
        g.gW[p] = u16(w[p]);
        g.gB2[p] = reinterpret_cast<const uint16_t*>(ws + L.lb[p]);
        g.ga2[p] = p * rp;
        g.gC[p] = static_cast<uint16_t*>(out[p]);
        g.gldc[p] = ldo[p];
        g.gN[p] = int(N[p]);
        g.gblk[p + 1] = g.gblk[p] + int(cdiv(N[p], 256));
      }
    }
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

void lora_tuning_override(int32_t op, int32_t variant) {
  if (op == 0) g_shrink_override = (variant >= 0 && variant < lmx::num_shrink_variants()) ? variant : -1;
  if (op == 1) g_expand_override = (variant >= 0 && variant < lmx::num_expand_variants()) ? variant : -1;
  if (op == 2) g_expand_bn_override = (variant > 0 && variant <= 65536) ? variant : -1;
  if (op == 3) g_sk_override = (variant >= 0 && variant <= 65535) ? variant : -1;
  if (op == 4) g_lds_override = (variant == 0 || variant == 1) ? variant : -1;
}

size_t lora_shrink_workspace_size(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                                  int32_t G) {
  if (T <= 0 || G <= 0 || K <= 0 || S <= 0 || R <= 0 || !valid_dtype(dtype)) return 0;
  // the kernel family depends on pointer alignment, which the query does not see: cover both
  const size_t reg = shrink_ws(int(dtype), T, K, S, R, G, false).total;
  if (dtype == LORA_F32 || K % 8 != 0 || g_lds_override == 0) return reg;
  return std::max(reg, shrink_ws(int(dtype), T, K, S, R, G, true).total);
}

size_t lora_expand_workspace_size(lora_dtype dtype, int64_t T, int32_t S, int32_t R, int32_t G,
                                  int64_t N) {
  (void)dtype; (void)S; (void)R; (void)N;
  if (T <= 0 || G <= 0) return 0;
  return schedule_bytes(T, G, 16);  // the smallest tile of any expand shape: the longest list
}

lora_status lora_shrink(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R, int32_t L,
                        int32_t G, const void* x, int64_t ldx, const void* w_a, int64_t lda,
                        const int32_t* seg_indptr, const int32_t* weight_indices,
                        const int32_t* permutation, const int32_t* lora_ranks, void* h,
                        int64_t ldh, void* workspace, size_t workspace_bytes, void* stream) {
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
  const bool lds = dtype != LORA_F32 && aligned && K % 8 == 0 && prefer_lds(T, K, S, R);
  const ShrinkWs ws = shrink_ws(int(dtype), T, K, S, R, G, lds);
  const int variant = ws.variant;
  const int bm = ws.bm;
  if (ws.total > 0 && (workspace == nullptr || workspace_bytes < ws.total)) return LORA_EWORKSPACE;
  if (ws.q > 0 && (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return LORA_EWORKSPACE;
  const int64_t bound = ws.bound;
  if (bound >= INT_MAX) return LORA_EUNSUPPORTED;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  lmx::ShrinkArgs a{};
  a.x = x; a.w_a = w_a; a.seg_indptr = seg_indptr; a.weight_indices = weight_indices;
  a.permutation = permutation; a.lora_ranks = lora_ranks; a.h = h;
  a.K = K; a.ldx = ldx; a.lda = lda; a.ldh = ldh; a.S = S; a.R = R; a.G = G; a.T = int(T);
  if (ws.sched > 0) {
    int4* tiles = reinterpret_cast<int4*>(static_cast<char*>(workspace) + 256);
    int* count = static_cast<int*>(workspace);
    hipError_t e = lmx::launch_schedule(seg_indptr, weight_indices, G, bm, tiles, count, st);
    if (e != hipSuccess) return LORA_EHIP;
    a.tiles = tiles; a.tile_count = count;
  }
  a.sk_q = ws.q; a.sk_tiles = int(bound); a.sk_mp = ws.mp; a.sk_unit = ws.unit;
  if (ws.q > 0) a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.part);
  lmx::ShrinkPlan plan{variant, ws.grid_x, aligned, ws.lds};
  if (lmx::launch_shrink(int(dtype), a, plan, st) != hipSuccess) return LORA_EHIP;
  if (ws.q > 0) return hip_status(lmx::launch_shrink_sk_reduce(int(dtype), a, bm, st));
  return LORA_OK;
}

lora_status lora_expand(lora_dtype dtype, int64_t T, int32_t S, int32_t R, int32_t L, int32_t G,
                        int64_t N, const void* h, int64_t ldh, const void* w_b, int64_t ldb,
                        const int32_t* slice_offsets, const int32_t* seg_indptr,
                        const int32_t* weight_indices, const int32_t* permutation,
                        const int32_t* lora_ranks, const float* scalings, void* y, int64_t ldy,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return LORA_EUNSUPPORTED;
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
  const int variant = expand_variant(T, dtype != LORA_F32 && R == 16 && aligned_b && aligned_y);
  const int bm = lmx::expand_plan_bm(int(dtype), variant);
  const bool shared = dtype != LORA_F32 && (variant == lmx::kExpandSharedD1 ||
                                            variant == lmx::kExpandSharedD2);
  const int bn = expand_bn(T, G, N, bm, lmx::expand_plan_waves(int(dtype), variant),
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
    hipError_t e = lmx::launch_schedule(seg_indptr, weight_indices, G, bm, tiles, count, st);
    if (e != hipSuccess) return LORA_EHIP;
    a.tiles = tiles; a.tile_count = count;
  }
  lmx::ExpandPlan plan{variant, int(bound), aligned_b, aligned_y};
  return hip_status(lmx::launch_expand(int(dtype), a, plan, st));
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
  // 2. [xa_g | xa_u] = round(x [A_g; A_u]^T), ranks padded with zeros to rp
  {
    lmx::ShrinkArgs a{};
    a.x = x; a.ldx = ldx; a.K = H; a.S = 2; a.R = int(rp); a.G = 1; a.T = int(M);
    a.dense_rank = r; a.w_a_slice[0] = a_gate; a.w_a_slice[1] = a_up; a.w_a = a_gate; a.lda = H;
    a.h = xa_gu; a.ldh = 2 * rp;
    // x is 16-byte aligned with a 16-byte row stride (checked above); A rows are H long, H % 32 == 0
    const bool al = al16(a_gate) && al16(a_up);
    const ShrinkWs& sp = al ? L.s_gu : L.r_gu;
    a.sk_q = sp.q; a.sk_tiles = int(sp.bound); a.sk_mp = sp.mp; a.sk_unit = sp.unit;
    a.part = reinterpret_cast<float*>(ws + L.part);
    lmx::ShrinkPlan plan{sp.variant, sp.grid_x, al, sp.lds};
    if ((e = lmx::launch_shrink(LORA_BF16, a, plan, st)) != hipSuccess) return LORA_EHIP;
    if (sp.q > 0 && (e = lmx::launch_shrink_sk_reduce(LORA_BF16, a, sp.bm, st)) != hipSuccess)
      return LORA_EHIP;
  }
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
  {
    lmx::ShrinkArgs a{};
    a.x = hmid; a.ldx = I; a.K = I; a.S = 1; a.R = int(rp); a.G = 1; a.T = int(M);
    a.dense_rank = r; a.w_a_slice[0] = a_down; a.w_a = a_down; a.lda = I;
    a.h = xa_d; a.ldh = rp;
    const bool al = al16(a_down);
    const ShrinkWs& sp = al ? L.s_d : L.r_d;
    a.sk_q = sp.q; a.sk_tiles = int(sp.bound); a.sk_mp = sp.mp; a.sk_unit = sp.unit;
    a.part = reinterpret_cast<float*>(ws + L.part);
    lmx::ShrinkPlan plan{sp.variant, sp.grid_x, al, sp.lds};
    if ((e = lmx::launch_shrink(LORA_BF16, a, plan, st)) != hipSuccess) return LORA_EHIP;
    if (sp.q > 0 && (e = lmx::launch_shrink_sk_reduce(LORA_BF16, a, sp.bm, st)) != hipSuccess)
      return LORA_EHIP;
  }
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
  uint16_t *dxa_gu = W(L.dxa_gu), *hmid = W(L.hmid), *dedv = W(L.dedv);
  void* part = ws + L.part;
  // 1. operands: s B_d^T [r][H], s B_g^T, s B_u^T [r][I]; A_d^T [I][rp]; [A_g^T | A_u^T] [H][2 rp]
  {
    lmx::TJobs t{};
    t.n = 6;
    t.job[0] = {u16(b_down), r, sbdt, H, r, int(H), 0, int(H), scale};
    t.job[1] = {u16(b_gate), r, sbgt, I, r, int(I), 0, int(I), scale};
    t.job[2] = {u16(b_up), r, sbut, I, r, int(I), 0, int(I), scale};
    t.job[3] = {u16(a_down), I, adt, rp, int(I), rp, 0, r, 1.0f};
    t.job[4] = {u16(a_gate), H, agut, 2 * rp, int(H), rp, 0, r, 1.0f};
    t.job[5] = {u16(a_up), H, agut + rp, 2 * rp, int(H), rp, 0, r, 1.0f};
    if (lmx::launch_small_transposes(t, st) != hipSuccess) return LORA_EHIP;
  }
  // 2. [xa_g | xa_u] = round(x [A_g; A_u]^T)
  {
    const void* A[2] = {a_gate, a_up};
    if (dense_shrink(x, ldx, H, 2, A, H, M, rp, r, xa_gu, 2 * rp, L.s_x, L.r_x, part, st) != hipSuccess)
      return LORA_EHIP;
  }
  // 3. dxa_d = round(dout (s B_d))
  {
    const void* A[1] = {sbdt};
    if (dense_shrink(dout, lddo, H, 1, A, H, M, rp, r, dxa_d, rp, L.s_w, L.s_w, part, st) != hipSuccess)
      return LORA_EHIP;
  }
  // 4. dhmid = dout W_d + dxa_d A_d with the SwiGLU backward in the epilogue:
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
  // 5. xa_d = round(hmid A_d^T)
  {
    const void* A[1] = {a_down};
    if (dense_shrink(hmid, I, I, 1, A, I, M, rp, r, xa_d, rp, L.s_i, L.r_i, part, st) != hipSuccess)
      return LORA_EHIP;
  }
  // 6. dxa_g = round(de (s B_g)), dxa_u = round(dv (s B_u))
  {
    const void* Ag[1] = {sbgt};
    const void* Au[1] = {sbut};
    if (dense_shrink(dedv, 2 * I, I, 1, Ag, I, M, rp, r, dxa_gu, 2 * rp, L.s_i, L.s_i, part, st) != hipSuccess ||
        dense_shrink(dedv + I, 2 * I, I, 1, Au, I, M, rp, r, dxa_gu + rp, 2 * rp, L.s_i, L.s_i, part, st) != hipSuccess)
      return LORA_EHIP;
  }
  // 7. LoRA weight gradients (sums over the M tokens)
  {
    lmx::ColJobs j = L.cj;
    auto set = [&](int q, const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq, void* out,
                   int64_t osc, int64_t osj, float sc) {
      j.job[q].P = P; j.job[q].ldp = ldp; j.job[q].Q = Q; j.job[q].ldq = ldq;
      j.job[q].out = static_cast<uint16_t*>(out); j.job[q].osc = osc; j.job[q].osj = osj;
      j.job[q].scale = sc;
    };
    set(0, u16(x), ldx, dxa_gu, 2 * rp, da_gate, 1, H, 1.0f);          // dA_g = dxa_g^T x
    set(1, u16(x), ldx, dxa_gu + rp, 2 * rp, da_up, 1, H, 1.0f);       // dA_u = dxa_u^T x
    set(2, dedv, 2 * I, xa_gu, 2 * rp, db_gate, r, 1, scale);          // dB_g = s de^T xa_g
    set(3, dedv + I, 2 * I, xa_gu + rp, 2 * rp, db_up, r, 1, scale);   // dB_u = s dv^T xa_u
    set(4, hmid, I, dxa_d, rp, da_down, 1, I, 1.0f);                   // dA_d = dxa_d^T hmid
    set(5, u16(dout), lddo, xa_d, rp, db_down, r, 1, scale);           // dB_d = s dout^T xa_d
    if (lmx::launch_colred(j, reinterpret_cast<float*>(ws + L.colpart), st) != hipSuccess)
      return LORA_EHIP;
  }
  // 8. dx = round(de W_g + dv W_u + dxa_g A_g + dxa_u A_u)
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
