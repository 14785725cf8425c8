// C ABI of the library: argument validation, kernel-shape selection and launches.
// Every check here runs on the host before anything is enqueued; nothing reads device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>

#include "../../include/lora_mi355x.h"
#include "sgmv_kernels.hpp"

namespace {

constexpr int kInlineMaxSegments = 1024;  // above this the standalone scheduler builds the list
constexpr int kMaxSlices = 64;
constexpr int kMaxRank = 1024;

int g_shrink_override = -1;
int g_expand_override = -1;
int g_expand_bn_override = -1;

bool valid_dtype(int d) { return d == LORA_F32 || d == LORA_BF16 || d == LORA_F16; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int esize(int dtype) { return dtype == LORA_F32 ? 4 : 2; }

// Columns per expand workgroup: enough blocks for about 2048 workgroups, in multiples of the
// 64-column chunks the waves walk.
int expand_bn(int64_t T, int32_t G, int64_t N, int bm, int waves) {
  const int unit = 64 * waves;
  if (g_expand_bn_override > 0) return int(cdiv(g_expand_bn_override, unit) * unit);
  const int64_t tiles = cdiv(T, bm) + G;
  const int64_t blocks = std::max<int64_t>(1, cdiv(2048, tiles));  // about 2048 workgroups
  int64_t bn = cdiv(cdiv(N, blocks), unit) * unit;
  bn = std::min<int64_t>(std::max<int64_t>(bn, unit), 4096);
  return int(bn);
}

// Kernel shape for a shrink call, from host-known sizes only.
// Shapes picked from rocprofv3 sweeps on MI355X over the decode, prefill and irregular
// workloads: small problems favour one 16-column block per workgroup with 8 waves splitting K;
// large ones 32-token tiles covering up to 4 blocks with a 4-deep x ring.
int shrink_variant(int64_t T, int32_t S, int32_t R) {
  if (g_shrink_override >= 0) return g_shrink_override;
  const int64_t nblk = int64_t(S) * ((R + 15) / 16);
  return T * std::max<int64_t>(1, nblk / 4) >= 4096 ? 2 : 3;
}

int expand_variant(int64_t T) {
  if (g_expand_override >= 0) return g_expand_override;
  return T <= 512 ? 1 : 0;
}

size_t schedule_bytes(int64_t T, int32_t G, int bm) {
  if (G <= kInlineMaxSegments) return 0;
  return size_t(cdiv(T, bm) + G) * 16 + 256;
}

lora_status hip_status(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_EHIP; }

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
}

size_t lora_shrink_workspace_size(lora_dtype dtype, int64_t T, int64_t K, int32_t S, int32_t R,
                                  int32_t G) {
  (void)dtype; (void)K; (void)S; (void)R;
  if (T <= 0 || G <= 0) return 0;
  return schedule_bytes(T, G, lmx::shrink_plan_bm(int(dtype), shrink_variant(T, S, R)));
}

size_t lora_expand_workspace_size(lora_dtype dtype, int64_t T, int32_t S, int32_t R, int32_t G,
                                  int64_t N) {
  (void)dtype; (void)S; (void)R; (void)N;
  if (T <= 0 || G <= 0) return 0;
  return schedule_bytes(T, G, lmx::expand_plan_bm(int(dtype), expand_variant(T)));
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
  if (!x || !w_a || !seg_indptr || !weight_indices || !permutation || !lora_ranks || !h)
    return LORA_EINVAL;
  if (ldx < K || lda < K || ldh < int64_t(S) * R) return LORA_EINVAL;
  const int variant = shrink_variant(T, S, R);
  const int bm = lmx::shrink_plan_bm(int(dtype), variant);
  const size_t need = schedule_bytes(T, G, bm);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LORA_EWORKSPACE;
  const int64_t bound = cdiv(T, bm) + G;
  if (bound >= INT_MAX) return LORA_EUNSUPPORTED;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  lmx::ShrinkArgs a{};
  a.x = x; a.w_a = w_a; a.seg_indptr = seg_indptr; a.weight_indices = weight_indices;
  a.permutation = permutation; a.lora_ranks = lora_ranks; a.h = h;
  a.K = K; a.ldx = ldx; a.lda = lda; a.ldh = ldh; a.S = S; a.R = R; a.G = G;
  if (need > 0) {
    int4* tiles = reinterpret_cast<int4*>(static_cast<char*>(workspace) + 256);
    int* count = static_cast<int*>(workspace);
    hipError_t e = lmx::launch_schedule(seg_indptr, weight_indices, G, bm, tiles, count, st);
    if (e != hipSuccess) return LORA_EHIP;
    a.tiles = tiles; a.tile_count = count;
  }
  const int e = esize(dtype);
  const bool aligned = al16(x) && al16(w_a) && (ldx * e) % 16 == 0 && (lda * e) % 16 == 0;
  lmx::ShrinkPlan plan{variant, int(bound), aligned};
  return hip_status(lmx::launch_shrink(int(dtype), a, plan, st));
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
  if (!h || !w_b || !slice_offsets || !seg_indptr || !weight_indices || !permutation ||
      !lora_ranks || !scalings || !y)
    return LORA_EINVAL;
  if (ldh < int64_t(S) * R || ldb < R || ldy < N) return LORA_EINVAL;
  if (R > lmx::expand_max_rank(int(dtype))) return LORA_EUNSUPPORTED;
  const int variant = expand_variant(T);
  const int bm = lmx::expand_plan_bm(int(dtype), variant);
  const int bn = expand_bn(T, G, N, bm, lmx::expand_plan_waves(int(dtype), variant));
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
  const int e = esize(dtype);
  const bool aligned_b = al16(h) && al16(w_b) && (ldh * e) % 16 == 0 && (ldb * e) % 16 == 0 &&
                         (int64_t(R) * e) % 16 == 0;
  const bool aligned_y = al16(y) && (ldy * e) % 16 == 0;
  lmx::ExpandPlan plan{variant, int(bound), aligned_b, aligned_y};
  return hip_status(lmx::launch_expand(int(dtype), a, plan, st));
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
