// Device-side building blocks shared by the gfx950 kernels: storage types, fp32 <-> storage
// conversions (round to nearest even), 16-byte operand fragments and the MFMA step.
//
// MFMA operand layout used throughout (v_mfma_f32_16x16x32_{bf16,f16} and, four at a time,
// v_mfma_f32_16x16x4_f32): lane l supplies row (l % 16) of the 16-row A operand and column
// (l % 16) of the 16-column B operand, with the reduction index set by the lane group
// (l / 16) and the element inside the lane's 16-byte fragment; both operands use the same
// (lane group, element) -> k assignment, so any consistent k order is a valid contraction.
// The 16x16 fp32 result D[i][j] lives in lane j + 16 * (i / 4), register i % 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmx {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

template <int DT>
struct Traits;

template <>
struct Traits<DT_F32> {
  using store_t = uint32_t;     // raw bits
  static constexpr int kPerFrag = 4;   // elements per 16-byte fragment
  static constexpr int kStep = 16;     // reduction indices covered by one fragment step
  static __device__ __forceinline__ float to_f32(uint32_t b) { return __uint_as_float(b); }
  static __device__ __forceinline__ uint32_t from_f32(float f) { return __float_as_uint(f); }
};

template <>
struct Traits<DT_BF16> {
  using store_t = uint16_t;
  static constexpr int kPerFrag = 8;
  static constexpr int kStep = 32;
  static __device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
  // Round to nearest even; NaN stays NaN (quiet); overflow rounds to infinity.
  static __device__ __forceinline__ uint16_t from_f32(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
  }
};

template <>
struct Traits<DT_F16> {
  using store_t = uint16_t;
  static constexpr int kPerFrag = 8;
  static constexpr int kStep = 32;
  static __device__ __forceinline__ float to_f32(uint16_t b) {
    return float(__builtin_bit_cast(_Float16, b));
  }
  static __device__ __forceinline__ uint16_t from_f32(float f) {
    return __builtin_bit_cast(uint16_t, _Float16(f));  // v_cvt_f16_f32: round to nearest even
  }
};

// Branch-free 16-byte operand fetch, split in two so that a run of fetches stays in flight:
// fetch() only computes an address and issues the load(s); raw() / masked(valid) (called where the
// operand is consumed) funnel-shift and, for masked(), zero every element at or beyond `valid`
// (the same count that was passed to fetch()).
// `p` points at an element of a row, `valid` is the number of elements from p that belong to the
// operand (<= 0: none; a fragment holds 16/sizeof(S) elements) and `safe` is an element address
// known to be readable (fetched instead of p when nothing is valid).
//
// ALIGNED: p and safe are 16-byte aligned, one load; a partial fragment stays inside its own
// aligned block. Otherwise p may sit at any element boundary: the two aligned 16-byte blocks
// covering the fragment are loaded and shifted; a block that holds no valid byte is replaced by
// the first block, so no load touches a 16-byte block without a valid byte in it (such a block
// never shares a page with memory the operand does not own).
template <typename S>
__device__ __forceinline__ uint4 mask_elems(uint4 v, int valid) {
  uint32_t u[4] = {v.x, v.y, v.z, v.w};
  if constexpr (sizeof(S) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t m = (2 * i < valid ? 0x0000ffffu : 0u) | (2 * i + 1 < valid ? 0xffff0000u : 0u);
      u[i] &= m;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = i < valid ? u[i] : 0u;
  }
  return make_uint4(u[0], u[1], u[2], u[3]);
}

// 16-byte load through an explicitly global pointer (a generic pointer would become a flat load,
// which the compiler cannot track precisely and answers with full waits).
__device__ __forceinline__ uint4 gload16(const void* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(1))) u32x4_t gu4;
  const u32x4_t v = *(gu4*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename S, bool ALIGNED>
struct Frag;

template <typename S>
struct Frag<S, true> {
  uint4 a;
  __device__ __forceinline__ void fetch(const S* p, int v, const S* safe) {
    a = gload16(v > 0 ? p : safe);
  }
  __device__ __forceinline__ uint4 raw() const { return a; }
  __device__ __forceinline__ uint4 masked(int valid) const { return mask_elems<S>(a, valid); }
};

template <typename S>
struct Frag<S, false> {
  uint4 a, b;
  uint32_t off;
  __device__ __forceinline__ void fetch(const S* p, int v, const S* safe) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(v > 0 ? p : safe);
    const uintptr_t lo = pa & ~uintptr_t(15);
    off = uint32_t(pa & 15u);
    const bool hi_ok = v > 0 && int(off) + v * int(sizeof(S)) > 16;
    a = gload16(reinterpret_cast<const void*>(lo));
    b = gload16(reinterpret_cast<const void*>(hi_ok ? lo + 16 : lo));
  }
  __device__ __forceinline__ uint4 raw() const {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const uint32_t d = off >> 2, sh = off & 3u;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w0 = d == 0 ? w[i] : d == 1 ? w[i + 1] : d == 2 ? w[i + 2] : w[i + 3];
      const uint32_t w1 = d == 0 ? w[i + 1] : d == 1 ? w[i + 2] : d == 2 ? w[i + 3] : w[i + 4];
      o[i] = __builtin_amdgcn_alignbyte(w1, w0, sh);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
  __device__ __forceinline__ uint4 masked(int valid) const { return mask_elems<S>(raw(), valid); }
};

// Non-temporal 16-byte load and store for data touched exactly once (the expand's y rows): the
// lines are not kept in the caches, so they neither evict reused operands nor leave dirty lines
// behind for the next kernel to wait on.
__device__ __forceinline__ uint4 gload16_nt(const void* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(1))) u32x4_t gu4;
  const u32x4_t v = __builtin_nontemporal_load((gu4*)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void gstore16_nt(void* p, uint4 a) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) u32x4_t gu4;
  const u32x4_t v = {a.x, a.y, a.z, a.w};
  __builtin_nontemporal_store(v, (gu4*)(p));
}

// 8-byte variant of Frag for the streamed output rows (4 elements of a 16-bit type, 2 of fp32).
__device__ __forceinline__ uint2 gload8(const void* p) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  typedef const __attribute__((address_space(1))) u32x2_t gu2;
  const u32x2_t v = *(gu2*)(p);
  return make_uint2(v.x, v.y);
}

template <typename S, bool ALIGNED>
struct Frag8;

template <typename S>
struct Frag8<S, true> {
  uint2 a;
  __device__ __forceinline__ void fetch(const S* p, int v, const S* safe) {
    a = gload8(v > 0 ? p : safe);
  }
  __device__ __forceinline__ uint2 raw() const { return a; }
};

template <typename S>
struct Frag8<S, false> {
  uint2 a, b;
  uint32_t off;
  __device__ __forceinline__ void fetch(const S* p, int v, const S* safe) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(v > 0 ? p : safe);
    const uintptr_t lo = pa & ~uintptr_t(7);
    off = uint32_t(pa & 7u);
    const bool hi_ok = v > 0 && int(off) + v * int(sizeof(S)) > 8;
    a = gload8(reinterpret_cast<const void*>(lo));
    b = gload8(reinterpret_cast<const void*>(hi_ok ? lo + 8 : lo));
  }
  __device__ __forceinline__ uint2 raw() const {
    const uint32_t w[4] = {a.x, a.y, b.x, b.y};
    const uint32_t d = off >> 2, sh = off & 3u;
    const uint32_t o0 = __builtin_amdgcn_alignbyte(d ? w[2] : w[1], d ? w[1] : w[0], sh);
    const uint32_t o1 = __builtin_amdgcn_alignbyte(d ? w[3] : w[2], d ? w[2] : w[1], sh);
    return make_uint2(o0, o1);
  }
};

// Wave index as a scalar, so loop bounds derived from it stay uniform branches.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6); }

// acc += A_frag * B_frag over one fragment step (32 reduction indices for 16-bit types,
// 16 for fp32 as four 16x16x4 steps over the fragment's four elements).
template <int DT>
__device__ __forceinline__ f32x4_t mma_step(uint4 a, uint4 b, f32x4_t acc);

template <>
__device__ __forceinline__ f32x4_t mma_step<DT_BF16>(uint4 a, uint4 b, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4_t mma_step<DT_F16>(uint4 a, uint4 b, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4_t mma_step<DT_F32>(uint4 a, uint4 b, f32x4_t acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// One direct-to-LDS 16-byte load per lane: the wave writes 1 KiB of LDS at byte address
// `lds_addr` (wave-uniform; lane L at +16 L). Issued from an asm block with no register
// outputs: the compiler does not track it, so waits on these loads are explicit (vm_wait); the
// compiler's own waits on other loads stay correct because the counter completes in order and
// can only over-wait.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset (the
// scalar-base addressing form), so the per-lane address needs no vector arithmetic.
// The base must be wave-uniform; it is passed through readfirstlane so that it sits in SGPRs
// even where the compiler's uniformity analysis cannot prove it (free when it already does).
__device__ __forceinline__ void dma16_saddr(const void* base, uint32_t voff, uint32_t lds_addr) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(b >> 32));
  const void* sb = reinterpret_cast<const void*>((uint64_t(hi) << 32) | lo);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(lds_addr)
               : "memory", "m0");
}

template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) T*)p));
}

// s_waitcnt immediate for vmcnt(n) alone (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt
// 6:4 and lgkmcnt 11:8 left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | ((N >> 4) << 14));
}

}  // namespace lmx
