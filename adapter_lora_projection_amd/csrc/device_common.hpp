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

// One 16-byte operand fragment: kPerFrag consecutive elements of a row starting at element k,
// zero-filled at and beyond `kend`. Uses a single dwordx4 load when the address is 16-byte
// aligned and the fragment is whole, dword loads when it is 4-byte aligned, element loads
// otherwise.
template <typename S>
__device__ __forceinline__ uint4 load_frag(const S* __restrict__ row, int64_t k, int64_t kend) {
  constexpr int n = 16 / sizeof(S);
  const S* p = row + k;
  if (k + n <= kend) {
    const uintptr_t addr = reinterpret_cast<uintptr_t>(p);
    if ((addr & 15u) == 0) return *reinterpret_cast<const uint4*>(p);
    if ((addr & 3u) == 0) {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
      return make_uint4(q[0], q[1], q[2], q[3]);
    }
  }
  union {
    S e[n];
    uint4 v;
  } u;
#pragma unroll
  for (int i = 0; i < n; ++i) u.e[i] = (k + i < kend) ? p[i] : S(0);
  return u.v;
}

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

}  // namespace lmx
