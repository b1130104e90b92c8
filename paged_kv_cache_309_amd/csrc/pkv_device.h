// pkv_device.h - device-side helpers shared by the gfx950 kernels.
//
// Storage types are handled as raw 32-bit words: a 16-byte global load
// brings four words, i.e. eight fp16/bf16 elements or four fp32 elements,
// and elements are widened to fp32 in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };
template <> struct Elem<DT_F16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };

// Element j of a run of words (j counts elements, not words).
template <int DT>
__device__ __forceinline__ float elem(const uint32_t *w, int j) {
  if constexpr (DT == DT_F32) {
    return __uint_as_float(w[j]);
  } else if constexpr (DT == DT_BF16) {
    const uint32_t x = w[j >> 1];
    return (j & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
  } else {
    const f16x2 h = __builtin_bit_cast(f16x2, w[j >> 1]);
    return (j & 1) ? static_cast<float>(h.y) : static_cast<float>(h.x);
  }
}

// fp32 -> storage bits, rounding to nearest-even.
template <int DT> __device__ __forceinline__ uint32_t from_f32(float x);
template <> __device__ __forceinline__ uint32_t from_f32<DT_F32>(float x) {
  return __float_as_uint(x);
}
template <> __device__ __forceinline__ uint32_t from_f32<DT_F16>(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
template <> __device__ __forceinline__ uint32_t from_f32<DT_BF16>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <int DT>
__device__ __forceinline__ void store_elem(void *base, size_t idx, float x) {
  if constexpr (DT == DT_F32) {
    static_cast<float *>(base)[idx] = x;
  } else {
    static_cast<uint16_t *>(base)[idx] = static_cast<uint16_t>(from_f32<DT>(x));
  }
}

// DPP lane permutations inside a row of 16 lanes.
enum : int {
  DPP_QUAD_XOR1 = 0xB1,    // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,    // quad_perm [2,3,0,1]
  DPP_ROW_MIRROR = 0x140,  // lane i <- lane 15-i
  DPP_ROW_HMIRROR = 0x141  // lane i <- lane 7-i within each half row
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a row; every lane of the row receives the same
// bits (each step adds the same two partial sums, in either order).
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<DPP_QUAD_XOR1>(x);
  x += dpp<DPP_QUAD_XOR2>(x);
  x += dpp<DPP_ROW_HMIRROR>(x);
  x += dpp<DPP_ROW_MIRROR>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

}  // namespace pkv
