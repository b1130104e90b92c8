// mfma_ops.h - matrix-core building blocks shared by the decode and the
// prefill kernels: the two 16x16 MFMA shapes used for the logit and value
// products, the conversion of probabilities to 16-bit operands, the tile of
// operands one wavefront loads, and the exact widening of E4M3 codes.
#pragma once

#include "pkv_device.h"

namespace pkv {

template <int DT> struct MfmaOps;

template <> struct MfmaOps<DT_BF16> {
  __device__ static __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // the same 16x16x32 product with the values as A over 32 tokens
  __device__ static __forceinline__ f32x4 pv32(u32x4 a, u32x4 b, f32x4 c) {
    return qk(a, b, c);
  }
  // two floats -> packed bfloat16 pair, nearest even (one instruction on
  // gfx950)
  __device__ static __forceinline__ uint32_t pack2(float p0, float p1) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{p0, p1}), bf16x2));
  }
  __device__ static __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
  // two probabilities -> one packed pair of bfloat16, rounded to nearest
  // even; r0, r1 receive the rounded values
  __device__ static __forceinline__ uint32_t round2(float p0, float p1, float &r0, float &r1) {
    uint32_t u0 = __float_as_uint(p0), u1 = __float_as_uint(p1);
    u0 = (u0 + 0x7fffu + ((u0 >> 16) & 1u)) & 0xffff0000u;  // p finite, >= 0
    u1 = (u1 + 0x7fffu + ((u1 >> 16) & 1u)) & 0xffff0000u;
    r0 = __uint_as_float(u0);
    r1 = __uint_as_float(u1);
    return __builtin_amdgcn_perm(u1, u0, 0x07060302u);
  }
  // two probabilities -> packed (hi, lo) bfloat16 pairs with hi + lo ~= p:
  // hi keeps the top 16 bits of p, lo the top 16 bits of the remainder
  __device__ static __forceinline__ void split2(float p0, float p1, uint32_t &hi,
                                                uint32_t &lo) {
    const uint32_t h0 = __float_as_uint(p0) & 0xffff0000u;
    const uint32_t h1 = __float_as_uint(p1) & 0xffff0000u;
    const uint32_t r0 = __float_as_uint(p0 - __uint_as_float(h0));
    const uint32_t r1 = __float_as_uint(p1 - __uint_as_float(h1));
    hi = __builtin_amdgcn_perm(h1, h0, 0x07060302u);
    lo = __builtin_amdgcn_perm(r1, r0, 0x07060302u);
  }
};

template <> struct MfmaOps<DT_F16> {
  __device__ static __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 pv32(u32x4 a, u32x4 b, f32x4 c) {
    return qk(a, b, c);
  }
  __device__ static __forceinline__ uint32_t pack2(float p0, float p1) {
    const f16x2 h = {static_cast<_Float16>(p0), static_cast<_Float16>(p1)};  // nearest even
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ static __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(
        __builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t round2(float p0, float p1, float &r0, float &r1) {
    const f16x2 h = {static_cast<_Float16>(p0), static_cast<_Float16>(p1)};  // nearest even
    r0 = static_cast<float>(h.x);
    r1 = static_cast<float>(h.y);
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ static __forceinline__ void split2(float p0, float p1, uint32_t &hi,
                                                uint32_t &lo) {
    const f16x2 h = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p0, p1));
    const f16x2 r = __builtin_bit_cast(
        f16x2, __builtin_amdgcn_cvt_pkrtz(p0 - static_cast<float>(h.x),
                                          p1 - static_cast<float>(h.y)));
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, r);
  }
};

// One 16-token tile as loaded: 16-byte chunks of K and of V per lane.
// 16-bit caches: chunk kk of K is the A operand of logit MFMA kk, chunk u of
// V holds the A operands of value n-tiles 2u and 2u+1.  8-bit caches: chunk
// cp of K holds logit MFMAs 2cp and 2cp+1, chunk u of V holds n-tiles
// 4u .. 4u+3; they are widened to 16 bits in registers.
template <int CT, int D>
struct MfmaTile {
  static constexpr int NC = CT == DT_FP8 ? D / 64 : D / 32;
  u32x4 k[NC];
  u32x4 v[NC];
};

// Two E4M3 bytes -> two 16-bit operands of type OT, exactly (every E4M3
// value is a bfloat16 and a binary16 value, so the unit scale of CDNA4's
// packed scaled conversion rounds nothing).  `hi` picks bytes 2-3 of w.
template <int OT>
__device__ __forceinline__ uint32_t fp8x2_to_16(uint32_t w, bool hi) {
  if constexpr (OT == DT_BF16) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  } else {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  }
}

}  // namespace pkv
