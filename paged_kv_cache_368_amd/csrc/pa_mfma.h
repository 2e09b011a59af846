// Matrix-core helpers shared by the gfx950 kernels that run attention as
// small dense products (grouped-query decode, prefill): 16x16 MFMA wrappers
// for fp16/bf16 and the split of fp32 weights into 16-bit high and low parts.
#pragma once

#include "pa_device.h"

namespace pa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

template <int DT>
__device__ __forceinline__ f32x4 mfma_k32(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x4 mfma_k16(const u32x2 &a, const u32x2 &b, const f32x4 &c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Split two fp32 weights into packed 16-bit (hi, lo) words: hi keeps the top
// bits (truncation, so p - hi is exact in fp32), lo the next ones.
template <int DT>
__device__ __forceinline__ void split2(float p0, float p1, uint32_t &hi, uint32_t &lo) {
  if constexpr (DT == kBF16) {
    const uint32_t b0 = __builtin_bit_cast(uint32_t, p0), b1 = __builtin_bit_cast(uint32_t, p1);
    hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u);                 // upper halves
    const float r0 = p0 - __builtin_bit_cast(float, b0 & 0xffff0000u);
    const float r1 = p1 - __builtin_bit_cast(float, b1 & 0xffff0000u);
    lo = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, r1), __builtin_bit_cast(uint32_t, r0),
                               0x07060302u);
  } else {
    const auto h = __builtin_amdgcn_cvt_pkrtz(p0, p1);     // round toward zero
    const float h0 = (float)h.x, h1 = (float)h.y;
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p0 - h0, p1 - h1));
  }
}

}  // namespace pa
