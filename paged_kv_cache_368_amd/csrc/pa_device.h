// Device-side helpers shared by the gfx950 kernels: storage decoding, 16-byte
// vector types, DPP row reductions and the XCD-aware work-group order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- storage words ---------------------------------------------------------

// Reinterpret a 32-bit word as float.  Takes the word by value on purpose:
// hipcc's __builtin_bit_cast applied directly to an ext_vector element
// (v.y, v.z, ...) reads element 0 instead, so vector elements must be copied
// to a scalar first.
__device__ __forceinline__ float as_f32(uint32_t w) { return __builtin_bit_cast(float, w); }

template <int DT> struct Storage;
template <> struct Storage<kF32> { static constexpr int kBytes = 4; };
template <> struct Storage<kF16> { static constexpr int kBytes = 2; };
template <> struct Storage<kBF16> { static constexpr int kBytes = 2; };
template <> struct Storage<kFP8> { static constexpr int kBytes = 1; };

// Widen the two 16-bit values packed in a 32-bit word.
template <int DT> __device__ __forceinline__ float lo_f32(uint32_t w);
template <int DT> __device__ __forceinline__ float hi_f32(uint32_t w);
template <> __device__ __forceinline__ float lo_f32<kF16>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w).x;
}
template <> __device__ __forceinline__ float hi_f32<kF16>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w).y;
}
template <> __device__ __forceinline__ float lo_f32<kBF16>(uint32_t w) {
  return __builtin_bit_cast(float, w << 16);
}
template <> __device__ __forceinline__ float hi_f32<kBF16>(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

// acc + a.lo*b.lo + a.hi*b.hi on the packed dot units; products of two
// 16-bit values are exact in float32.
template <int DT> __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc);
template <> __device__ __forceinline__ float dot2<kF16>(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc,
                                false);
}
template <> __device__ __forceinline__ float dot2<kBF16>(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}

// Two E4M3 codes (bytes 0-1 or 2-3 of a word) as a packed 16-bit pair of a
// 16-bit type QT; exact (every E4M3 value is a binary16 and a bfloat16 value).
template <int QT, bool HI>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t w) {
  if constexpr (QT == kBF16)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Work-groups go to the 8 XCDs round-robin (XCD = hardware index % 8), each
// XCD with its own L2.  When G consecutive logical items read the same K/V
// (the query heads of one kv head on the vector kernel, the query tiles of
// one kv head on the matrix-core kernel), this mapping puts every such
// group on one XCD and next to each other in dispatch order, so after the
// first of them the group's K/V come from that XCD's L2 (with the identity
// mapping the G reads of a tile went to G different L2s).  Items past the
// last whole span of 8 groups keep the identity mapping.
__device__ __forceinline__ int group_on_xcd(int b, int n, int G) {
  constexpr int kXcds = 8;
  const int span = kXcds * G;
  if (G == 1 || b >= n / span * span) return b;
  const int blk = b / span, r = b - blk * span;
  const int x = r % kXcds, j = r / kXcds;      // XCD x, j-th item of the span on it
  return blk * span + x * G + j;               // head j of group blk * 8 + x
}

// XCD-major order of n independent items: the hardware hands work-groups to
// the XCDs round-robin (XCD = index % 8), so giving XCD x the consecutive
// items x*per .. x*per+per-1 (per = n / 8) keeps neighbouring items, e.g. the
// pieces of one block, on one XCD and next to each other in its dispatch
// order.  Items past the last whole 8*per keep the identity mapping.
__device__ __forceinline__ long long xcd_major(long long b, long long n) {
  const long long per = n / 8;
  if (b >= per * 8) return b;
  return (b % 8) * per + b / 8;
}

// Round float32 to the storage type, nearest-even; returns the storage bits.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t b = __builtin_bit_cast(uint32_t, x);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays a quiet NaN
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

// Store n float32 values as storage words of type DT (nearest-even).
template <int DT>
__device__ __forceinline__ void store_out(void *base, size_t elem, const float *o, int n) {
  if constexpr (DT == kF32) {
    float *p = reinterpret_cast<float *>(base) + elem;
    for (int i = 0; i < n; ++i) p[i] = o[i];
  } else {
    uint16_t *p = reinterpret_cast<uint16_t *>(base) + elem;
    for (int i = 0; i < n; ++i)
      p[i] = (uint16_t)(DT == kF16 ? f32_to_f16_bits(o[i]) : f32_to_bf16_bits(o[i]));
  }
}

// E4M3 code of a float32 value (the value already divided by the pool's
// scale): nearest code with ties to the even code, magnitudes above 448
// saturated to 448, NaN to 0x7F.  Done by exact power-of-two scaling and
// rintf (round to nearest even on the integer grid of the target format), so
// no hardware conversion mode is involved.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, x);
  if ((bits & 0x7fffffffu) > 0x7f800000u) return 0x7fu;
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fminf(__builtin_fabsf(x), 448.f);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = (uint32_t)__builtin_rintf(a * 512.f);             // subnormal grid, step 2^-9
  } else {
    const uint32_t ab = __builtin_bit_cast(uint32_t, a);
    const int e = (int)(ab >> 23) - 127;                      // 2^e <= a < 2^(e+1), e in [-6, 8]
    const float m = __builtin_bit_cast(float, (ab & 0x007fffffu) | 0x3f800000u);   // a / 2^e
    const uint32_t mq = (uint32_t)__builtin_rintf((m - 1.f) * 8.f);   // 0..8; 8 carries
    code = ((uint32_t)(e + 7) << 3) + mq;
  }
  return code | sign;
}

// The 16 E4M3 codes (one per byte, element order) of 16 consecutive source
// elements of type ST held in SW = 16 * bytes / 16 words, each divided by
// the pool's scale first.
template <int ST>
__device__ __forceinline__ u32x4 e4m3_codes16(const u32x4 *w, float scale) {
  constexpr int SW = Storage<ST>::kBytes;
  float x[16];
#pragma unroll
  for (int j = 0; j < SW; ++j) {
    const uint32_t ww[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (ST == kF32) {
        x[4 * j + k] = as_f32(ww[k]);
      } else {
        x[8 * j + 2 * k] = lo_f32<ST>(ww[k]);
        x[8 * j + 2 * k + 1] = hi_f32<ST>(ww[k]);
      }
    }
  }
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word |= e4m3_code(x[4 * k + b] / scale) << (8 * b);
    out[k] = word;
  }
  return u32x4{out[0], out[1], out[2], out[3]};
}

// A pointer the caller knows to be the same in every lane, pinned to scalar
// registers.  Buffer descriptors built from a base the compiler has placed in
// VGPRs are wrapped in a per-load "waterfall" loop (readfirstlane, compare,
// exec mask) around every buffer load; this keeps the base scalar.
template <typename T>
__device__ __forceinline__ T *scalar_ptr(T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T *>(((uint64_t)hi << 32) | lo);
}

// Split-context partial states of the vector kernel (read once, by the merge
// launch that follows): written through to memory with agent-scope stores
// rather than left dirty in the XCD's L2.  Measured on a 32k-token, 64-way
// split: 2.7% less time per call than plain stores; on the grouped-query
// kernel's few, larger partials plain stores were 1.5% faster, so that
// kernel keeps them.
__device__ __forceinline__ void store_partial(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- cross-lane ------------------------------------------------------------

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;     // within a 16-lane row this is lane ^ 8
constexpr int kDppRowHalfMirror = 0x141;

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of N lanes (N in {4, 8, 16, 32}); every lane of
// the group receives the total.
template <int N> __device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group");
  if constexpr (N == 8) {
    v += dpp<kDppRowHalfMirror>(v);
  } else if constexpr (N >= 16) {
    v += dpp<kDppRowRor8>(v);
    v += dpp<kDppRowRor4>(v);
  }
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppQuadXor1>(v);
  if constexpr (N == 32) v += __shfl_xor(v, 16);
  return v;
}

// Combine each lane's value with that of lane l ^ 16 (or l ^ 32) through the
// gfx950 permlane swaps, which stay in the VALU (no LDS round trip).  With
// both operands equal, the two results of a swap are x[l] and x[l ^ 16] (x[l ^
// 32]) in an order that depends on the lane, so only symmetric combinations
// (sum, max) are formed; a + b is exact-order-independent in IEEE arithmetic.
__device__ __forceinline__ void swap16(float x, float &a, float &b) {
  const uint32_t w = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = as_f32(r0);
  b = as_f32(r1);
}
__device__ __forceinline__ void swap32(float x, float &a, float &b) {
  const uint32_t w = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = as_f32(r0);
  b = as_f32(r1);
}
__device__ __forceinline__ float sum_xor16(float x) { float a, b; swap16(x, a, b); return a + b; }
__device__ __forceinline__ float sum_xor32(float x) { float a, b; swap32(x, a, b); return a + b; }
__device__ __forceinline__ float max_xor16(float x) { float a, b; swap16(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float max_xor32(float x) { float a, b; swap32(x, a, b); return fmaxf(a, b); }

// Word 3 of a raw (untyped, unswizzled) buffer descriptor on CDNA3/CDNA4.
constexpr int kBufferFlags = 0x00020000;

// Cache-policy operand of the K/V buffer loads: the non-temporal bit (bit 1,
// "nt" on gfx940-family targets).  K/V rows are read exactly once per call,
// so they are marked as streaming; on MI355X this lifts a plain read of 4 KB
// tiles in random order from ~5.8 to ~6.5 TB/s at 672 MB and from ~6.1 to
// ~6.8 TB/s at 2.7 GB.
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
