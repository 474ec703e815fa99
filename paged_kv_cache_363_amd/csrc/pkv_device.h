// Device-side helpers shared by the HIP kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv.h"

namespace pkvd {

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// Loads of cache tiles.  Every K/V byte of a decode step is read once, so
// the streaming form carries the non-temporal hint and does not displace
// other lines from the L2 and the Infinity Cache.  Measured on MI355X: random
// 4 KiB tiles stream at 6.8 TB/s with the hint against 6.1 TB/s without; the
// balanced kernel gains with it on every cache type, and so does the
// fixed-partition kernel on one-byte caches (E4M3 and INT8, once the loads
// stay in the loaded vector type, see below).  The fixed-partition kernel on
// 16-bit caches is faster without it: there sequences that share a prefix
// re-read its blocks, and the hint evicts them.  NT is a choice per call
// site.
template <bool NT>
__device__ __forceinline__ uint4 ld_tile16(const void* p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}
template <bool NT>
__device__ __forceinline__ uint2 ld_tile8(const void* p) {
  if constexpr (NT) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
  } else {
    return *reinterpret_cast<const uint2*>(p);
  }
}
template <bool NT>
__device__ __forceinline__ uint32_t ld_tile4(const void* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  } else {
    return *reinterpret_cast<const uint32_t*>(p);
  }
}

// The same loads kept in the loaded vector type.  A loop that carries the
// result of a non-temporal load across its back edge after converting it to
// a struct type (uint4, uint2) can get register copies there, and a copy of
// a register still being loaded waits for every load in flight.
template <bool NT>
__device__ __forceinline__ u32x4 ld_vec16(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ u32x2 ld_vec8(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  else return *reinterpret_cast<const u32x2*>(p);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

template <int DT>
struct DType;
template <>
struct DType<PKV_F32> {
  static constexpr int bytes = 4;
};
template <>
struct DType<PKV_F16> {
  static constexpr int bytes = 2;
};
template <>
struct DType<PKV_BF16> {
  static constexpr int bytes = 2;
};
template <>
struct DType<PKV_FP8_E4M3> {
  static constexpr int bytes = 1;
};
template <>
struct DType<PKV_INT8> {
  static constexpr int bytes = 1;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Round a binary32 to bfloat16, nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Widen 4 elements of one 32-bit word group (a uint4 holds 16 bytes) to f32.
// Element e of a 16-byte chunk, for each storage type.
template <int DT>
__device__ __forceinline__ void chunk_to_f32(const uint4& r, float* f);

template <>
__device__ __forceinline__ void chunk_to_f32<PKV_F32>(const uint4& r, float* f) {
  f[0] = __uint_as_float(r.x);
  f[1] = __uint_as_float(r.y);
  f[2] = __uint_as_float(r.z);
  f[3] = __uint_as_float(r.w);
}
template <>
__device__ __forceinline__ void chunk_to_f32<PKV_BF16>(const uint4& r, float* f) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}
template <>
__device__ __forceinline__ void chunk_to_f32<PKV_F16>(const uint4& r, float* f) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = f16_lo(w[i]);
    f[2 * i + 1] = f16_hi(w[i]);
  }
}
// OCP E4M3FN codes -> f32 with the hardware converter (scale 1.0: exact).
template <>
__device__ __forceinline__ void chunk_to_f32<PKV_FP8_E4M3>(const uint4& r, float* f) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], 1.0f, false);
    f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], 1.0f, true);
    f[4 * i + 0] = a[0];
    f[4 * i + 1] = a[1];
    f[4 * i + 2] = b[0];
    f[4 * i + 3] = b[1];
  }
}

// Signed INT8 codes -> f32 (exact).
template <>
__device__ __forceinline__ void chunk_to_f32<PKV_INT8>(const uint4& r, float* f) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < 4; ++b) f[4 * i + b] = (float)(int32_t)(int8_t)(w[i] >> (8 * b));
}

// Binary32 -> INT8 code: nearest integer, ties to even (rintf in the default
// rounding mode), saturated to +-127, NaN -> 0.  Returned as the code's byte.
__device__ __forceinline__ uint32_t f32_to_i8(float x) {
  if (x != x) return 0u;
  const float r = fminf(fmaxf(__builtin_rintf(x), -127.0f), 127.0f);
  return (uint32_t)(int32_t)r & 0xFFu;
}

// Binary32 -> E4M3FN code: nearest, ties to even, |x| >= 448 (and +-inf)
// saturate to +-448, NaN -> 0x7F.  Integer arithmetic only, so the result
// does not depend on the float rounding mode.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  u &= 0x7FFFFFFFu;
  if (u > 0x7F800000u) return 0x7Fu;              // NaN
  if (u >= 0x43E00000u) return sign | 0x7Eu;      // >= 448: saturate (incl. inf)
  if (u < 0x3C800000u) {                          // below 2^-6: subnormal codes
    // m = round_half_even(|x| * 2^9) in 0..8; 8 is the smallest normal code
    float q = __uint_as_float(u) * 512.0f;        // exact: power-of-two scale
    uint32_t m = (uint32_t)__builtin_rintf(q);
    return sign | m;
  }
  // normal: keep 3 mantissa bits with round-to-nearest-even on bit 20
  uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  uint32_t code = (r >> 20) - (120u << 3);        // rebias exponent 127 -> 7
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// N = 1, 2, 4 or 8 consecutive elements of a new K or V row in the 16-bit
// dtype NEW_DT (raw: their bits, the first N * 2 bytes of the 16), in the
// cache dtype KV_DT as the cache append stores them: the same bits for a
// 16-bit cache (KV_DT == NEW_DT), else each element's code from x * inv in
// binary32 (f32_to_e4m3 / f32_to_i8), byte i of the chunk at bits 8 (i % 4)
// of word i / 4.  w receives the N * bytes(KV_DT) bytes in whole words (the
// bytes past them zero).
template <int NEW_DT, int KV_DT, int N>
__device__ __forceinline__ void encode_new_chunk(uint4 raw, float inv, uint32_t* w) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "1, 2, 4 or 8 elements");
  static_assert(NEW_DT == PKV_F16 || NEW_DT == PKV_BF16, "16-bit new rows");
  if constexpr (N <= 4) {
    raw.z = 0u;
    raw.w = 0u;
  }
  if constexpr (N <= 2) raw.y = 0u;
  if constexpr (N == 1) raw.x &= 0xFFFFu;
  if constexpr (KV_DT == NEW_DT) {
    w[0] = raw.x;
    if constexpr (N >= 4) w[1] = raw.y;
    if constexpr (N == 8) {
      w[2] = raw.z;
      w[3] = raw.w;
    }
  } else {
    static_assert(KV_DT == PKV_FP8_E4M3 || KV_DT == PKV_INT8, "one-byte codes");
    float f[8];
    chunk_to_f32<NEW_DT>(raw, f);
    constexpr int NW = N < 4 ? 1 : N / 4;
    uint32_t word[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) word[k] = 0u;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float x = f[i] * inv;
      word[i / 4] |= (KV_DT == PKV_FP8_E4M3 ? f32_to_e4m3(x) : f32_to_i8(x)) << (8 * (i % 4));
    }
#pragma unroll
    for (int k = 0; k < NW; ++k) w[k] = word[k];
  }
}

}  // namespace pkvd
