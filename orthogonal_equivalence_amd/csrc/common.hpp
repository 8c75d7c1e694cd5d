// Shared device helpers for the POET-X kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

typedef uint16_t bf16_t;  // bfloat16 storage (upper half of a float32)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float32 -> bfloat16 (NaN stays NaN, quieted).
// Written as a select, not a branch, so that unrolled epilogues stay
// straight-line code.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x40u;
  return static_cast<bf16_t>((u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded);
}

// Pack two floats into a bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// OCP E4M3 fp8 byte (sign, 4-bit exponent with bias 7, 3-bit mantissa; the
// NaN bytes 0x7F / 0xFF are never stored here) in the low 8 bits of c, as a
// float: v_cvt_f32_fp8 reads OCP E4M3 on gfx950 (checked against the format's
// definition for all 256 bytes). Exact, and exact again in bfloat16.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(c), 0);
}

// float -> E4M3 byte: nearest value, ties to the even code, magnitudes past
// 448 saturated to 448, the sign bit that of x. Below 2^-6 the steps are
// 2^-9 (rintf: ties to even; 8 steps is the smallest normal); above, the
// float's mantissa is rounded to 3 bits on its bits, the carry moving into
// the exponent.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t sgn = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  uint32_t mag;
  if (a < 0x1p-6f) {
    mag = static_cast<uint32_t>(rintf(a * 512.f));
  } else {
    const uint32_t u = __float_as_uint(a);
    mag = ((u + 0x7ffffu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sgn | mag;
}

template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct ElemTraits<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

__device__ __forceinline__ float load_as_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_as_f32(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_from_f32(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_from_f32(bf16_t* p, float v) { *p = f32_to_bf16(v); }

__device__ __forceinline__ int clamp_index(int32_t i, int64_t dim) {
  return i < 0 ? 0 : (i >= dim ? static_cast<int>(dim - 1) : i);
}

// Remap a linear workgroup id so that the ids dispatched to one XCD (hardware
// hands consecutive ids to the 8 XCDs in turn) form one contiguous range of
// logical tiles; neighbouring tiles then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  constexpr int kXcd = 8;
  const int per = nwg / kXcd;
  const int full = per * kXcd;
  if (wg >= full) return wg;
  return (wg % kXcd) * per + wg / kXcd;
}

}  // namespace poetx
