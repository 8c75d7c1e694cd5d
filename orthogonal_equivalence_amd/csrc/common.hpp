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

// Round-to-nearest-even float32 -> bfloat16 (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Pack two floats into a bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
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
