// Device-side helpers shared by the HIP kernels of libtileshare (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define TS_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return float(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return bf16(v); }

// Load / store 4 consecutive elements as fp32.
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{float(v[0]), float(v[1]), float(v[2]), float(v[3])};
}
__device__ __forceinline__ void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
  bf16x4 o = {bf16(v[0]), bf16(v[1]), bf16(v[2]), bf16(v[3])};
  *reinterpret_cast<bf16x4*>(p) = o;
}

// Load / store 8 consecutive elements (16-byte aligned) as two fp32 quads.
__device__ __forceinline__ void load8(const float* p, f32x4& a, f32x4& b) {
  a = load4(p);
  b = load4(p + 4);
}
__device__ __forceinline__ void load8(const bf16* p, f32x4& a, f32x4& b) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
  a = f32x4{float(v[0]), float(v[1]), float(v[2]), float(v[3])};
  b = f32x4{float(v[4]), float(v[5]), float(v[6]), float(v[7])};
}
__device__ __forceinline__ void store8(float* p, f32x4 a, f32x4 b) {
  store4(p, a);
  store4(p + 4, b);
}
__device__ __forceinline__ void store8(bf16* p, f32x4 a, f32x4 b) {
  const bf16x8 o = {bf16(a[0]), bf16(a[1]), bf16(a[2]), bf16(a[3]), bf16(b[0]), bf16(b[1]), bf16(b[2]), bf16(b[3])};
  *reinterpret_cast<bf16x8*>(p) = o;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Exact GELU, x * Phi(x) with Phi written through erf.
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
