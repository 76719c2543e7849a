// Device helpers shared by the libkda HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;

// ---------------------------------------------------------------- io types

// Loads of io elements as fp32 (bf16 -> fp32 is exact).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

// fp32 -> io dtype, round to nearest even.
template <typename IO> __device__ __forceinline__ IO from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Four consecutive io elements as a float4 (p 8- or 16-byte aligned).
__device__ __forceinline__ float4 load4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ float4 load4(const bf16* p) {
  typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

__device__ __forceinline__ void store4(float* p, float4 x) {
  *reinterpret_cast<float4*>(p) = x;
}
__device__ __forceinline__ void store4(bf16* p, float4 x) {
  typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v;
  v[0] = (bf16)x.x;
  v[1] = (bf16)x.y;
  v[2] = (bf16)x.z;
  v[3] = (bf16)x.w;
  *reinterpret_cast<bf16x4*>(p) = v;
}

// ------------------------------------------------------------ float4 math

__device__ __forceinline__ float4 f4(float s) { return make_float4(s, s, s, s); }
__device__ __forceinline__ float4 operator+(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 operator-(float4 a, float4 b) {
  return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
}
__device__ __forceinline__ float4 operator*(float s, float4 a) {
  return make_float4(s * a.x, s * a.y, s * a.z, s * a.w);
}
// a + s * b, one rounding per lane (fma)
__device__ __forceinline__ float4 fma4(float s, float4 b, float4 a) {
  return make_float4(fmaf(s, b.x, a.x), fmaf(s, b.y, a.y), fmaf(s, b.z, a.z),
                     fmaf(s, b.w, a.w));
}

// Four consecutive fp32 values with the non-temporal hint (streamed once:
// the caches need not keep them).
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load4_nt(const float* p) {
  const f32x4_nt y = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(p));
  return make_float4(y[0], y[1], y[2], y[3]);
}
__device__ __forceinline__ void store4_nt(float* p, float4 x) {
  __builtin_nontemporal_store(f32x4_nt{x.x, x.y, x.z, x.w}, reinterpret_cast<f32x4_nt*>(p));
}

// A buffer resource over `bytes` bytes from `base`: loads through it at or
// past that range return zero without touching memory, and stores there are
// dropped.  Word 3 of the descriptor selects 32-bit raw data (the gfx9 value).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Butterfly sum over the lanes whose index differs only in the bits from
// lo_mask (a power of two) up to 32; every lane of such a group ends with
// the group's sum.  xor_sum(x, 1) is the sum over the whole wave.
__device__ __forceinline__ float xor_sum(float x, int lo_mask) {
  for (int m = lo_mask; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

}  // namespace kda
