// Measured machine ceilings for the roofline of libkda's kernels (gfx950).
//
// Plain streaming kernels in the access patterns of libkda's paths, and a
// loop of independent bf16 matrix-core products.  Each is timed by the caller
// (HIP events around one launch); the achieved rates are the "measured peak"
// beside the published one.  Nothing here belongs to the method.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_probe.h"

namespace {

constexpr int NT = 1024;      // threads per streaming workgroup
constexpr int SPAN4 = NT;     // 16-byte elements per workgroup: one per thread (16 KiB)
constexpr int NTM = 256;      // threads per matrix-core workgroup (four waves)

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One 16 KiB span per workgroup, one non-temporal 16-byte access per thread
// and direction: the fastest streaming shape found on this chip (many short
// workgroups, every wave access one contiguous 1 KiB).
template <int MODE>
__global__ __launch_bounds__(NT) void stream_kernel(const f32x4* __restrict__ src,
                                                    f32x4* __restrict__ dst, size_t n4) {
  const size_t i = (size_t)blockIdx.x * SPAN4 + threadIdx.x;
  const bool in = i < n4;
  if (MODE == 0 && in) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
  if (MODE == 1 && in) __builtin_nontemporal_store(0.5f * __builtin_nontemporal_load(dst + i) + 1.f, dst + i);
  if (MODE == 3 && in) __builtin_nontemporal_store(f32x4{1.f, 1.f, 1.f, 1.f}, dst + i);
  if (MODE == 2) {
    const f32x4 x = in ? __builtin_nontemporal_load(src + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    float acc = (x[0] + x[1]) + (x[2] + x[3]);
    // one partial sum per workgroup: lanes, then the sixteen waves
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    __shared__ float part[NT / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
      float s = 0.f;
      for (int w = 0; w < NT / 64; ++w) s += part[w];
      reinterpret_cast<float*>(dst)[blockIdx.x] = s;
    }
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Operands fixed per lane: A and B fragments of 8 bf16 each (lane l, value
// 0.001 * ((l + j) & 7) and 0.001 * ((3 l + j) & 7) for j = 0..7).
__device__ __forceinline__ void probe_operands(bf16x8& a, bf16x8& b) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)((l + j) & 7));
    b[j] = (__bf16)(0.001f * (float)((l * 3 + j) & 7));
  }
}

// One MFMA accumulating in place.  Written as inline assembly so that the
// loop below is nothing but the MFMAs: with the compiler builtins, hipcc
// moves every accumulator between register files in each iteration of such
// a loop, and the probe then measures those moves.  Consecutive products
// write different accumulators (a dependent pair is eight products apart),
// so no wait states are needed between them.
#define KDA_MFMA_16(acc) \
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))
#define KDA_MFMA_32(acc) \
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))

// Each wave: `iters` rounds of eight independent products of one shape; the
// accumulators carry the dependence.  One fp32 per wave goes out: the sum
// over its lanes of every accumulator entry.
template <bool BIG>
__global__ __launch_bounds__(NTM) void mfma_kernel(int iters, float* __restrict__ out) {
  bf16x8 a, b;
  probe_operands(a, b);
  float s = 0.f;
  if constexpr (BIG) {
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
    for (int it = 0; it < iters; ++it) {
      KDA_MFMA_32(c0); KDA_MFMA_32(c1); KDA_MFMA_32(c2); KDA_MFMA_32(c3);
      KDA_MFMA_32(c4); KDA_MFMA_32(c5); KDA_MFMA_32(c6); KDA_MFMA_32(c7);
    }
    const f32x16 t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
#pragma unroll
    for (int e = 0; e < 16; ++e) s += t[e];
  } else {
    f32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
    for (int it = 0; it < iters; ++it) {
      KDA_MFMA_16(c0); KDA_MFMA_16(c1); KDA_MFMA_16(c2); KDA_MFMA_16(c3);
      KDA_MFMA_16(c4); KDA_MFMA_16(c5); KDA_MFMA_16(c6); KDA_MFMA_16(c7);
    }
    const f32x4 t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    s = (t[0] + t[1]) + (t[2] + t[3]);
  }
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (NTM / 64) + (threadIdx.x >> 6)] = s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" int kda_probe_hbm(int mode, const void* src, void* dst, size_t bytes, void* stream) {
  if (mode < 0 || mode > 3 || bytes == 0 || bytes % 64 != 0 || dst == nullptr || !aligned16(dst))
    return 1;
  if ((mode == 0 || mode == 2) && (src == nullptr || !aligned16(src))) return 1;
  if (mode == 0) {
    const char* s = static_cast<const char*>(src);
    const char* d = static_cast<const char*>(dst);
    if (s < d + bytes && d < s + bytes) return 1;  // overlapping copy
  }
  const size_t n4 = bytes / 16;
  const size_t grid = (n4 + SPAN4 - 1) / SPAN4;
  if (grid > 0x7fffffffu) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const f32x4* s4 = static_cast<const f32x4*>(src);
  f32x4* d4 = static_cast<f32x4*>(dst);
  const dim3 g((unsigned)grid), b(NT);
  switch (mode) {
    case 0: hipLaunchKernelGGL(stream_kernel<0>, g, b, 0, st, s4, d4, n4); break;
    case 1: hipLaunchKernelGGL(stream_kernel<1>, g, b, 0, st, s4, d4, n4); break;
    case 2: hipLaunchKernelGGL(stream_kernel<2>, g, b, 0, st, s4, d4, n4); break;
    default: hipLaunchKernelGGL(stream_kernel<3>, g, b, 0, st, s4, d4, n4); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

extern "C" int kda_probe_mfma_bf16(int shape, int32_t blocks, int32_t iters, float* out,
                                   void* stream) {
  if ((shape != 0 && shape != 1) || blocks < 1 || blocks > 65536 || iters < 1 ||
      iters > (1 << 24) || out == nullptr)
    return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape == 0)
    hipLaunchKernelGGL(mfma_kernel<true>, dim3(blocks), dim3(NTM), 0, st, iters, out);
  else
    hipLaunchKernelGGL(mfma_kernel<false>, dim3(blocks), dim3(NTM), 0, st, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
