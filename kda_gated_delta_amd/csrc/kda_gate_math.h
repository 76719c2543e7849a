// Gate activation math of KDA, shared by the gate kernel and the gated
// prefill ("Linear attention" tutorial, sections "Gated DeltaNet" and "KDA"):
//   softplus gate  g = -exp(A_log) * softplus(x),   x = a + dt_bias
//   safe gate      g = lower_bound * sigmoid(exp(A_log) * x)
//   beta = sigmoid(b)
// with softplus(x) = x above the threshold 20.  Both users call these same
// functions, so a gate computed inside the prefill is bit-identical to the
// one the gate kernel writes.
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

// e^y on the hardware base-2 exponential.  y log2(e) is formed with its
// rounding error carried separately (Cody and Waite's argument splitting:
// log2(e) = L2E_HI + L2E_LO, the product error recovered by an fma), so the
// result stays within a few ulp for large |y| instead of losing |y| 2^-24
// relative to the rounding of the product.  Overflows to +inf above ~88.7,
// underflows to 0 below ~-87.3 (denormal results are flushed).
__device__ __forceinline__ float exp_split(float y) {
  constexpr float L2E_HI = 1.4426950216293335f;  // log2(e) rounded to fp32
  constexpr float L2E_LO = 1.925963033500011e-08f;  // log2(e) - L2E_HI
  constexpr float LN2 = 0.6931471824645996f;
  const float p = y * L2E_HI;
  const float pl = fmaf(y, L2E_HI, -p) + y * L2E_LO;
  return __builtin_amdgcn_exp2f(p) * fmaf(pl, LN2, 1.f);
}

// log(1 + u) for u in [0, 1].  Below 2^-8 the series u - u^2/2 + u^3/3
// (truncation below u^3/4 relative); above, Goldberg's correction of a
// rounded log: with w = 1 + u rounded, log(w) * u / (w - 1) (w - 1 is exact
// since w lies in [1, 2]).
__device__ __forceinline__ float log1p_unit(float u) {
  constexpr float LN2 = 0.6931471824645996f;
  const float series = u * fmaf(u, fmaf(u, 0.3333333432674408f, -0.5f), 1.f);
  const float w = 1.f + u;
  const float corrected = __builtin_amdgcn_logf(w) * LN2 * (u * __builtin_amdgcn_rcpf(w - 1.f));
  return u < 0x1p-8f ? series : corrected;
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log(1 + e^-|x|), and x itself
// above the threshold 20.
__device__ __forceinline__ float softplus20(float x) {
  const float sp = fmaxf(x, 0.f) + log1p_unit(exp_split(-fabsf(x)));
  return x > 20.f ? x : sp;
}

// sigmoid(z) = 1 / (1 + e^-z); e^-z overflowing to +inf gives 0.
__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.f + exp_split(-z));
}

template <bool SAFE>
__device__ __forceinline__ float gate1(float x, float rate, float lb) {
  if (SAFE) return lb * sigmoid_fast(rate * x);
  return -rate * softplus20(x);
}

}  // namespace kda
