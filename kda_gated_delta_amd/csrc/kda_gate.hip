// Gate activation of KDA ("Linear attention" tutorial, sections
// "Gated DeltaNet" and "KDA：逐通道的遗忘门"):
//   g    = -exp(A_log[h]) * softplus(a + dt_bias[h, c])         (lower_bound = 0)
//   g    = lower_bound * sigmoid(exp(A_log[h]) * (a + dt_bias))  (safe gate)
//   beta = sigmoid(b)
// softplus(x) = x above the threshold 20, as in the kernels analysed on the
// ReplaySSM page (section 3.8) and the target-verify PR report.
//
// Purely elementwise and HBM-bound: 128-bit loads and stores, a grid-stride
// loop over float4 groups of the [T*H, K] row-major gate tensor.

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <bool SAFE>
__device__ __forceinline__ float gate1(float x, float rate, float lb) {
  if (SAFE) return lb / (1.f + expf(-rate * x));
  const float sp = x > 20.f ? x : log1pf(expf(x));
  return -rate * sp;
}

template <int K, bool SAFE>
__global__ __launch_bounds__(256) void gate_kernel(
    const float* __restrict__ a, const float* __restrict__ b,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    int64_t TH, int H, float lb, float* __restrict__ g,
    float* __restrict__ beta) {
  constexpr int Q = K / 4;  // float4 groups per (token, head) row
  const int64_t n4 = TH * Q;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += stride) {
    const uint32_t row = (uint32_t)(i / Q);
    const int c = (int)(i % Q) * 4;
    const int h = (int)(row % (uint32_t)H);
    const float rate = expf(A_log[h]);
    float4 x = load4(a + i * 4);
    if (dt_bias) x = x + load4(dt_bias + h * K + c);
    store4(g + i * 4, make_float4(gate1<SAFE>(x.x, rate, lb), gate1<SAFE>(x.y, rate, lb),
                                  gate1<SAFE>(x.z, rate, lb), gate1<SAFE>(x.w, rate, lb)));
  }
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < TH; i += stride)
    beta[i] = 1.f / (1.f + expf(-b[i]));
}

template <int K>
hipError_t launch_gate(const GateArgs& p, hipStream_t st) {
  const int64_t TH = p.T * p.H;
  const int64_t n4 = TH * (K / 4);
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;  // grid-stride beyond 64 blocks per CU
  if (blocks < 1) blocks = 1;
  if (p.lower_bound != 0.f)
    hipLaunchKernelGGL((gate_kernel<K, true>), dim3((unsigned)blocks), dim3(256), 0, st,
                       p.a, p.b, p.A_log, p.dt_bias, TH, p.H, p.lower_bound, p.g, p.beta);
  else
    hipLaunchKernelGGL((gate_kernel<K, false>), dim3((unsigned)blocks), dim3(256), 0, st,
                       p.a, p.b, p.A_log, p.dt_bias, TH, p.H, p.lower_bound, p.g, p.beta);
  return hipGetLastError();
}

}  // namespace

hipError_t run_gate(const GateArgs& p, hipStream_t stream) {
  switch (p.K) {
    case 16: return launch_gate<16>(p, stream);
    case 32: return launch_gate<32>(p, stream);
    case 64: return launch_gate<64>(p, stream);
    case 128: return launch_gate<128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
