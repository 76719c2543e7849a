// Gate activation of KDA ("Linear attention" tutorial, sections
// "Gated DeltaNet" and "KDA：逐通道的遗忘门"):
//   g    = -exp(A_log[h]) * softplus(a + dt_bias[h, c])         (lower_bound = 0)
//   g    = lower_bound * sigmoid(exp(A_log[h]) * (a + dt_bias))  (safe gate)
//   beta = sigmoid(b)
// softplus(x) = x above the threshold 20, as in the kernels analysed on the
// ReplaySSM page (section 3.8) and the target-verify PR report.
//
// Purely elementwise and HBM-bound: 128-bit loads and stores over float4
// groups of the [T*H, K] row-major gate tensor.

#include "kda_common.h"
#include "kda_gate_math.h"
#include "kda_internal.h"

namespace kda {
namespace {

// Each thread takes UNROLL float4 groups, a block-stride apart, and issues
// all of their loads before any arithmetic (several 16-byte loads in flight
// per thread); a block covers UNROLL * 256 / (K / 4) whole (token, head)
// rows, whose beta its first threads compute.
constexpr int GATE_UNROLL = 4;

template <int K, bool SAFE>
__global__ __launch_bounds__(256) void gate_kernel(
    const float* __restrict__ a, const float* __restrict__ b,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    int64_t TH, int H, float lb, float* __restrict__ g,
    float* __restrict__ beta) {
  constexpr int Q = K / 4;  // float4 groups per (token, head) row
  constexpr int ROWS = GATE_UNROLL * 256 / Q;
  const int64_t n4 = TH * Q;
  const int64_t base = (int64_t)blockIdx.x * (GATE_UNROLL * 256) + threadIdx.x;
  float4 x[GATE_UNROLL];
#pragma unroll
  for (int u = 0; u < GATE_UNROLL; ++u) {
    const int64_t i = base + u * 256;
    x[u] = i < n4 ? load4(a + i * 4) : f4(0.f);
  }
  // b of this block's rows
  const int64_t row0 = (int64_t)blockIdx.x * ROWS;
  const bool has_b = threadIdx.x < ROWS && row0 + threadIdx.x < TH;
  const float bb = has_b ? b[row0 + threadIdx.x] : 0.f;
#pragma unroll
  for (int u = 0; u < GATE_UNROLL; ++u) {
    const int64_t i = base + u * 256;
    if (i < n4) {
      const int c = (int)(i % Q) * 4;
      const int h = (int)((uint64_t)(i / Q) % (uint32_t)H);
      const float rate = exp_split(A_log[h]);
      float4 y = x[u];
      if (dt_bias) y = y + load4(dt_bias + h * K + c);
      store4(g + i * 4, make_float4(gate1<SAFE>(y.x, rate, lb), gate1<SAFE>(y.y, rate, lb),
                                    gate1<SAFE>(y.z, rate, lb), gate1<SAFE>(y.w, rate, lb)));
    }
  }
  if (has_b) beta[row0 + threadIdx.x] = sigmoid_fast(bb);
}

template <int K>
hipError_t launch_gate(const GateArgs& p, hipStream_t st) {
  const int64_t TH = p.T * p.H;
  const int64_t n4 = TH * (K / 4);
  const int64_t per_block = GATE_UNROLL * 256;
  const int64_t blocks = (n4 + per_block - 1) / per_block;
  if (blocks < 1) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
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
