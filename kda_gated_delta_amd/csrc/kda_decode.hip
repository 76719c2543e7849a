// Recurrent decode and multi-token verify of the KDA gated delta rule.
//
// One workgroup of up to 1024 threads per (request, head).  The head's
// K x V fp32 state is held in registers: thread t owns the float4 column
// group cg = t % (V/4) of the rows rg, rg + RG, rg + 2 RG, ... (rg = t /
// (V/4)), so each wave reads and writes whole 512-byte state rows with
// 128-bit non-temporal accesses, a thread holds only four of them (many
// loads in flight per CU), and the state crosses HBM exactly once in each
// direction.  The reductions over K (k.S', q.S' and q.k) are a butterfly
// inside the wave, then an LDS exchange across waves in two levels.
//
// Per token ("Linear attention" tutorial, sections "Gated DeltaNet" and
// "KDA：逐通道的遗忘门"):  S' = Diag(exp g) S;  v_hat = k S';
//   d = beta (v - v_hat);  S = S' + k^T d;  o = scale q S = scale (q S' + (q.k) d)
// The last identity is the decode read-out of the ReplaySSM analysis
// (section 3.12): it avoids a second pass over the updated state.
// A negative slot index marks a padding row (ReplaySSM analysis, section 3.6).

#include "kda.h"
#include "kda_common.h"
#include "kda_gate_math.h"
#include "kda_internal.h"

#include <type_traits>

namespace kda {
namespace {

// State columns per workgroup (all of them: whole 512-byte rows stream best).
template <int V>
constexpr int slice_cols() { return V; }

template <int K, int V>
struct StepShape {  // V: the columns one workgroup holds
  static constexpr int NT = (K * V / 4 < 1024) ? K * V / 4 : 1024;  // threads
  static constexpr int CG = V / 4;     // float4 column groups per row
  static constexpr int RG = NT / CG;   // row groups
  static constexpr int RPT = K / RG;   // state rows per thread
  static constexpr int NW = NT / 64;   // waves
  static constexpr int RED = NW * CG * 9 + CG * 9;  // reduction scratch (floats)
  static_assert(NT % 64 == 0 && RPT >= 1 && RG * RPT == K, "bad shape");
};

// Partial sums of one thread: k.S' (float4), q.S' (float4), q.k.
struct Partials {
  float4 vh, qs;
  float qk;
};

// Sums the partials of the threads sharing a column group.  red is an LDS
// buffer of RED floats (per-wave partials, then the column sums); the caller
// synchronises before reuse.
template <int K, int V>
__device__ __forceinline__ Partials reduce_rows(Partials p, float* red) {
  typedef StepShape<K, V> Sh;
  const int t = threadIdx.x;
  p.vh.x = xor_sum(p.vh.x, Sh::CG);
  p.vh.y = xor_sum(p.vh.y, Sh::CG);
  p.vh.z = xor_sum(p.vh.z, Sh::CG);
  p.vh.w = xor_sum(p.vh.w, Sh::CG);
  p.qs.x = xor_sum(p.qs.x, Sh::CG);
  p.qs.y = xor_sum(p.qs.y, Sh::CG);
  p.qs.z = xor_sum(p.qs.z, Sh::CG);
  p.qs.w = xor_sum(p.qs.w, Sh::CG);
  p.qk = xor_sum(p.qk, Sh::CG);
  if (Sh::NW == 1) return p;
  const int lane = t & 63, w = t >> 6, cg = t % Sh::CG;
  if (lane < Sh::CG) {
    float* dst = red + (w * Sh::CG + lane) * 9;
    dst[0] = p.vh.x; dst[1] = p.vh.y; dst[2] = p.vh.z; dst[3] = p.vh.w;
    dst[4] = p.qs.x; dst[5] = p.qs.y; dst[6] = p.qs.z; dst[7] = p.qs.w;
    dst[8] = p.qk;
  }
  __syncthreads();
  Partials s;
  if (Sh::NW <= 4) {
    s.vh = f4(0.f);
    s.qs = f4(0.f);
    s.qk = 0.f;
#pragma unroll
    for (int i = 0; i < Sh::NW; ++i) {
      const float* src = red + (i * Sh::CG + cg) * 9;
      s.vh = s.vh + make_float4(src[0], src[1], src[2], src[3]);
      s.qs = s.qs + make_float4(src[4], src[5], src[6], src[7]);
      s.qk += src[8];
    }
    return s;
  }
  // many waves: CG * 9 threads each sum one value over the waves, then every
  // thread reads the nine sums of its column group
  float* sums = red + Sh::NW * Sh::CG * 9;
  if (t < Sh::CG * 9) {
    const int c = t / 9, j = t % 9;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < Sh::NW; ++i) acc += red[(i * Sh::CG + c) * 9 + j];
    sums[t] = acc;
  }
  __syncthreads();
  const float* src = sums + cg * 9;
  s.vh = make_float4(src[0], src[1], src[2], src[3]);
  s.qs = make_float4(src[4], src[5], src[6], src[7]);
  s.qk = src[8];
  return s;
}

// Register-resident slice of a head's state owned by one thread.
template <int RPT>
struct Rows {
  float4 s[RPT];
};

// One token on the register-resident state.  sq/sk/sa hold q, k and exp(g)
// of the token in LDS; on return s[] holds the updated state and o the
// (unscaled) read-out q S of this thread's column group.
template <int K, int V>
__device__ __forceinline__ float4 token_step(Rows<StepShape<K, V>::RPT>& st,
                                             const float* sq, const float* sk,
                                             const float* sa, float4 vv,
                                             float beta, float* red) {
  typedef StepShape<K, V> Sh;
  const int rg = threadIdx.x / Sh::CG;
  float4* s = st.s;
  Partials p;
  p.vh = f4(0.f);
  p.qs = f4(0.f);
  p.qk = 0.f;
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) {
    const int row = rg + Sh::RG * i;
    s[i] = sa[row] * s[i];
    p.vh = fma4(sk[row], s[i], p.vh);
    p.qs = fma4(sq[row], s[i], p.qs);
    p.qk = fmaf(sq[row], sk[row], p.qk);
  }
  p = reduce_rows<K, V>(p, red);
  const float4 d = beta * (vv - p.vh);
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) s[i] = fma4(sk[rg + Sh::RG * i], d, s[i]);
  return fma4(p.qk, d, p.qs);
}

// ------------------------------------------------------ layer options

// Log decay of key channel c of token row `row` (r * H + h): the activated
// g, or the gate of the raw a ("Linear attention" tutorial, sections "Gated
// DeltaNet" and "KDA") with the gate kernel's own functions, so that the
// result is the value kda_gate_prep would have written.  A per-head gate
// (the Gated DeltaNet case) decays every channel alike.
__device__ __forceinline__ float gate_of(float x, int c, int K, int h, const StepOpts& op) {
  if (op.gate_mode == 0) return x;
  if (op.dt_bias) x = x + (op.per_head_gate ? op.dt_bias[h] : op.dt_bias[h * K + c]);
  const float rate = exp_split(op.A_log[h]);
  return op.gate_mode == 2 ? gate1<true>(x, rate, op.lower_bound)
                           : gate1<false>(x, rate, op.lower_bound);
}
__device__ __forceinline__ float decay_of(const float* __restrict__ g, int64_t row, int c, int K,
                                          int h, const StepOpts& op) {
  return gate_of(op.per_head_gate ? g[row] : g[row * K + c], c, K, h, op);
}

// Write strength of a token: beta, or sigmoid of the raw b.
__device__ __forceinline__ float strength_of(float b, const StepOpts& op) {
  return op.gate_mode != 0 ? sigmoid_fast(b) : b;
}

// Reciprocal L2 norms 1 / sqrt(sum x^2 + 1e-6) of the q and k rows of nb
// tokens (in-kernel normalisation, ReplaySSM analysis section 3.10), one
// wave per token; written to qn[j], kn[j].  All threads call it.
template <typename IO, int K, int NW, typename RowOf>
__device__ __forceinline__ void qk_rnorms(const IO* __restrict__ q, const IO* __restrict__ k,
                                          RowOf row_of, int nb, float* qn, float* kn) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int j = wv; j < nb; j += NW) {
    const int64_t row = row_of(j);
    float sq2 = 0.f, sk2 = 0.f;
    for (int c = lane; c < K; c += 64) {
      const float a = to_f32(q[row * K + c]), b = to_f32(k[row * K + c]);
      sq2 = fmaf(a, a, sq2);
      sk2 = fmaf(b, b, sk2);
    }
    sq2 = xor_sum(sq2, 1);
    sk2 = xor_sum(sk2, 1);
    if (lane == 0) {
      qn[j] = 1.f / sqrtf(sq2 + 1e-6f);
      kn[j] = 1.f / sqrtf(sk2 + 1e-6f);
    }
  }
}

// Gated RMSNorm of one (token, head) output (the layer's o_norm: RMS over the
// V columns, times a weight and an activation of the gate z): the CG
// threads of row group 0 hold o, four columns each, all in wave 0.  Every
// thread calls it (the sum is a butterfly over aligned groups of CG lanes).
template <typename IO, int V, int CG>
__device__ __forceinline__ float4 out_norm(float4 x, bool holder, const IO* __restrict__ z,
                                           int c0, const StepOpts& op) {
  float ss = holder ? fmaf(x.x, x.x, fmaf(x.y, x.y, fmaf(x.z, x.z, x.w * x.w))) : 0.f;
#pragma unroll
  for (int m = 1; m < CG; m <<= 1) ss += __shfl_xor(ss, m, 64);
  if (!holder) return x;
  const float f = 1.f / sqrtf(ss / (float)V + op.o_norm_eps);
  const float4 zz = load4(z + c0), w = load4(op.o_norm_w + c0);
  auto act = [&](float u) {
    const float sg = 1.f / (1.f + expf(-u));
    return op.o_gate_act ? u * sg : sg;
  };
  return make_float4(x.x * f * w.x * act(zz.x), x.y * f * w.y * act(zz.y),
                     x.z * f * w.z * act(zz.z), x.w * f * w.w * act(zz.w));
}

template <typename IO, int K, int V>
__global__ __launch_bounds__((StepShape<K, slice_cols<V>()>::NT)) void decode_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k,
    const IO* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, float scale, float* __restrict__ pool,
    const int32_t* __restrict__ slot_idx, int H, IO* __restrict__ o, StepOpts op,
    int64_t n_slots) {
  constexpr int VS = slice_cols<V>(), NS = V / VS;
  typedef StepShape<K, VS> Sh;
  __shared__ float sq[K], sk[K], sa[K];
  __shared__ float sn[2];
  __shared__ float red[Sh::RED];
  const int t = threadIdx.x, cg = t % Sh::CG, rg = t / Sh::CG;
  const int64_t rh = blockIdx.x / NS;  // r * H + h
  const int r = (int)(rh / H), h = (int)(rh % H);
  const int c0 = (blockIdx.x % NS) * VS + 4 * cg;  // this thread's first state column
  const int64_t slot = slot_idx[r];
  if (slot < 0 || slot >= n_slots) {
    // padding row: o = 0; a slot past the pool: o = NaN (a caller error made
    // visible).  Neither touches the pool.
    if (rg == 0) store4(o + rh * V + c0, f4(slot < 0 ? 0.f : __builtin_nanf("")));
    return;
  }
  float* S = pool + (slot * H + h) * (int64_t)(K * V);
  Rows<Sh::RPT> st;
  float4* s = st.s;
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) s[i] = load4_nt(S + (rg + Sh::RG * i) * V + c0);
  // q and k rows: grouped heads share them (value head h reads q/k head
  // h / (H / HK))
  const int HK = op.qk_heads > 0 ? op.qk_heads : H;
  const int64_t qk = (int64_t)r * HK + h / (H / HK);
  float qn = 1.f, kn = 1.f;
  if (op.qk_l2norm) {
    qk_rnorms<IO, K, Sh::NW>(q, k, [&](int) { return qk; }, 1, sn, sn + 1);
    __syncthreads();
    qn = sn[0];
    kn = sn[1];
  }
  for (int c = t; c < K; c += Sh::NT) {
    sq[c] = to_f32(q[qk * K + c]) * qn;
    sk[c] = to_f32(k[qk * K + c]) * kn;
    sa[c] = expf(decay_of(g, rh, c, K, h, op));
  }
  const float4 vv = load4(v + rh * V + c0);
  const float b = strength_of(beta[rh], op);
  __syncthreads();
  const float4 oq = token_step<K, VS>(st, sq, sk, sa, vv, b, red);
  float4 out = scale * oq;
  if (op.o_gate != nullptr)
    out = out_norm<IO, V, Sh::CG>(out, rg == 0, static_cast<const IO*>(op.o_gate) + rh * V, c0, op);
  if (rg == 0) store4(o + rh * V + c0, out);
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) store4_nt(S + (rg + Sh::RG * i) * V + c0, s[i]);
}

// Draft tokens are staged TVB at a time: q, k, exp(g), beta and v of a batch
// go to LDS before its first token, so the token steps issue no loads.
constexpr int TVB = 8;

template <typename IO, int K, int V>
__global__ __launch_bounds__((StepShape<K, slice_cols<V>()>::NT)) void verify_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k,
    const IO* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, float scale,
    const float* __restrict__ pool, const int32_t* __restrict__ slot_idx,
    int Tv, int H, float* __restrict__ inter, IO* __restrict__ o, StepOpts op, int64_t n_slots) {
  constexpr int VS = slice_cols<V>(), NS = V / VS;
  typedef StepShape<K, VS> Sh;
  __shared__ float sq[TVB][K], sk[TVB][K], sa[TVB][K], sb[TVB];
  __shared__ __align__(16) float sv[TVB][VS];
  __shared__ float sqn[TVB], skn[TVB];
  __shared__ __align__(16) float sout[TVB][V];
  __shared__ float red[2][Sh::RED];
  const int t = threadIdx.x, cg = t % Sh::CG, rg = t / Sh::CG;
  const int rh = blockIdx.x / NS;  // r * H + h
  const int r = rh / H, h = rh % H;
  const int v0 = (blockIdx.x % NS) * VS;  // first state column of the workgroup
  const int c0 = v0 + 4 * cg;             // this thread's first state column
  const int64_t slot = slot_idx[r];
  if (slot < 0 || slot >= n_slots) {
    // padding row: o = 0; a slot past the pool: o = NaN.  inter stays unwritten.
    if (rg == 0)
      for (int s = 0; s < Tv; ++s)
        store4(o + (((int64_t)r * Tv + s) * H + h) * V + c0,
               f4(slot < 0 ? 0.f : __builtin_nanf("")));
    return;
  }
  const float* S0 = pool + (slot * H + h) * (int64_t)(K * V);
  Rows<Sh::RPT> st;
  float4* s = st.s;
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) s[i] = load4_nt(S0 + (rg + Sh::RG * i) * V + c0);
  int step = 0;
  for (int s0 = 0; s0 < Tv; s0 += TVB) {
    const int nb = (Tv - s0 < TVB) ? Tv - s0 : TVB;
    if (s0 > 0) __syncthreads();  // previous batch fully consumed
    // q/k rows of the batch's tokens (grouped heads share them)
    const int HK = op.qk_heads > 0 ? op.qk_heads : H;
    if (op.qk_l2norm) {
      qk_rnorms<IO, K, Sh::NW>(
          q, k, [&](int j) { return ((int64_t)r * Tv + s0 + j) * HK + h / (H / HK); }, nb, sqn,
          skn);
      __syncthreads();
    }
    for (int e = t; e < nb * K; e += Sh::NT) {
      const int j = e / K, c = e % K;
      const int64_t row = ((int64_t)r * Tv + s0 + j) * H + h;
      const int64_t qrow = ((int64_t)r * Tv + s0 + j) * HK + h / (H / HK);
      const float qn = op.qk_l2norm ? sqn[j] : 1.f, kn = op.qk_l2norm ? skn[j] : 1.f;
      sq[j][c] = to_f32(q[qrow * K + c]) * qn;
      sk[j][c] = to_f32(k[qrow * K + c]) * kn;
      sa[j][c] = expf(decay_of(g, row, c, K, h, op));
    }
    for (int e = t; e < nb * VS; e += Sh::NT) {
      const int j = e / VS, c = e % VS;
      sv[j][c] = to_f32(v[(((int64_t)r * Tv + s0 + j) * H + h) * V + v0 + c]);
    }
    if (t < nb) sb[t] = strength_of(beta[((int64_t)r * Tv + s0 + t) * H + h], op);
    __syncthreads();
    // Every load of the batch (and the initial state) has landed here.  The
    // explicit wait keeps the compiler from waiting inside the token steps,
    // where stores are in flight and any wait on the memory counter would
    // also wait for them.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
    for (int j = 0; j < TVB; ++j) {
      if (j < nb) {
        const int64_t rsh = ((int64_t)r * Tv + s0 + j) * H + h;
        const float4 vv = *reinterpret_cast<const float4*>(&sv[j][4 * cg]);
        const float4 oq = token_step<K, VS>(st, sq[j], sk[j], sa[j], vv, sb[j],
                                            red[step & 1]);
        ++step;
        if (rg == 0) {
          if (op.o_gate != nullptr)  // normalised after the batch
            *reinterpret_cast<float4*>(&sout[j][c0]) = scale * oq;
          else
            store4(o + rsh * V + c0, scale * oq);
        }
        float* I = inter + rsh * (int64_t)(K * V);
#pragma unroll
        for (int i = 0; i < Sh::RPT; ++i) store4_nt(I + (rg + Sh::RG * i) * V + c0, s[i]);
      }
    }
    if (op.o_gate != nullptr) {
      // gated RMSNorm of the batch's outputs, one wave per token
      __syncthreads();
      const int lane = t & 63, wv = t >> 6;
      for (int j = wv; j < nb; j += Sh::NW) {
        const int64_t rsh = ((int64_t)r * Tv + s0 + j) * H + h;
        const bool holder = lane < Sh::CG;
        const float4 x = holder ? *reinterpret_cast<const float4*>(&sout[j][4 * lane]) : f4(0.f);
        const float4 y = out_norm<IO, V, Sh::CG>(x, holder, static_cast<const IO*>(op.o_gate) + rsh * V,
                                                 4 * lane, op);
        if (holder) store4(o + rsh * V + 4 * lane, y);
      }
    }
  }
}

// ---------------------------------------------------------------- replay

// Buffered ("replay") decode (ReplaySSM analysis, sections 2 and 3): the pool
// holds a checkpoint S0 that is only read, and a per-(slot, head) ring keeps
// (d_j, k_j, g_j) of the m = write_pos tokens decoded since the checkpoint.
// The state before the current token is
//   S_m = Diag(e^{G_m}) S0 + sum_j Diag(e^{G_m - G_j}) k_j^T d_j,
// G_j the sum of g_1 .. g_j.  The current token decays it by a = e^{g}; its
// products with k and q need no rebuilt state: with A = a e^{G_m} and
// w_j = a e^{G_m - G_j} (per key channel),
//   k S' = (k A) S0 + sum_j (k . (w_j k_j)) d_j,  and the same for q,
// one pass over S0 plus m dot products of length K.  Then d = beta (v - k S'),
// o = scale (q S' + (q.k) d).  At the ring's last position (or when forced)
// the state S' + k^T d is written back as the new checkpoint; otherwise
// (d, k, g) is appended at write_pos.  With an empty ring every operation is
// that of the plain decode step in the same order, so the results are
// bit-identical to it.
constexpr int RING_MAX = KDA_RING_MAX;

template <typename IO, int K, int V, bool OPT>
__global__ __launch_bounds__((StepShape<K, V>::NT)) __attribute__((amdgpu_waves_per_eu(StepShape<K, V>::NT == 1024 ? 8 : 1))) void replay_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float scale,
    float* __restrict__ pool, const int32_t* __restrict__ slot_idx,
    const int32_t* __restrict__ write_pos, const int32_t* __restrict__ force_flush, int L,
    float* __restrict__ ring_d, IO* __restrict__ ring_k, float* __restrict__ ring_g, int H,
    IO* __restrict__ o, int32_t* __restrict__ next_pos, StepOpts op, int64_t n_slots) {
  typedef StepShape<K, V> Sh;
  __shared__ float sq[K], sk[K], sa[K], sg[K];
  __shared__ __align__(16) float swk[RING_MAX][K], sgr[RING_MAX][K], sd[RING_MAX][V];
  __shared__ float sck[RING_MAX], scq[RING_MAX];
  __shared__ float snq[2], snr[RING_MAX];  // L2 norm option: token q, k; ring k rows
  __shared__ float sdump[3];
  __shared__ float spart[Sh::NT / K][K];
  __shared__ float red[Sh::RED];
  const int t = threadIdx.x, cg = t % Sh::CG, rg = t / Sh::CG;
  const int64_t rh = blockIdx.x;  // r * H + h
  const int r = (int)(rh / H), h = (int)(rh % H);
  const int c0 = 4 * cg;
  const int64_t slot = slot_idx[r];
  const int pos = write_pos[r];
  if (slot < 0 || slot >= n_slots || pos < 0 || pos >= L) {
    // padding row: o = 0; a slot past the pool or a cursor outside the
    // ring: o = NaN (a caller error made visible).  None touches the pool
    // or the ring.
    if (rg == 0) store4(o + rh * V + c0, f4(slot < 0 ? 0.f : __builtin_nanf("")));
    if (h == 0 && t == 0 && next_pos != nullptr) next_pos[r] = pos;
    return;
  }
  const bool flush = pos == L - 1 || (force_flush != nullptr && force_flush[r] != 0);
  const int m = pos;  // ring entries since the checkpoint
  float* S = pool + (slot * H + h) * (int64_t)(K * V);
  const int64_t e0 = (slot * H + h) * (int64_t)L;  // ring entry (slot, h, 0)
  // Every load is unconditional and the small ones go first: ring entries
  // 0 .. m-1 and the token's q, k, g are buffer resources whose range ends
  // there (reads past it return zero without touching memory), then the
  // checkpoint.  Staging the small ones in LDS then waits for them alone,
  // and the ring arithmetic below runs while the checkpoint is in flight.
  // option-dependent addresses first, so that the loads below form one
  // straight block: grouped heads read q/k head h / (H / HK), a per-head
  // gate is one word
  // (OPT: the kernel instance that reads the options; the other one is the
  // plain step, with no option code at all)
  const int HK = OPT && op.qk_heads > 0 ? op.qk_heads : H;
  const int64_t qk = OPT ? (int64_t)r * HK + h / (H / HK) : rh;
  const bool ph = OPT && op.per_head_gate;
  constexpr int RK = (RING_MAX * K / 4 + Sh::NT - 1) / Sh::NT;  // 4-channel groups
  constexpr int RD = (RING_MAX * V / 4 + Sh::NT - 1) / Sh::NT;  // 4-column groups
  typedef typename std::conditional<sizeof(IO) == 2, uint2, uint4>::type RawK;
  const auto rk = buffer_rsrc(ring_k + e0 * K, (uint32_t)(m * K * sizeof(IO)));
  const auto rgr = buffer_rsrc(ring_g + e0 * K, (uint32_t)(m * K * 4));
  const auto rd = buffer_rsrc(ring_d + e0 * V, (uint32_t)(m * V * 4));
  RawK kr[RK];
  float4 gr[RK], dr[RD];
#pragma unroll
  for (int i = 0; i < RK; ++i) {
    const uint32_t e = (uint32_t)(t + i * Sh::NT) * 4;  // first element of the group
    if constexpr (sizeof(IO) == 2)
      kr[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, e * 2, 0, 0));
    else
      kr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, e * 4, 0, 0));
    gr[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rgr, e * 4, 0, 0));
  }
#pragma unroll
  for (int i = 0; i < RD; ++i) {
    const uint32_t e = (uint32_t)(t + i * Sh::NT) * 4;
    dr[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rd, e * 4, 0, 0));
  }
  // the token: thread c < K holds channel c of q, k and g (K <= NT)
  static_assert(K <= Sh::NT, "one channel per thread");
  float tq, tk, tg;
  {
    const uint32_t off = (uint32_t)t * (uint32_t)sizeof(IO);
    if constexpr (sizeof(IO) == 2) {
      tq = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
               buffer_rsrc(q + qk * K, K * 2), off, 0, 0) << 16);
      tk = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
               buffer_rsrc(k + qk * K, K * 2), off, 0, 0) << 16);
    } else {
      tq = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
               buffer_rsrc(q + qk * K, K * 4), off, 0, 0));
      tk = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
               buffer_rsrc(k + qk * K, K * 4), off, 0, 0));
    }
    // (a per-head gate is one word, which every channel reads)
    tg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
             ph ? buffer_rsrc(g + rh, 4) : buffer_rsrc(g + rh * K, K * 4),
             ph ? 0u : (uint32_t)t * 4, 0, 0));
  }
  const float4 vv = load4(v + rh * V + c0);
  const float braw = beta[rh];
  Rows<Sh::RPT> st;
  float4* s = st.s;
  __builtin_amdgcn_sched_barrier(0);  // keep the checkpoint's loads last
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) s[i] = load4_nt(S + (rg + Sh::RG * i) * V + c0);
  // stage the ring and the token in LDS (threads past K store to a dump
  // word: a store on every thread keeps the token's loads ahead of the
  // checkpoint's instead of sunk into a branch behind them)
  {
    const bool tok = t < K;
    *(tok ? sq + t : sdump) = tq;
    *(tok ? sk + t : sdump + 1) = tk;
    *(tok ? sg + t : sdump + 2) = tg;
  }
#pragma unroll
  for (int i = 0; i < RK; ++i) {
    const int e = (t + i * Sh::NT) * 4, j = e / K, c = e % K;
    if (j < RING_MAX) {
      float4 kf;
      if constexpr (sizeof(IO) == 2)
        kf = make_float4(__uint_as_float(kr[i].x << 16), __uint_as_float(kr[i].x & 0xffff0000u),
                         __uint_as_float(kr[i].y << 16), __uint_as_float(kr[i].y & 0xffff0000u));
      else
        kf = __builtin_bit_cast(float4, kr[i]);
      *reinterpret_cast<float4*>(&swk[j][c]) = kf;
      *reinterpret_cast<float4*>(&sgr[j][c]) = gr[i];
    }
  }
#pragma unroll
  for (int i = 0; i < RD; ++i) {
    const int e = (t + i * Sh::NT) * 4, j = e / V, c = e % V;
    if (j < RING_MAX) *reinterpret_cast<float4*>(&sd[j][c]) = dr[i];
  }
  __syncthreads();
  if (OPT && op.gate_mode != 0) {  // the gate from the raw a, in place
    if (t < K) sg[t] = gate_of(sg[t], t, K, h, op);
    __syncthreads();
  }
  if (OPT && op.qk_l2norm) {
    // The token's q and k by the decode kernel's own norms.  The ring keeps
    // raw k rows (exact in the io dtype); each entry's row is normalised
    // here again, before its decay weight multiplies it: entry j's LPE
    // lanes sum its squares, every LPE-th channel each.
    qk_rnorms<IO, K, Sh::NW>(q, k, [&](int) { return qk; }, 1, snq, snq + 1);
    constexpr int LPE = Sh::NT / RING_MAX, CPL = K / LPE;
    const int j = t / LPE, pl = t % LPE;
    float ss = 0.f;
    if (j < m) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) ss = fmaf(swk[j][pl + LPE * i], swk[j][pl + LPE * i], ss);
    }
#pragma unroll
    for (int x = 1; x < LPE; x <<= 1) ss += __shfl_xor(ss, x, 64);
    if (pl == 0 && j < m) snr[j] = 1.f / sqrtf(ss + 1e-6f);
    __syncthreads();
    if (t < K) {
      sq[t] *= snq[0];
      sk[t] *= snq[1];
    }
    for (int e = t; e < m * K; e += Sh::NT) swk[e / K][e % K] *= snr[e / K];
    __syncthreads();
  }
  const float b = OPT ? strength_of(braw, op) : braw;
  // Decay weights per key channel, newest entry first: w_j k_j in place of
  // k_j, then A.  The NG = NT / K thread groups of a channel take EPG
  // consecutive entries each; a group starts from the sum of the current g
  // and of the entries of the groups after it.
  {
    constexpr int NG = Sh::NT / K, EPG = (RING_MAX + NG - 1) / NG;
    const int c = t % K, grp = t / K, j0 = grp * EPG;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < EPG; ++i)
      if (j0 + i < m) part += sgr[j0 + i][c];
    spart[grp][c] = part;
    __syncthreads();
    float suf = sg[c];
    for (int q2 = NG - 1; q2 > grp; --q2) suf += spart[q2][c];
#pragma unroll
    for (int i = EPG - 1; i >= 0; --i) {
      const int j = j0 + i;
      if (j < m) {
        swk[j][c] *= expf(suf);
        suf += sgr[j][c];
      }
    }
    if (grp == 0) sa[c] = expf(suf);
  }
  __syncthreads();
  // ring coefficients k . (w_j k_j) and q . (w_j k_j): LPE lanes per entry,
  // each over every LPE-th channel, then summed across the group
  {
    constexpr int LPE = Sh::NT / RING_MAX, CPL = K / LPE;
    static_assert(LPE >= 1 && LPE <= 64 && CPL >= 1, "entry groups fit a wave");
    const int j = t / LPE, pl = t % LPE;
    float pk = 0.f, pq = 0.f;
    if (j < m) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = pl + LPE * i;
        pk = fmaf(sk[c], swk[j][c], pk);
        pq = fmaf(sq[c], swk[j][c], pq);
      }
    }
#pragma unroll
    for (int x = 1; x < LPE; x <<= 1) {
      pk += __shfl_xor(pk, x, 64);
      pq += __shfl_xor(pq, x, 64);
    }
    if (pl == 0 && j < m) {
      sck[j] = pk;
      scq[j] = pq;
    }
  }
  __syncthreads();
  Partials p;
  p.vh = f4(0.f);
  p.qs = f4(0.f);
  p.qk = 0.f;
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) {
    const int row = rg + Sh::RG * i;
    s[i] = sa[row] * s[i];
    p.vh = fma4(sk[row], s[i], p.vh);
    p.qs = fma4(sq[row], s[i], p.qs);
    p.qk = fmaf(sq[row], sk[row], p.qk);
  }
  for (int j = rg; j < m; j += Sh::RG) {
    const float4 dj = *reinterpret_cast<const float4*>(&sd[j][c0]);
    p.vh = fma4(sck[j], dj, p.vh);
    p.qs = fma4(scq[j], dj, p.qs);
  }
  p = reduce_rows<K, V>(p, red);
  const float4 d = b * (vv - p.vh);
  const float4 oq = fma4(p.qk, d, p.qs);
  float4 out = scale * oq;
  if (OPT && op.o_gate != nullptr)  // the layer's gated RMSNorm, as in decode
    out = out_norm<IO, V, Sh::CG>(out, rg == 0, static_cast<const IO*>(op.o_gate) + rh * V, c0, op);
  if (rg == 0) store4(o + rh * V + c0, out);
  if (flush) {
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) s[i] = fma4(sk[rg + Sh::RG * i], d, s[i]);
    for (int j = 0; j < m; ++j) {
      const float4 dj = *reinterpret_cast<const float4*>(&sd[j][c0]);
#pragma unroll
      for (int i = 0; i < Sh::RPT; ++i) s[i] = fma4(swk[j][rg + Sh::RG * i], dj, s[i]);
    }
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) store4_nt(S + (rg + Sh::RG * i) * V + c0, s[i]);
  } else {
    if (rg == 0) store4(ring_d + (e0 + pos) * V + c0, d);
    if (t < K) {  // k as read (raw: exact in io), g as activated
      ring_k[(e0 + pos) * K + t] = from_f32<IO>(tk);
      ring_g[(e0 + pos) * K + t] = OPT ? sg[t] : tg;
    }
  }
  if (h == 0 && t == 0 && next_pos != nullptr) next_pos[r] = flush ? 0 : pos + 1;
}

template <typename IO, int K, int V>
hipError_t launch_replay(const ReplayArgs& a, hipStream_t stream) {
  typedef StepShape<K, V> Sh;
  const bool opt = a.opts.gate_mode != 0 || a.opts.per_head_gate != 0 ||
                   (a.opts.qk_heads > 0 && a.opts.qk_heads != a.H) || a.opts.qk_l2norm != 0 ||
                   a.opts.o_gate != nullptr;
  hipLaunchKernelGGL((opt ? replay_kernel<IO, K, V, true> : replay_kernel<IO, K, V, false>),
                     dim3((unsigned)a.B * a.H), dim3(Sh::NT), 0, stream, (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, a.g, a.beta,
                     a.scale, a.pool, a.slot_idx, a.write_pos, a.force_flush, a.L, a.ring_d,
                     (IO*)a.ring_k, a.ring_g, a.H, (IO*)a.o, a.next_pos, a.opts, a.n_slots);
  return hipGetLastError();
}

template <typename IO, int K>
hipError_t replay_v(const ReplayArgs& a, hipStream_t st) {
  switch (a.V) {
    case 16: return launch_replay<IO, K, 16>(a, st);
    case 32: return launch_replay<IO, K, 32>(a, st);
    case 64: return launch_replay<IO, K, 64>(a, st);
    case 128: return launch_replay<IO, K, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename IO>
hipError_t replay_k(const ReplayArgs& a, hipStream_t st) {
  switch (a.K) {
    case 16: return replay_v<IO, 16>(a, st);
    case 32: return replay_v<IO, 32>(a, st);
    case 64: return replay_v<IO, 64>(a, st);
    case 128: return replay_v<IO, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename IO, int K, int V>
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  typedef StepShape<K, slice_cols<V>()> Sh;
  hipLaunchKernelGGL((decode_kernel<IO, K, V>), dim3((unsigned)a.B * a.H * (V / slice_cols<V>())),
                     dim3(Sh::NT), 0, stream, (const IO*)a.q, (const IO*)a.k, (const IO*)a.v,
                     a.g, a.beta, a.scale, a.pool, a.slot_idx, a.H, (IO*)a.o, a.opts, a.n_slots);
  return hipGetLastError();
}

template <typename IO, int K, int V>
hipError_t launch_verify(const DecodeArgs& a, hipStream_t stream) {
  typedef StepShape<K, slice_cols<V>()> Sh;
  hipLaunchKernelGGL((verify_kernel<IO, K, V>), dim3((unsigned)a.B * a.H * (V / slice_cols<V>())),
                     dim3(Sh::NT), 0, stream, (const IO*)a.q, (const IO*)a.k, (const IO*)a.v,
                     a.g, a.beta, a.scale, a.pool, a.slot_idx, a.Tv, a.H, a.inter, (IO*)a.o,
                     a.opts, a.n_slots);
  return hipGetLastError();
}

template <typename IO, int K>
hipError_t decode_v(const DecodeArgs& a, hipStream_t st) {
  switch (a.V) {
    case 16: return launch_decode<IO, K, 16>(a, st);
    case 32: return launch_decode<IO, K, 32>(a, st);
    case 64: return launch_decode<IO, K, 64>(a, st);
    case 128: return launch_decode<IO, K, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename IO>
hipError_t decode_k(const DecodeArgs& a, hipStream_t st) {
  switch (a.K) {
    case 16: return decode_v<IO, 16>(a, st);
    case 32: return decode_v<IO, 32>(a, st);
    case 64: return decode_v<IO, 64>(a, st);
    case 128: return decode_v<IO, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename IO, int K>
hipError_t verify_v(const DecodeArgs& a, hipStream_t st) {
  switch (a.V) {
    case 16: return launch_verify<IO, K, 16>(a, st);
    case 32: return launch_verify<IO, K, 32>(a, st);
    case 64: return launch_verify<IO, K, 64>(a, st);
    case 128: return launch_verify<IO, K, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename IO>
hipError_t verify_k(const DecodeArgs& a, hipStream_t st) {
  switch (a.K) {
    case 16: return verify_v<IO, 16>(a, st);
    case 32: return verify_v<IO, 32>(a, st);
    case 64: return verify_v<IO, 64>(a, st);
    case 128: return verify_v<IO, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t run_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.bf16_io ? decode_k<bf16>(a, stream) : decode_k<float>(a, stream);
}

hipError_t run_verify(const DecodeArgs& a, hipStream_t stream) {
  return a.bf16_io ? verify_k<bf16>(a, stream) : verify_k<float>(a, stream);
}

hipError_t run_replay(const ReplayArgs& a, hipStream_t stream) {
  return a.bf16_io ? replay_k<bf16>(a, stream) : replay_k<float>(a, stream);
}

}  // namespace kda
