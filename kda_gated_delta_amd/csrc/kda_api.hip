// C ABI of libkda (declared in include/kda.h): argument validation, status
// codes, and dispatch to the kernel launchers.  Nothing here allocates,
// synchronises or keeps state; every launch goes to the caller's stream.

#include "kda.h"
#include "kda_profile.h"

#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <vector>
#include "kda_internal.h"

namespace {

bool head_dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned8(const void* p) { return ((uintptr_t)p & 7u) == 0; }

// io tensors whose rows are read as 4-element groups need 8-byte alignment
// (bf16) or 16-byte alignment (fp32).
bool io_aligned(kda_dtype io, const void* p) {
  return io == KDA_BF16 ? aligned8(p) : aligned16(p);
}

kda_status launch_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH; }

// Debug checks of the device-resident preconditions, on when the environment
// variable KDA_CHECK is "1" (read at every call): the index arrays are copied
// to the host, which waits for the stream, and checked before anything is
// enqueued.  Off (the default), nothing is read back and nothing waits.
bool debug_checks() {
  const char* e = std::getenv("KDA_CHECK");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

kda_status read_back(const int32_t* src, size_t n, hipStream_t st, std::vector<int32_t>& dst) {
  dst.resize(n);
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return KDA_ERR_LAUNCH;
  return KDA_OK;
}

// cu_seqlens: cu[0] = 0, cu[N] = T, non-decreasing.
kda_status check_cu(const int32_t* cu, int32_t N, int64_t T, hipStream_t st) {
  std::vector<int32_t> h;
  if (kda_status s = read_back(cu, (size_t)N + 1, st, h)) return s;
  if (h[0] != 0 || h[N] != T) return KDA_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < N; ++i)
    if (h[i + 1] < h[i]) return KDA_ERR_INVALID_ARGUMENT;
  return KDA_OK;
}

// slot_idx: every live (non-negative) slot below n_slots, no slot twice.
kda_status check_slots(const int32_t* idx, int32_t B, int64_t n_slots, hipStream_t st) {
  std::vector<int32_t> h;
  if (kda_status s = read_back(idx, (size_t)B, st, h)) return s;
  std::vector<int32_t> live;
  for (int32_t x : h) {
    if (x < 0) continue;
    if (x >= n_slots) return KDA_ERR_INVALID_ARGUMENT;
    live.push_back(x);
  }
  std::sort(live.begin(), live.end());
  return std::adjacent_find(live.begin(), live.end()) == live.end() ? KDA_OK
                                                                    : KDA_ERR_INVALID_ARGUMENT;
}

// write_pos of the buffered decode: every cursor in [0, ring_len).
kda_status check_cursors(const int32_t* pos, int32_t B, int32_t L, hipStream_t st) {
  std::vector<int32_t> h;
  if (kda_status s = read_back(pos, (size_t)B, st, h)) return s;
  for (int32_t x : h)
    if (x < 0 || x >= L) return KDA_ERR_INVALID_ARGUMENT;
  return KDA_OK;
}

// Checks the model-layer options and converts them (NULL = the plain step).
kda_status step_opts(const kda_step_opts* in, kda_dtype io, int32_t H, kda::StepOpts& out) {
  out = kda::StepOpts{};
  if (!in) return KDA_OK;
  if (in->gate_mode < 0 || in->gate_mode > 2) return KDA_ERR_INVALID_ARGUMENT;
  if (in->gate_mode != 0 && !in->A_log) return KDA_ERR_INVALID_ARGUMENT;
  if (in->gate_mode == 2 && !(in->lower_bound < 0.f)) return KDA_ERR_INVALID_ARGUMENT;
  if (in->qk_heads < 0 || (in->qk_heads > 0 && H % in->qk_heads != 0))
    return KDA_ERR_INVALID_ARGUMENT;
  if (in->o_gate) {
    if (!in->o_norm_w || !aligned16(in->o_norm_w) || !io_aligned(io, in->o_gate))
      return KDA_ERR_INVALID_ARGUMENT;
    if (!(in->o_norm_eps >= 0.f) || in->o_gate_act < 0 || in->o_gate_act > 1)
      return KDA_ERR_INVALID_ARGUMENT;
  }
  out.gate_mode = in->gate_mode;
  out.A_log = in->A_log;
  out.dt_bias = in->dt_bias;
  out.lower_bound = in->gate_mode == 2 ? in->lower_bound : 0.f;
  out.per_head_gate = in->per_head_gate != 0;
  out.qk_l2norm = in->qk_l2norm != 0;
  out.qk_heads = in->qk_heads;
  out.o_gate = in->o_gate;
  out.o_norm_w = in->o_norm_w;
  out.o_norm_eps = in->o_norm_eps;
  out.o_gate_act = in->o_gate_act;
  return KDA_OK;
}

kda_status prefill_checked(kda_dtype io, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const int32_t* cu_seqlens,
                           int32_t N, int64_t T, int32_t H, int32_t K, int32_t V,
                           int32_t chunk, float scale, const float* h0, float* ht, void* o,
                           void* workspace, size_t workspace_bytes, void* stream,
                           void* const* marks, int gate_mode = 0,
                           const float* A_log = nullptr, const float* dt_bias = nullptr,
                           float lower_bound = 0.f, float* snaps = nullptr,
                           int snap_interval = 0, int64_t snap_rows = 0, int qk_heads = 0,
                           int per_head_gate = 0, int qk_l2norm = 0,
                           bool single_stream = false) {
  if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (N < 1 || H < 1 || T < 0) return KDA_ERR_INVALID_ARGUMENT;
  if (!head_dim_ok(K) || !head_dim_ok(V) || K != V) return KDA_ERR_UNSUPPORTED;
  if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_UNSUPPORTED;
  if ((uint64_t)T * (uint64_t)H >= (1ull << 31)) return KDA_ERR_UNSUPPORTED;
  if (!cu_seqlens) return KDA_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!io_aligned(io, q) || !io_aligned(io, k) || !io_aligned(io, v) ||
                !io_aligned(io, o) || !aligned16(g)))
    return KDA_ERR_INVALID_ARGUMENT;
  if ((h0 && !aligned16(h0)) || (ht && !aligned16(ht))) return KDA_ERR_INVALID_ARGUMENT;
  const size_t need = kda::prefill_workspace_bytes(T, N, H, K, V, chunk);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return KDA_ERR_WORKSPACE;
  if (gate_mode != 0 && T > 0 && (!A_log || (dt_bias && !aligned16(dt_bias))))
    return KDA_ERR_INVALID_ARGUMENT;
  if (debug_checks())
    if (kda_status st = check_cu(cu_seqlens, N, T, (hipStream_t)stream)) return st;
  kda::PrefillArgs p{io == KDA_BF16, q, k, v, g, beta, cu_seqlens, N, T, H, K, V,
                     chunk, scale, h0, ht, o, workspace, workspace_bytes, marks,
                     gate_mode, A_log, dt_bias, lower_bound, snaps, snap_interval,
                     snap_rows, qk_heads, per_head_gate, qk_l2norm, single_stream};
  return launch_status(kda::run_prefill(p, (hipStream_t)stream));
}

// ------------------------------------------------------ static scratch

// The prefill workspace of kda_chunk_prefill_noalloc, for callers that cannot
// allocate: one array per GPU the library runs on, held until the process
// ends.  In host code `scratch` only names the symbol; its device address on
// each GPU comes from hipGetSymbolAddress (scratch_on), and only that address
// is ever passed to a kernel.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the GPU that runs `stream` (looked up once
// per device, with that device current), or nullptr if the lookup fails.
void* scratch_on(hipStream_t stream) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  hipDevice_t dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

kda_status prefill_ex_impl(kda_dtype io, const void* q, const void* k,
                                const void* v, const float* g, const float* beta,
                                const int32_t* cu_seqlens, int32_t N, int64_t T,
                                int32_t H, int32_t K, int32_t V, int32_t chunk,
                                float scale, const float* h0, float* ht, void* o,
                                void* workspace, size_t workspace_bytes,
                                const kda_prefill_opts* opts, void* stream,
                                bool single_stream) {
  if (!opts)
    return prefill_checked(io, q, k, v, g, beta, cu_seqlens, N, T, H, K, V, chunk, scale, h0,
                           ht, o, workspace, workspace_bytes, stream, nullptr, 0, nullptr,
                           nullptr, 0.f, nullptr, 0, 0, 0, 0, 0, single_stream);
  if (opts->gate_mode < 0 || opts->gate_mode > 2) return KDA_ERR_INVALID_ARGUMENT;
  if (opts->gate_mode == 2 && !(opts->lower_bound < 0.f)) return KDA_ERR_INVALID_ARGUMENT;
  if (opts->qk_heads < 0 || (opts->qk_heads > 0 && H % opts->qk_heads != 0))
    return KDA_ERR_INVALID_ARGUMENT;
  if (opts->per_head_gate && H % 4 != 0) return KDA_ERR_UNSUPPORTED;
  int interval = 0;
  if (opts->snapshots) {
    interval = opts->snapshot_interval;
    if (interval < 1 || chunk < 1 || interval % chunk != 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned16(opts->snapshots) || T < 0 || opts->snapshot_rows < T / interval)
      return KDA_ERR_INVALID_ARGUMENT;
  }
  return prefill_checked(io, q, k, v, g, beta, cu_seqlens, N, T, H, K, V, chunk, scale, h0, ht,
                         o, workspace, workspace_bytes, stream, nullptr, opts->gate_mode,
                         opts->A_log, opts->dt_bias,
                         opts->gate_mode == 2 ? opts->lower_bound : 0.f, opts->snapshots,
                         interval, opts->snapshots ? opts->snapshot_rows : 0, opts->qk_heads,
                         opts->per_head_gate != 0,
                         opts->qk_l2norm != 0, single_stream);
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_SCRATCH_LIMIT: return "KDA_ERR_SCRATCH_LIMIT";
  }
  return "KDA_ERR_UNKNOWN";
}

kda_status kda_gate_prep(const float* a, const float* b, const float* A_log,
                         const float* dt_bias, int64_t T, int32_t H, int32_t K,
                         float lower_bound, float* g, float* beta, void* stream) {
  if (T < 0 || H < 1 || !(lower_bound <= 0.f)) return KDA_ERR_INVALID_ARGUMENT;
  if (!head_dim_ok(K)) return KDA_ERR_UNSUPPORTED;
  if ((uint64_t)T * (uint64_t)H >= (1ull << 32)) return KDA_ERR_UNSUPPORTED;
  if (T == 0) return KDA_OK;
  if (!a || !b || !A_log || !g || !beta) return KDA_ERR_INVALID_ARGUMENT;
  if (!aligned16(a) || !aligned16(g) || (dt_bias && !aligned16(dt_bias)))
    return KDA_ERR_INVALID_ARGUMENT;
  kda::GateArgs p{a, b, A_log, dt_bias, T, H, K, lower_bound, g, beta};
  return launch_status(kda::run_gate(p, (hipStream_t)stream));
}

kda_status kda_chunk_prefill_workspace_size(int64_t T, int32_t N, int32_t H,
                                            int32_t K, int32_t V, int32_t chunk,
                                            size_t* bytes) {
  if (T < 0 || N < 1 || H < 1 || !bytes) return KDA_ERR_INVALID_ARGUMENT;
  if (!head_dim_ok(K) || !head_dim_ok(V) || K != V) return KDA_ERR_UNSUPPORTED;
  if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_UNSUPPORTED;
  *bytes = kda::prefill_workspace_bytes(T, N, H, K, V, chunk);
  return KDA_OK;
}

kda_status kda_chunk_prefill_schedule(int64_t T, int32_t N, int32_t H, int32_t K, int32_t V,
                                      int32_t chunk, kda_prefill_schedule* out) {
  size_t bytes = 0;
  const kda_status st = kda_chunk_prefill_workspace_size(T, N, H, K, V, chunk, &bytes);
  if (st != KDA_OK) return st;
  if (!out) return KDA_ERR_INVALID_ARGUMENT;
  int s[6];
  kda::prefill_schedule(T, N, H, K, chunk, s);
  *out = kda_prefill_schedule{s[0], s[1], s[2], s[3], s[4], s[5]};
  return KDA_OK;
}

kda_status kda_chunk_prefill(kda_dtype io, const void* q, const void* k,
                             const void* v, const float* g, const float* beta,
                             const int32_t* cu_seqlens, int32_t N, int64_t T,
                             int32_t H, int32_t K, int32_t V, int32_t chunk,
                             float scale, const float* h0, float* ht, void* o,
                             void* workspace, size_t workspace_bytes,
                             void* stream) {
  return prefill_checked(io, q, k, v, g, beta, cu_seqlens, N, T, H, K, V, chunk, scale,
                         h0, ht, o, workspace, workspace_bytes, stream, nullptr);
}

kda_status kda_chunk_prefill_snapshots(kda_dtype io, const void* q, const void* k,
                                       const void* v, const float* g, const float* beta,
                                       const int32_t* cu_seqlens, int32_t N, int64_t T,
                                       int32_t H, int32_t K, int32_t V, int32_t chunk,
                                       float scale, const float* h0, float* ht, void* o,
                                       float* snapshots, int64_t snapshot_rows,
                                       int32_t snapshot_interval, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (snapshot_interval < 1 || chunk < 1 || snapshot_interval % chunk != 0)
    return KDA_ERR_INVALID_ARGUMENT;
  if (!snapshots || !aligned16(snapshots) || T < 0 || snapshot_rows < T / snapshot_interval)
    return KDA_ERR_INVALID_ARGUMENT;
  return prefill_checked(io, q, k, v, g, beta, cu_seqlens, N, T, H, K, V, chunk, scale, h0, ht,
                         o, workspace, workspace_bytes, stream, nullptr, 0, nullptr, nullptr,
                         0.f, snapshots, snapshot_interval, snapshot_rows);
}

kda_status kda_chunk_prefill_ex(kda_dtype io, const void* q, const void* k,
                                const void* v, const float* g, const float* beta,
                                const int32_t* cu_seqlens, int32_t N, int64_t T,
                                int32_t H, int32_t K, int32_t V, int32_t chunk,
                                float scale, const float* h0, float* ht, void* o,
                                void* workspace, size_t workspace_bytes,
                                const kda_prefill_opts* opts, void* stream) {
  return prefill_ex_impl(io, q, k, v, g, beta, cu_seqlens, N, T, H, K, V, chunk, scale, h0, ht,
                         o, workspace, workspace_bytes, opts, stream, false);
}

kda_status kda_chunk_prefill_marked(kda_dtype io, const void* q, const void* k,
                                    const void* v, const float* a, const float* b,
                                    const float* A_log, const float* dt_bias,
                                    float lower_bound, const int32_t* cu_seqlens, int32_t N,
                                    int64_t T, int32_t H, int32_t K, int32_t V, int32_t chunk,
                                    float scale, const float* h0, float* ht, void* o,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    void* const* marks) {
  if (!marks || !marks[0] || !marks[1] || !marks[2] || !marks[3])
    return KDA_ERR_INVALID_ARGUMENT;
  if (!(lower_bound <= 0.f)) return KDA_ERR_INVALID_ARGUMENT;
  return prefill_checked(io, q, k, v, a, b, cu_seqlens, N, T, H, K, V, chunk, scale, h0, ht,
                         o, workspace, workspace_bytes, stream, marks,
                         lower_bound < 0.f ? 2 : 1, A_log, dt_bias, lower_bound, nullptr, 0, 0,
                         0, 0, 0, /*single_stream=*/true);
}

kda_status kda_chunk_prefill_gated(kda_dtype io, const void* q, const void* k,
                                   const void* v, const float* a, const float* b,
                                   const float* A_log, const float* dt_bias,
                                   float lower_bound, const int32_t* cu_seqlens, int32_t N,
                                   int64_t T, int32_t H, int32_t K, int32_t V, int32_t chunk,
                                   float scale, const float* h0, float* ht, void* o,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!(lower_bound <= 0.f)) return KDA_ERR_INVALID_ARGUMENT;
  return prefill_checked(io, q, k, v, a, b, cu_seqlens, N, T, H, K, V, chunk, scale, h0, ht,
                         o, workspace, workspace_bytes, stream, nullptr,
                         lower_bound < 0.f ? 2 : 1, A_log, dt_bias, lower_bound);
}

kda_status kda_recurrent_decode(kda_dtype io, const void* q, const void* k,
                                const void* v, const float* g,
                                const float* beta, float scale,
                                float* state_pool, int64_t n_slots,
                                const int32_t* slot_idx, int32_t B, int32_t H,
                                int32_t K, int32_t V, void* o, void* stream) {
  return kda_recurrent_decode_ex(io, q, k, v, g, beta, scale, state_pool, n_slots, slot_idx, B,
                                 H, K, V, o, nullptr, stream);
}

kda_status kda_recurrent_decode_ex(kda_dtype io, const void* q, const void* k,
                                   const void* v, const float* g,
                                   const float* beta, float scale,
                                   float* state_pool, int64_t n_slots,
                                   const int32_t* slot_idx, int32_t B, int32_t H,
                                   int32_t K, int32_t V, void* o,
                                   const kda_step_opts* opts, void* stream) {
  if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || n_slots < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (!head_dim_ok(K) || !head_dim_ok(V)) return KDA_ERR_UNSUPPORTED;
  if ((uint64_t)B * (uint64_t)H >= (1ull << 31)) return KDA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !beta || !state_pool || !slot_idx || !o)
    return KDA_ERR_INVALID_ARGUMENT;
  if (!io_aligned(io, v) || !io_aligned(io, o) || !aligned16(state_pool))
    return KDA_ERR_INVALID_ARGUMENT;
  kda::StepOpts op;
  if (kda_status st = step_opts(opts, io, H, op)) return st;
  if (debug_checks())
    if (kda_status st = check_slots(slot_idx, B, n_slots, (hipStream_t)stream)) return st;
  kda::DecodeArgs p{io == KDA_BF16, q, k, v, g, beta, scale, state_pool, slot_idx,
                    B, 1, H, K, V, nullptr, o, op, n_slots};
  return launch_status(kda::run_decode(p, (hipStream_t)stream));
}

kda_status kda_verify(kda_dtype io, const void* q, const void* k,
                      const void* v, const float* g, const float* beta,
                      float scale, const float* state_pool, int64_t n_slots,
                      const int32_t* slot_idx, int32_t B, int32_t Tv,
                      int32_t H, int32_t K, int32_t V, float* inter_states,
                      void* o, void* stream) {
  return kda_verify_ex(io, q, k, v, g, beta, scale, state_pool, n_slots, slot_idx, B, Tv, H, K,
                       V, inter_states, o, nullptr, stream);
}

kda_status kda_verify_ex(kda_dtype io, const void* q, const void* k,
                         const void* v, const float* g, const float* beta,
                         float scale, const float* state_pool, int64_t n_slots,
                         const int32_t* slot_idx, int32_t B, int32_t Tv,
                         int32_t H, int32_t K, int32_t V, float* inter_states,
                         void* o, const kda_step_opts* opts, void* stream) {
  if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (B < 1 || Tv < 1 || H < 1 || n_slots < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (!head_dim_ok(K) || !head_dim_ok(V)) return KDA_ERR_UNSUPPORTED;
  if ((uint64_t)B * (uint64_t)H >= (1ull << 31)) return KDA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !beta || !state_pool || !slot_idx || !inter_states || !o)
    return KDA_ERR_INVALID_ARGUMENT;
  if (!io_aligned(io, v) || !io_aligned(io, o) || !aligned16(state_pool) ||
      !aligned16(inter_states))
    return KDA_ERR_INVALID_ARGUMENT;
  kda::StepOpts op;
  if (kda_status st = step_opts(opts, io, H, op)) return st;
  if (debug_checks())
    if (kda_status st = check_slots(slot_idx, B, n_slots, (hipStream_t)stream)) return st;
  kda::DecodeArgs p{io == KDA_BF16, q, k, v, g, beta, scale,
                    const_cast<float*>(state_pool), slot_idx, B, Tv, H, K, V,
                    inter_states, o, op, n_slots};
  return launch_status(kda::run_verify(p, (hipStream_t)stream));
}

kda_status kda_replay_decode(kda_dtype io, const void* q, const void* k,
                             const void* v, const float* g, const float* beta,
                             float scale, float* state_pool, int64_t n_slots,
                             const int32_t* slot_idx, const int32_t* write_pos,
                             const int32_t* force_flush, int32_t ring_len, float* ring_d,
                             void* ring_k, float* ring_g, int32_t B, int32_t H,
                             int32_t K, int32_t V, void* o, int32_t* next_write_pos,
                             void* stream) {
  return kda_replay_decode_ex(io, q, k, v, g, beta, scale, state_pool, n_slots, slot_idx,
                              write_pos, force_flush, ring_len, ring_d, ring_k, ring_g, B, H, K,
                              V, o, next_write_pos, nullptr, stream);
}

kda_status kda_replay_decode_ex(kda_dtype io, const void* q, const void* k,
                                const void* v, const float* g, const float* beta,
                                float scale, float* state_pool, int64_t n_slots,
                                const int32_t* slot_idx, const int32_t* write_pos,
                                const int32_t* force_flush, int32_t ring_len, float* ring_d,
                                void* ring_k, float* ring_g, int32_t B, int32_t H,
                                int32_t K, int32_t V, void* o, int32_t* next_write_pos,
                                const kda_step_opts* opts, void* stream) {
  if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || n_slots < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (ring_len < 1 || ring_len > KDA_RING_MAX) return KDA_ERR_INVALID_ARGUMENT;
  if (!head_dim_ok(K) || !head_dim_ok(V)) return KDA_ERR_UNSUPPORTED;
  if ((uint64_t)B * (uint64_t)H >= (1ull << 31)) return KDA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !beta || !state_pool || !slot_idx || !write_pos || !ring_d ||
      !ring_k || !ring_g || !o)
    return KDA_ERR_INVALID_ARGUMENT;
  if (!io_aligned(io, v) || !io_aligned(io, o) || !aligned16(state_pool) || !aligned16(ring_d))
    return KDA_ERR_INVALID_ARGUMENT;
  if (next_write_pos) {
    // the cursor output is written while other workgroups still read the
    // cursors and flush flags: it must not overlap them
    const uintptr_t n0 = (uintptr_t)next_write_pos, n1 = n0 + (uintptr_t)B * 4;
    const uintptr_t w0 = (uintptr_t)write_pos, w1 = w0 + (uintptr_t)B * 4;
    if (n0 < w1 && w0 < n1) return KDA_ERR_INVALID_ARGUMENT;
    if (force_flush) {
      const uintptr_t f0 = (uintptr_t)force_flush, f1 = f0 + (uintptr_t)B * 4;
      if (n0 < f1 && f0 < n1) return KDA_ERR_INVALID_ARGUMENT;
    }
  }
  kda::StepOpts op;
  if (kda_status st = step_opts(opts, io, H, op)) return st;
  if (debug_checks()) {
    if (kda_status st = check_slots(slot_idx, B, n_slots, (hipStream_t)stream)) return st;
    if (kda_status st = check_cursors(write_pos, B, ring_len, (hipStream_t)stream)) return st;
  }
  kda::ReplayArgs p{io == KDA_BF16, q, k, v, g, beta, scale, state_pool, slot_idx,
                    write_pos, force_flush, ring_len, ring_d, ring_k, ring_g, B, H, K, V, o,
                    next_write_pos, op, n_slots};
  return launch_status(kda::run_replay(p, (hipStream_t)stream));
}

kda_status kda_chunk_prefill_noalloc(kda_dtype io, const void* q, const void* k,
                                     const void* v, const float* g, const float* beta,
                                     const int32_t* cu_seqlens, int32_t N, int64_t T,
                                     int32_t H, int32_t K, int32_t V, int32_t chunk,
                                     float scale, const float* h0, float* ht, void* o,
                                     const kda_prefill_opts* opts, void* stream) {
  size_t need = 0;
  if (kda_status st = kda_chunk_prefill_workspace_size(T, N, H, K, V, chunk, &need)) return st;
  if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH_LIMIT;
  void* ws = scratch_on((hipStream_t)stream);
  if (ws == nullptr) return KDA_ERR_LAUNCH;
  return prefill_ex_impl(io, q, k, v, g, beta, cu_seqlens, N, T, H, K, V, chunk, scale, h0, ht,
                         o, ws, (size_t)KDA_NOALLOC_SCRATCH_BYTES, opts, stream,
                         /*single_stream=*/true);
}

}  // extern "C"
