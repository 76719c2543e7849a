// Internal launcher interface between the C ABI (kda_api.hip) and the kernel
// translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct GateArgs {
  const float *a, *b, *A_log, *dt_bias;
  int64_t T;
  int H, K;
  float lower_bound;
  float *g, *beta;
};

// Model-layer options of decode and verify (kda_step_opts); all zero is the
// plain step.
struct StepOpts {
  int gate_mode;  // 0: g, beta activated; 1: softplus gate, 2: safe gate (raw a, b given)
  const float *A_log, *dt_bias;
  float lower_bound;
  int per_head_gate;  // g (or a) and dt_bias per head: every key channel decays alike
  int qk_l2norm;      // q, k L2-normalised in the kernel
  int qk_heads;       // heads of q and k (0: H)
  const void* o_gate;      // io dtype [.., H, V]: gated RMSNorm of o when not null
  const float* o_norm_w;   // [V]
  float o_norm_eps;
  int o_gate_act;          // 0: sigmoid, 1: silu
};

struct DecodeArgs {
  bool bf16_io;
  const void *q, *k, *v;
  const float *g, *beta;
  float scale;
  float* pool;  // decode: in place; verify: read only
  const int32_t* slot_idx;
  int B, Tv, H, K, V;
  float* inter;  // verify only
  void* o;
  StepOpts opts;
  int64_t n_slots;  // live slots must be below it (checked in the kernels)
};

struct ReplayArgs {
  bool bf16_io;
  const void *q, *k, *v;
  const float *g, *beta;
  float scale;
  float* pool;  // checkpoints: read, and written by flushing rows
  const int32_t *slot_idx, *write_pos, *force_flush;
  int L;  // ring length
  float* ring_d;
  void* ring_k;  // io dtype
  float* ring_g;
  int B, H, K, V;
  void* o;
  int32_t* next_pos;
  StepOpts opts;  // gate options and grouped heads (no L2 norm, no output norm)
  int64_t n_slots;
};

struct PrefillArgs {
  bool bf16_io;
  const void *q, *k, *v;
  const float *g, *beta;
  const int32_t* cu_seqlens;
  int N;
  int64_t T;
  int H, K, V, C;
  float scale;
  const float* h0;
  float* ht;
  void* o;
  void* ws;
  size_t ws_bytes;
  // Optional timing marks (hipEvent_t): recorded before the plan, intra and
  // state kernels and after the state kernel; nullptr for none.
  void* const* marks;
  // 0: g and beta are activated gates.  1: softplus gate, 2: safe gate; then
  // g and beta point to the raw a [T, H, K] and b [T, H].
  int gate_mode;
  const float *A_log, *dt_bias;
  float lower_bound;
  // Optional chunk-boundary states: [rows, H, K, V] fp32, the state of each
  // sequence after every snap_interval tokens (nullptr for none).
  float* snaps;
  int snap_interval;
  int64_t snap_rows;  // rows of snaps; rows at or past it are never written
  int qk_heads;       // heads of q and k (0: H)
  int per_head_gate;  // g (or a) is [T, H] and dt_bias [H]
  int qk_l2norm;      // q, k L2-normalised in the kernel
  // Every kernel on `stream` (no second stream, nothing created): the same
  // kernels and results, without the overlap of the intra-chunk work of one
  // wave of a long chain with the state pass of the previous.
  bool single_stream;
};

hipError_t run_gate(const GateArgs& a, hipStream_t stream);
hipError_t run_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t run_verify(const DecodeArgs& a, hipStream_t stream);
hipError_t run_replay(const ReplayArgs& a, hipStream_t stream);
hipError_t run_prefill(const PrefillArgs& a, hipStream_t stream);
size_t prefill_workspace_bytes(int64_t T, int N, int H, int K, int V, int C);
// Schedule of a prefill call: {n_waves, segment chunks, maps, intra launches,
// state launches, other launches}.
void prefill_schedule(int64_t T, int N, int H, int K, int C, int out[6]);

}  // namespace kda
