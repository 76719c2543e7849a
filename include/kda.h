/*
 * kda.h -- C ABI of libkda: Kimi Delta Attention (KDA) gated delta rule on
 * AMD Instinct MI355X (gfx950), hand-written HIP kernels.
 *
 * The method (sources cited by page title and section):
 *   "Linear attention" tutorial (zdszero.github.io), section "KDA：逐通道的遗忘门":
 *     S_t = (I - beta_t k_t^T k_t) Diag(exp g_t) S_{t-1} + beta_t k_t^T v_t,
 *     row vectors q_t, k_t in R^{1 x K}, v_t in R^{1 x V}, state S in R^{K x V};
 *     g_t in R^K is a per-key-channel log decay (g <= 0).
 *   same page, section "实例：Kimi K3": o_t = scale * q_t S_t (scale = K^-1/2
 *     in the model; here an explicit argument).
 *   same page, sections "Gated DeltaNet" / "KDA": the gate
 *     g = -exp(A_log[h]) * softplus(a + dt_bias[h, c]), beta = sigmoid(b);
 *     the safe gate g = lower_bound * sigmoid(exp(A_log[h]) (a + dt_bias)).
 *   same page, section "两种计算形态": chunkwise prefill (WY/UT form, one
 *     64x64 triangular solve per chunk, state carried between chunks) and
 *     recurrent single-token decode that rewrites the pool state in place.
 *   "PR #26888 report" ([KDA] target_verify): multi-token verify that records
 *     the state after every draft token and never updates the pool.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, to a
 *     row-major contiguous array, 16-byte aligned.  The library allocates no
 *     memory for the caller's data, never synchronises the stream, and may
 *     be called from several host threads at once.  Its only global state is
 *     per device: one library-owned second stream with a pool of events
 *     (created on first use, kept until the process ends; see below), and
 *     the static scratch array of kda_chunk_prefill_noalloc.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is ordered on it; a return of KDA_OK means "enqueued".  One
 *     exception to "all work runs on it": a prefill whose state chain is cut
 *     into waves (long sequences, few of them; kda_chunk_prefill_schedule in
 *     kda_profile.h tells) runs the intra-chunk kernel of each wave on the
 *     library's second stream of the current device (non-blocking, default
 *     priority), so that it overlaps the state pass of the previous wave.
 *     That stream first waits for the work already on `stream`, and the
 *     call's last kernel on `stream` waits for all it ran, so work enqueued
 *     on `stream` afterwards sees the finished results, exactly as with one
 *     stream.  The call keeps to `stream` alone when `stream` belongs to
 *     another device than the current one, when it is being captured into a
 *     graph, and in kda_chunk_prefill_noalloc.
 *   - States and gates are always fp32.  q, k, v and o share the io dtype.
 *   - State layout is [.., H, K, V] with V contiguous: row i of a head's
 *     state belongs to key channel i.
 *   - q and k are expected to be L2-normalised per (token, head) by the
 *     caller; the library does not renormalise.
 *   - Errors are returned, never thrown.  Host-side validation covers null
 *     pointers, alignment, sizes and supported shapes; on any error nothing
 *     is enqueued.  Values that live in device memory (cu_seqlens, slot
 *     indices, ring cursors) are the caller's contract and are not read by
 *     the host.  The kernels still keep every access in bounds whatever
 *     those arrays hold.  Sequence ranges are made disjoint: with c'_m =
 *     cu_seqlens[m] clamped into [0, T], sequence n covers tokens
 *     max(c'_0 .. c'_n) .. max(c'_0 .. c'_{n+1}) - 1 (for a valid array,
 *     exactly cu[n] .. cu[n+1]-1).  A live slot index at or past n_slots (or
 *     a ring cursor outside the ring) gives o = NaN for that row and touches
 *     no state.
 *   - Debug checks: when the environment variable KDA_CHECK is "1" (read at
 *     every call), each call copies those device arrays to the host (waiting
 *     for the stream) and returns KDA_ERR_INVALID_ARGUMENT, with nothing
 *     enqueued, unless cu_seqlens starts at 0, ends at T and never
 *     decreases; every live slot is below n_slots and appears once; and every
 *     ring cursor lies in [0, ring_len).
 *   - Supported head sizes: K, V in {16, 32, 64, 128}.  The prefill entry
 *     points also require K == V (the head layout of the pages' models,
 *     where the q/k head size equals the value head size); they return
 *     KDA_ERR_UNSUPPORTED otherwise.  Decode, verify and the buffered decode
 *     take any K, V of the set.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1, /* null pointer, misalignment, bad size   */
  KDA_ERR_UNSUPPORTED = 2,      /* shape or dtype outside the built set   */
  KDA_ERR_LAUNCH = 3,           /* the HIP runtime refused a launch       */
  KDA_ERR_WORKSPACE = 4,        /* workspace missing or too small         */
  KDA_ERR_SCRATCH_LIMIT = 5     /* the call needs more scratch than the
                                   library's static scratch array holds   */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype; /* dtype of q, k, v, o */

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_status_string(kda_status s);

/*
 * Gate activation (tutorial, sections "Gated DeltaNet" and "KDA").
 *   a       [T, H, K] fp32  raw per-channel gate input
 *   b       [T, H]    fp32  raw write-strength input
 *   A_log   [H]       fp32  per-head log decay rate
 *   dt_bias [H, K]    fp32  per-channel bias, or NULL for zero
 *   lower_bound: 0.f selects g = -exp(A_log) softplus(a + dt_bias) with
 *     softplus(x) = x for x > 20 (threshold of the ReplaySSM and target-verify
 *     kernels); a negative value selects the safe gate
 *     g = lower_bound * sigmoid(exp(A_log) (a + dt_bias)).
 *   g       [T, H, K] fp32  output log decay (<= 0)
 *   beta    [T, H]    fp32  output sigmoid(b)
 * T may be 0 (nothing is enqueued).  K in {16, 32, 64, 128}.
 */
kda_status kda_gate_prep(const float* a, const float* b, const float* A_log,
                         const float* dt_bias, int64_t T, int32_t H, int32_t K,
                         float lower_bound, float* g, float* beta,
                         void* stream);

/*
 * Bytes of device workspace kda_chunk_prefill needs for a packed batch of
 * T tokens in N sequences (an upper bound that holds for every split of T
 * into N lengths), written to *bytes.  Returns KDA_ERR_INVALID_ARGUMENT for
 * T < 0, N < 1, H < 1 or a NULL `bytes`, and KDA_ERR_UNSUPPORTED for a shape
 * the prefill does not build (K, V outside {16, 32, 64, 128}, K != V, chunk
 * outside {16, 32, 64}); *bytes is then left untouched.
 */
kda_status kda_chunk_prefill_workspace_size(int64_t T, int32_t N, int32_t H,
                                            int32_t K, int32_t V, int32_t chunk,
                                            size_t* bytes);

/*
 * Chunkwise varlen prefill (tutorial, section "两种计算形态"; the WY/UT form
 * of the unrolled delta rule, section "矩阵（并行）形式").
 *   q, k    [T, H, K] io dtype;  v [T, H, V] io dtype; K == V
 *     (KDA_ERR_UNSUPPORTED otherwise)
 *   g       [T, H, K] fp32 activated log decay;  beta [T, H] fp32
 *   cu_seqlens [N + 1] int32 (device): sequence n owns tokens
 *     cu[n] .. cu[n+1]-1; must satisfy cu[0] = 0 <= cu[1] <= ... <= cu[N] = T.
 *     Zero-length sequences are allowed (ht[n] = h0[n], or zeros).
 *   chunk   16, 32 or 64: chunks never cross a sequence boundary; the last
 *     chunk of a sequence may be short.  The result does not depend on it
 *     beyond rounding.
 *   scale   read-out factor (o_t = scale * q_t S_t)
 *   h0      [N, H, K, V] fp32 initial states, or NULL for zeros
 *   ht      [N, H, K, V] fp32 final states, or NULL to skip; may alias h0
 *   o       [T, H, V] io dtype output (fp32 accumulate, round to nearest even)
 *   workspace / workspace_bytes: caller-owned device scratch of at least
 *     kda_chunk_prefill_workspace_size(T, N, H, K, V, chunk) bytes, 256-byte
 *     aligned; its contents on entry are irrelevant.  It must not be reused
 *     by another call until this call's work on `stream` has finished.
 * T may be 0 (only ht = h0 is written).
 */
kda_status kda_chunk_prefill(kda_dtype io, const void* q, const void* k,
                             const void* v, const float* g, const float* beta,
                             const int32_t* cu_seqlens, int32_t N, int64_t T,
                             int32_t H, int32_t K, int32_t V, int32_t chunk,
                             float scale, const float* h0, float* ht, void* o,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Chunkwise varlen prefill with the gate applied inside (tutorial, sections
 * "Gated DeltaNet" and "KDA" for the gate, "两种计算形态" for the chunk form).
 * Same as kda_gate_prep followed by kda_chunk_prefill, without g and beta
 * ever being written to memory; the gate is evaluated by the same device
 * code as kda_gate_prep, so the results are those of the two-call sequence.
 *   a [T, H, K] fp32, b [T, H] fp32: raw gate inputs
 *   A_log [H] fp32, dt_bias [H, K] fp32 or NULL, lower_bound: as in
 *     kda_gate_prep (0 = softplus gate, < 0 = safe gate)
 * Every other argument, the workspace and the errors are those of
 * kda_chunk_prefill; additionally A_log must not be NULL when T > 0.
 */
kda_status kda_chunk_prefill_gated(kda_dtype io, const void* q, const void* k,
                                   const void* v, const float* a, const float* b,
                                   const float* A_log, const float* dt_bias,
                                   float lower_bound, const int32_t* cu_seqlens,
                                   int32_t N, int64_t T, int32_t H, int32_t K,
                                   int32_t V, int32_t chunk, float scale,
                                   const float* h0, float* ht, void* o,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * kda_chunk_prefill that also records chunk-boundary states, for prefix
 * caching and verify rollback (tutorial, section "两种计算形态": the chunk
 * form materialises the state at every chunk boundary; section "prefix cache
 * 与投机解码": those states are kept as prefix snapshots, at a tracking
 * interval).
 *   snapshot_interval: a positive multiple of chunk.  Sequence n contributes
 *     floor(len_n / snapshot_interval) rows: the state after its first
 *     snapshot_interval, 2 snapshot_interval, ... tokens.
 *   snapshots [snapshot_rows, H, K, V] fp32: rows of sequence n start after
 *     those of sequences 0 .. n-1 (row sum_{m<n} floor(len_m / interval) + j
 *     holds the state after (j + 1) interval tokens of sequence n); rows past
 *     the total are left untouched.  snapshot_rows must be at least
 *     T / snapshot_interval (a bound on the total for any split of T).
 * Every other argument, o, ht and the errors are those of kda_chunk_prefill
 * (the same kernels: o and ht are bit-identical to it), and each snapshot is
 * bit-identical to the ht of kda_chunk_prefill run on that prefix alone.
 */
kda_status kda_chunk_prefill_snapshots(kda_dtype io, const void* q, const void* k,
                                       const void* v, const float* g, const float* beta,
                                       const int32_t* cu_seqlens, int32_t N, int64_t T,
                                       int32_t H, int32_t K, int32_t V, int32_t chunk,
                                       float scale, const float* h0, float* ht, void* o,
                                       float* snapshots, int64_t snapshot_rows,
                                       int32_t snapshot_interval, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Model-layer options of kda_chunk_prefill_ex; NULL or all zero is
 * kda_chunk_prefill.
 *   gate_mode, A_log, dt_bias, lower_bound: as in kda_step_opts (the gate
 *     applied in the kernel from raw a and b, as kda_chunk_prefill_gated).
 *   per_head_gate: g (or a) is [T, H] and dt_bias [H]: one log decay per
 *     (token, head) shared by every key channel (the Gated DeltaNet gate,
 *     tutorial section "Gated DeltaNet"); H must be a multiple of 4.
 *   qk_heads: heads of q and k (0 = H; H a multiple): value head h reads q
 *     and k of head h / (H / qk_heads).
 *   snapshots, snapshot_rows, snapshot_interval: chunk-boundary states as in
 *     kda_chunk_prefill_snapshots (snapshots NULL = none).
 *   qk_l2norm: q and k are L2-normalised in the kernel, x / sqrt(|x|^2 +
 *     1e-6) per (token, q/k head) (ReplaySSM analysis, section 3.10), as
 *     kda_step_opts.qk_l2norm does for decode and verify.  The factor
 *     1 / sqrt(|x|^2 + 1e-6) of each row scales the products that row enters;
 *     q and k themselves are never rounded again.
 */
typedef struct {
  int32_t gate_mode;
  const float* A_log;
  const float* dt_bias;
  float lower_bound;
  int32_t per_head_gate;
  int32_t qk_heads;
  float* snapshots;
  int64_t snapshot_rows;
  int32_t snapshot_interval;
  int32_t qk_l2norm;
} kda_prefill_opts;

/*
 * kda_chunk_prefill with model-layer options: q, k are [T, qk_heads, K]; g
 * is [T, H, K] (or [T, H] with per_head_gate), raw a when gate_mode != 0
 * (then beta holds the raw b).  Workspace, outputs and errors as in
 * kda_chunk_prefill; with opts NULL the results are bit-identical to it.
 */
kda_status kda_chunk_prefill_ex(kda_dtype io, const void* q, const void* k,
                                const void* v, const float* g, const float* beta,
                                const int32_t* cu_seqlens, int32_t N, int64_t T,
                                int32_t H, int32_t K, int32_t V, int32_t chunk,
                                float scale, const float* h0, float* ht, void* o,
                                void* workspace, size_t workspace_bytes,
                                const kda_prefill_opts* opts, void* stream);

/* Bytes of the static scratch array behind kda_chunk_prefill_noalloc. */
#define KDA_NOALLOC_SCRATCH_BYTES (256u << 20)

/*
 * kda_chunk_prefill_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a static device array
 * of KDA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends; this call allocates nothing.  Every other argument, the
 * results (bit-identical to kda_chunk_prefill_ex with any workspace) and the
 * errors are those of kda_chunk_prefill_ex, plus:
 *   KDA_ERR_SCRATCH_LIMIT when kda_chunk_prefill_workspace_size(T, N, H, K,
 *     V, chunk) exceeds KDA_NOALLOC_SCRATCH_BYTES (nothing is enqueued).  At
 *     H = 32, K = V = 128, chunk 64 that allows about 3500 tokens in one
 *     sequence; fewer heads or shorter sequences fit more.
 *   KDA_ERR_LAUNCH when the array's device address cannot be looked up.
 * All calls on one GPU share its array: two calls whose work overlaps on
 * that GPU (on different streams, or from different host threads without
 * ordering) race on it.  Calls ordered on one stream are safe.
 */
kda_status kda_chunk_prefill_noalloc(kda_dtype io, const void* q, const void* k,
                                     const void* v, const float* g, const float* beta,
                                     const int32_t* cu_seqlens, int32_t N, int64_t T,
                                     int32_t H, int32_t K, int32_t V, int32_t chunk,
                                     float scale, const float* h0, float* ht, void* o,
                                     const kda_prefill_opts* opts, void* stream);

/*
 * Single-token decode on a slot-indexed state pool, updated in place
 * (tutorial, section "两种计算形态": the recurrent kernel rewrites the pool
 * state; ReplaySSM analysis, section 3.6: a negative slot marks a padding row).
 *   q, k [B, H, K], v [B, H, V] io dtype; g [B, H, K] fp32; beta [B, H] fp32
 *   state_pool [n_slots, H, K, V] fp32, read and written in place
 *   slot_idx [B] int32 (device): slot of each request; a negative value
 *     marks a padding row, whose o is zero and whose state is not touched.
 *     Live slots must be < n_slots and distinct within one call (two rows on
 *     one slot race).
 *   o [B, H, V] io dtype
 * Per (request, head): S' = Diag(exp g) S; v_hat = k S'; d = beta (v - v_hat);
 * S = S' + k^T d (written back); o = scale q S.
 */
kda_status kda_recurrent_decode(kda_dtype io, const void* q, const void* k,
                                const void* v, const float* g,
                                const float* beta, float scale,
                                float* state_pool, int64_t n_slots,
                                const int32_t* slot_idx, int32_t B, int32_t H,
                                int32_t K, int32_t V, void* o, void* stream);

/*
 * Multi-token verify without state update ("PR #26888 report": target_verify
 * with disable_state_update and an intermediate-state buffer).
 *   q, k [B, Tv, H, K], v [B, Tv, H, V] io dtype; g [B, Tv, H, K] fp32;
 *   beta [B, Tv, H] fp32; state_pool [n_slots, H, K, V] fp32, READ ONLY;
 *   slot_idx [B] int32 (device), negative = padding row (o = 0, inter rows
 *   left unwritten);
 *   inter_states [B, Tv, H, K, V] fp32: state after draft token s;
 *   o [B, Tv, H, V] io dtype.
 * Row r, step s equals the (s+1)-th of s+1 sequential decode calls started
 * from pool[slot_idx[r]].
 */
kda_status kda_verify(kda_dtype io, const void* q, const void* k,
                      const void* v, const float* g, const float* beta,
                      float scale, const float* state_pool, int64_t n_slots,
                      const int32_t* slot_idx, int32_t B, int32_t Tv,
                      int32_t H, int32_t K, int32_t V, float* inter_states,
                      void* o, void* stream);

/*
 * Model-layer options of kda_recurrent_decode_ex and kda_verify_ex; a NULL
 * options pointer, or all fields zero, is the plain step.
 *   gate_mode: 0 = g and beta are the activated log decay and strength;
 *     1 = softplus gate, 2 = safe gate: g and beta hold the raw a and b and
 *     the gate is applied in the kernel with kda_gate_prep's arithmetic
 *     (tutorial, sections "Gated DeltaNet" and "KDA"; the values are those
 *     kda_gate_prep would write).  A_log [H] is then required; dt_bias
 *     (per_head_gate ? [H] : [H, K]) may be NULL; lower_bound (< 0) is the
 *     safe gate's bound.
 *   per_head_gate: g (or a) is [.., H], one log decay per head that every
 *     key channel shares: the Gated DeltaNet gate (tutorial, "Gated
 *     DeltaNet"), run through the same kernels.
 *   qk_l2norm: q and k are L2-normalised in the kernel, x / sqrt(|x|^2 +
 *     1e-6) (ReplaySSM analysis, section 3.10).
 *   qk_heads: heads of q and k (0 = H); H must be a multiple.  Value head h
 *     reads q and k of head h / (H / qk_heads) (grouped value heads).
 *   o_gate: NULL, or [.., H, V] io dtype: o is replaced by the gated RMSNorm
 *     of the layer's output norm (tutorial, "一层 GDN / KDA 的完整数据流"):
 *     o / sqrt(mean_v o^2 + o_norm_eps) * o_norm_w[v] * act(o_gate), with
 *     act = sigmoid (o_gate_act 0, the KDA form) or silu (1, the GDN form);
 *     o_norm_w [V] fp32 is then required.
 */
typedef struct {
  int32_t gate_mode;
  const float* A_log;
  const float* dt_bias;
  float lower_bound;
  int32_t per_head_gate;
  int32_t qk_l2norm;
  int32_t qk_heads;
  const void* o_gate;
  const float* o_norm_w;
  float o_norm_eps;
  int32_t o_gate_act;
} kda_step_opts;

/*
 * kda_recurrent_decode with model-layer options.  q, k are [B, qk_heads, K];
 * g is [B, H, K] (or [B, H] with per_head_gate); every other argument is as
 * in kda_recurrent_decode.  With opts NULL the results are bit-identical to
 * kda_recurrent_decode.
 */
kda_status kda_recurrent_decode_ex(kda_dtype io, const void* q, const void* k,
                                   const void* v, const float* g,
                                   const float* beta, float scale,
                                   float* state_pool, int64_t n_slots,
                                   const int32_t* slot_idx, int32_t B, int32_t H,
                                   int32_t K, int32_t V, void* o,
                                   const kda_step_opts* opts, void* stream);

/*
 * kda_verify with model-layer options.  q, k are [B, Tv, qk_heads, K]; g is
 * [B, Tv, H, K] (or [B, Tv, H]); o_gate, when given, is [B, Tv, H, V].
 * inter_states hold the states (the output norm does not touch them).
 */
kda_status kda_verify_ex(kda_dtype io, const void* q, const void* k,
                         const void* v, const float* g, const float* beta,
                         float scale, const float* state_pool, int64_t n_slots,
                         const int32_t* slot_idx, int32_t B, int32_t Tv,
                         int32_t H, int32_t K, int32_t V, float* inter_states,
                         void* o, const kda_step_opts* opts, void* stream);

/* Longest ring kda_replay_decode accepts. */
#define KDA_RING_MAX 32

/*
 * Buffered single-token decode ("ReplaySSM" analysis, sections 2 and 3): the
 * pool holds per-slot checkpoints that are read every step and written only
 * every ring_len steps; in between, each (slot, head) appends the step's
 * (d, k, g) to a small ring, and the state the step needs is replayed from
 * the checkpoint and the ring without being formed.  Halves the state
 * traffic of kda_recurrent_decode for long rings.
 *   q, k [B, H, K], v [B, H, V] io dtype; g [B, H, K] fp32; beta [B, H] fp32;
 *   state_pool [n_slots, H, K, V] fp32: the checkpoint of each slot;
 *   slot_idx [B] int32 (device): as in kda_recurrent_decode (negative =
 *     padding row: o = 0, pool and ring untouched);
 *   write_pos [B] int32 (device): ring cursor of each row = steps decoded on
 *     the slot since its checkpoint, 0 .. ring_len-1.  A live row with a
 *     cursor outside that range gets o = NaN and touches nothing else.
 *   force_flush [B] int32 (device) or NULL: nonzero writes the checkpoint at
 *     this step whatever the cursor;
 *   ring_len L in 1 .. KDA_RING_MAX; the rings, indexed [slot, head, entry]:
 *     ring_d [n_slots, H, L, V] fp32, ring_k [n_slots, H, L, K] io dtype,
 *     ring_g [n_slots, H, L, K] fp32.  Entries 0 .. write_pos-1 of a live
 *     row's slot must hold the steps since its checkpoint (as this function
 *     left them); their contents are otherwise irrelevant.
 *   o [B, H, V] io dtype;
 *   next_write_pos [B] int32 (device) or NULL: receives 0 for rows that wrote
 *     their checkpoint, write_pos + 1 for the others, and write_pos for
 *     padding rows; it must not overlap write_pos or force_flush.
 * A row writes its checkpoint (S' + k^T d, the state after this step) when
 * write_pos = L-1 or force_flush is set, and otherwise appends
 * (d, k, g) at entry write_pos.  Every row's o equals that of
 * kda_recurrent_decode on the state the slot would hold after the same
 * steps; with L = 1 (or write_pos = 0 and a forced flush) the results are
 * bit-identical to kda_recurrent_decode.  Live slots must be distinct
 * within one call.
 */
kda_status kda_replay_decode(kda_dtype io, const void* q, const void* k,
                             const void* v, const float* g, const float* beta,
                             float scale, float* state_pool, int64_t n_slots,
                             const int32_t* slot_idx, const int32_t* write_pos,
                             const int32_t* force_flush, int32_t ring_len,
                             float* ring_d, void* ring_k, float* ring_g,
                             int32_t B, int32_t H, int32_t K, int32_t V, void* o,
                             int32_t* next_write_pos, void* stream);

/*
 * kda_replay_decode with model-layer options (kda_step_opts): the gate from
 * raw inputs, the per-head gate, grouped q/k heads (q, k [B, qk_heads, K];
 * g [B, H, K] or [B, H]), the in-kernel q/k L2 norm and the gated RMSNorm of
 * o (o_gate [B, H, V]).  The ring keeps the activated per-channel g and k
 * as given (with qk_l2norm each entry's k row is normalised again when it is
 * replayed).  With opts NULL the results are bit-identical to
 * kda_replay_decode.
 */
kda_status kda_replay_decode_ex(kda_dtype io, const void* q, const void* k,
                                const void* v, const float* g, const float* beta,
                                float scale, float* state_pool, int64_t n_slots,
                                const int32_t* slot_idx, const int32_t* write_pos,
                                const int32_t* force_flush, int32_t ring_len,
                                float* ring_d, void* ring_k, float* ring_g,
                                int32_t B, int32_t H, int32_t K, int32_t V, void* o,
                                int32_t* next_write_pos, const kda_step_opts* opts,
                                void* stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* KDA_H_ */
