/*
 * kda_oracle.c -- plain, slow, sequential fp64 reference of the Kimi Delta
 * Attention (KDA) gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the HIP path in kda_gated_delta_amd/.
 *
 * Everything is computed token by token in double precision, exactly as the
 * recurrence is written on the pages; there is no chunking, blocking or
 * re-association.  Sources (page title, section):
 *
 *  [LA]  "Linear attention" tutorial (zdszero.github.io/linear_attention.html)
 *        - section "Gated DeltaNet": the five-step token update
 *          decay -> read v_hat = k S' -> delta = beta (v - v_hat)
 *          -> S = S' + k^T delta -> o = q S, and the Mamba2-style gate
 *          g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b);
 *        - section "KDA: per-channel forget gate": the decay becomes a vector
 *          over the key channels, row i of S (key channel i) decays by
 *          exp(g[i]); the safe gate g = lb * sigmoid(exp(A_log) (f + dt_bias));
 *        - section "Kimi K3 weights": o_t = d^{-1/2} q_t S_t (read-out scale).
 *  [RS]  "ReplaySSM -- buffered output-only decode for GDN/KDA", section 3.6
 *        (a negative slot index marks a padding row: output zeros, no state
 *        access) and section 3.8 (softplus taken as x above threshold 20).
 *  [TV]  "PR #26888 report: [KDA] target_verify for speculative decoding":
 *        verify runs the draft tokens without updating the pool and records
 *        the state after every draft position.
 *
 * Readings where the pages leave a step open are listed in the design notes
 * of the repository; the ones that shape this file are:
 *  - state layout S[K][V] with V contiguous (row = key channel);
 *  - inter[r, s] is the state AFTER token s of request r;
 *  - padding verify rows write o = 0 and leave inter untouched;
 *  - a zero-length sequence copies h0 (or zeros) to ht.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ gate */

/* softplus with the threshold 20 used by the pages' kernels ([RS] 3.8). */
static double ref_softplus(double x) { return x > 20.0 ? x : log1p(exp(x)); }
static double ref_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/*
 * [LA] "Gated DeltaNet" / "KDA": per key channel
 *   lower_bound == 0:  g = -exp(A_log[h]) * softplus(a + dt_bias[h, c])
 *   lower_bound <  0:  g = lower_bound * sigmoid(exp(A_log[h]) * (a + dt_bias[h, c]))
 *   beta = sigmoid(b)
 * a, g: [T, H, K]; b, beta: [T, H]; A_log: [H]; dt_bias: [H, K] or NULL (= 0).
 */
void kda_ref_gate(const double *a, const double *b, const double *A_log,
                  const double *dt_bias, int64_t T, int32_t H, int32_t K,
                  double lower_bound, double *g, double *beta) {
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t h = 0; h < H; ++h) {
      const double rate = exp(A_log[h]);
      for (int32_t c = 0; c < K; ++c) {
        const int64_t i = (t * H + h) * K + c;
        const double x = a[i] + (dt_bias ? dt_bias[(int64_t)h * K + c] : 0.0);
        if (lower_bound == 0.0)
          g[i] = -rate * ref_softplus(x);
        else
          g[i] = lower_bound * ref_sigmoid(rate * x);
      }
      beta[t * H + h] = ref_sigmoid(b[t * H + h]);
    }
  }
}

/* ------------------------------------------------------------ one token */

/*
 * One KDA token update on S[K][V] (V contiguous), in the order of [LA]
 * "Gated DeltaNet" (five steps) with the per-channel decay of [LA] "KDA":
 *   1. S'[i][:] = exp(g[i]) * S[i][:]        (forget, row i = key channel i)
 *   2. v_hat    = k S'                        (read the old value at key k)
 *   3. delta    = beta * (v - v_hat)          (error to write)
 *   4. S        = S' + k^T delta              (rank-1 write)
 *   5. o        = scale * q S                 (read-out after the write)
 * vh and dl are caller-provided scratch of length V.
 */
static void ref_step(double *S, const double *q, const double *k,
                     const double *v, const double *g, double beta,
                     double scale, int32_t K, int32_t V, double *o,
                     double *vh, double *dl) {
  for (int32_t i = 0; i < K; ++i) {
    const double a = exp(g[i]);
    for (int32_t j = 0; j < V; ++j) S[(int64_t)i * V + j] *= a;
  }
  for (int32_t j = 0; j < V; ++j) vh[j] = 0.0;
  for (int32_t i = 0; i < K; ++i)
    for (int32_t j = 0; j < V; ++j) vh[j] += k[i] * S[(int64_t)i * V + j];
  for (int32_t j = 0; j < V; ++j) dl[j] = beta * (v[j] - vh[j]);
  for (int32_t i = 0; i < K; ++i)
    for (int32_t j = 0; j < V; ++j) S[(int64_t)i * V + j] += k[i] * dl[j];
  for (int32_t j = 0; j < V; ++j) {
    double acc = 0.0;
    for (int32_t i = 0; i < K; ++i) acc += q[i] * S[(int64_t)i * V + j];
    o[j] = scale * acc;
  }
}

/* Single-step entry for the tests: S is updated in place, o written. */
void kda_ref_step(double *S, const double *q, const double *k, const double *v,
                  const double *g, double beta, double scale, int32_t K,
                  int32_t V, double *o) {
  double *vh = (double *)malloc(sizeof(double) * (size_t)V * 2);
  ref_step(S, q, k, v, g, beta, scale, K, V, o, vh, vh + V);
  free(vh);
}

/* ---------------------------------------------------- threaded work loop */

typedef void (*unit_fn)(void *ctx, int64_t unit, double *scratch);

typedef struct {
  unit_fn fn;
  void *ctx;
  int64_t n_units;
  int64_t next;
  pthread_mutex_t lock;
  int64_t scratch_len;
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  double *scratch = (double *)malloc(sizeof(double) * (size_t)p->scratch_len);
  for (;;) {
    pthread_mutex_lock(&p->lock);
    const int64_t u = p->next++;
    pthread_mutex_unlock(&p->lock);
    if (u >= p->n_units) break;
    p->fn(p->ctx, u, scratch);
  }
  free(scratch);
  return NULL;
}

/* Runs fn over independent units on nthreads threads (dynamic scheduling).
 * The units never share state, so the result does not depend on nthreads. */
static void run_units(unit_fn fn, void *ctx, int64_t n_units,
                      int64_t scratch_len, int nthreads) {
  pool_t p;
  p.fn = fn;
  p.ctx = ctx;
  p.n_units = n_units;
  p.next = 0;
  p.scratch_len = scratch_len;
  pthread_mutex_init(&p.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 1024) nthreads = 1024;
  if (nthreads == 1) {
    pool_worker(&p);
  } else {
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&tid[i], NULL, pool_worker, &p);
    for (int i = 0; i < nthreads; ++i) pthread_join(tid[i], NULL);
    free(tid);
  }
  pthread_mutex_destroy(&p.lock);
}

/* --------------------------------------------------------------- prefill */

typedef struct {
  const int64_t *cu;
  int32_t H, K, V;
  const double *q, *k, *v, *g, *beta, *h0;
  double scale;
  double *ht, *o;
} prefill_ctx;

static void prefill_unit(void *vctx, int64_t unit, double *scratch) {
  const prefill_ctx *c = (const prefill_ctx *)vctx;
  const int32_t H = c->H, K = c->K, V = c->V;
  const int64_t n = unit / H, h = unit % H;
  const int64_t KV = (int64_t)K * V;
  double *S = scratch, *vh = scratch + KV, *dl = vh + V;
  if (c->h0)
    memcpy(S, c->h0 + (n * H + h) * KV, sizeof(double) * (size_t)KV);
  else
    memset(S, 0, sizeof(double) * (size_t)KV);
  for (int64_t t = c->cu[n]; t < c->cu[n + 1]; ++t) {
    const int64_t th = t * H + h;
    ref_step(S, c->q + th * K, c->k + th * K, c->v + th * V, c->g + th * K,
             c->beta[th], c->scale, K, V, c->o + th * V, vh, dl);
  }
  if (c->ht) memcpy(c->ht + (n * H + h) * KV, S, sizeof(double) * (size_t)KV);
}

/*
 * Varlen prefill: sequence n owns tokens cu[n] .. cu[n+1]-1 of the packed
 * batch and starts from h0[n] (zeros when h0 is NULL).  Each (sequence, head)
 * runs the token recurrence from its first token to its last; ht[n] receives
 * the final state when ht is not NULL.
 *   q, k, g: [T, H, K]; v, o: [T, H, V]; beta: [T, H]; h0, ht: [N, H, K, V]
 * Returns 0, or -1 if cu_seqlens is not monotone from 0.
 */
int kda_ref_prefill(const int64_t *cu_seqlens, int32_t N, int32_t H, int32_t K,
                    int32_t V, const double *q, const double *k,
                    const double *v, const double *g, const double *beta,
                    double scale, const double *h0, double *ht, double *o,
                    int nthreads) {
  if (cu_seqlens[0] != 0) return -1;
  for (int32_t n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  prefill_ctx c = {cu_seqlens, H, K, V, q, k, v, g, beta, h0, scale, ht, o};
  run_units(prefill_unit, &c, (int64_t)N * H, (int64_t)K * V + 2 * V, nthreads);
  return 0;
}

/* ---------------------------------------------------------------- decode */

typedef struct {
  int32_t H, K, V, Tv;
  const double *q, *k, *v, *g, *beta;
  double scale;
  double *pool;        /* decode: updated in place */
  const double *cpool; /* verify: read only */
  int64_t n_slots;
  const int64_t *idx;
  double *inter, *o;
} step_ctx;

static void decode_unit(void *vctx, int64_t unit, double *scratch) {
  const step_ctx *c = (const step_ctx *)vctx;
  const int32_t H = c->H, K = c->K, V = c->V;
  const int64_t r = unit / H, h = unit % H, rh = r * H + h;
  const int64_t slot = c->idx[r];
  if (slot < 0) { /* padding row ([RS] 3.6) */
    for (int32_t j = 0; j < V; ++j) c->o[rh * V + j] = 0.0;
    return;
  }
  double *S = c->pool + (slot * H + h) * (int64_t)K * V;
  ref_step(S, c->q + rh * K, c->k + rh * K, c->v + rh * V, c->g + rh * K,
           c->beta[rh], c->scale, K, V, c->o + rh * V, scratch, scratch + V);
}

/*
 * Single-token decode on a slot-indexed state pool, in place.
 *   q, k, g: [B, H, K]; v, o: [B, H, V]; beta: [B, H];
 *   pool: [n_slots, H, K, V]; slot_idx: [B] (negative = padding row).
 * Returns 0, or -1 if a slot index is >= n_slots.
 */
int kda_ref_decode(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, double scale,
                   double *pool, int64_t n_slots, const int64_t *slot_idx,
                   int32_t B, int32_t H, int32_t K, int32_t V, double *o,
                   int nthreads) {
  for (int32_t r = 0; r < B; ++r)
    if (slot_idx[r] >= n_slots) return -1;
  step_ctx c = {H, K, V, 1, q, k, v, g, beta, scale, pool, NULL, n_slots,
                slot_idx, NULL, o};
  run_units(decode_unit, &c, (int64_t)B * H, 2 * V, nthreads);
  return 0;
}

/* ---------------------------------------------------------------- verify */

static void verify_unit(void *vctx, int64_t unit, double *scratch) {
  const step_ctx *c = (const step_ctx *)vctx;
  const int32_t H = c->H, K = c->K, V = c->V, Tv = c->Tv;
  const int64_t KV = (int64_t)K * V;
  const int64_t r = unit / H, h = unit % H;
  const int64_t slot = c->idx[r];
  if (slot < 0) {
    for (int32_t s = 0; s < Tv; ++s)
      for (int32_t j = 0; j < V; ++j)
        c->o[(((int64_t)r * Tv + s) * H + h) * V + j] = 0.0;
    return;
  }
  double *S = scratch, *vh = scratch + KV, *dl = vh + V;
  memcpy(S, c->cpool + (slot * H + h) * KV, sizeof(double) * (size_t)KV);
  for (int32_t s = 0; s < Tv; ++s) {
    const int64_t rsh = ((int64_t)r * Tv + s) * H + h;
    ref_step(S, c->q + rsh * K, c->k + rsh * K, c->v + rsh * V, c->g + rsh * K,
             c->beta[rsh], c->scale, K, V, c->o + rsh * V, vh, dl);
    memcpy(c->inter + rsh * KV, S, sizeof(double) * (size_t)KV);
  }
}

/*
 * Multi-token verify ([TV]): request r runs its Tv draft tokens from a copy of
 * pool[slot_idx[r]]; the pool is never written.  inter[r, s] = state after
 * draft token s.
 *   q, k, g: [B, Tv, H, K]; v, o: [B, Tv, H, V]; beta: [B, Tv, H];
 *   inter: [B, Tv, H, K, V].
 */
int kda_ref_verify(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, double scale,
                   const double *pool, int64_t n_slots,
                   const int64_t *slot_idx, int32_t B, int32_t Tv, int32_t H,
                   int32_t K, int32_t V, double *inter, double *o,
                   int nthreads) {
  for (int32_t r = 0; r < B; ++r)
    if (slot_idx[r] >= n_slots) return -1;
  step_ctx c = {H, K, V, Tv, q, k, v, g, beta, scale, NULL, pool, n_slots,
                slot_idx, inter, o};
  run_units(verify_unit, &c, (int64_t)B * H, (int64_t)K * V + 2 * V, nthreads);
  return 0;
}
