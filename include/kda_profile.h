/*
 * kda_profile.h -- timing hooks of libkda for benchmarks and profilers.  They
 * are not part of the computation's interface (include/kda.h): one records
 * HIP events around the prefill's kernels so that each stage can be timed on
 * the stream it runs on, the other says which kernels a prefill call of
 * given sizes launches.
 */
#ifndef KDA_PROFILE_H_
#define KDA_PROFILE_H_

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * kda_chunk_prefill_gated (include/kda.h) with kernel timing marks.  Same
 * arguments, work and results; in addition it records four caller-created
 * HIP events (hipEvent_t passed as void*) on `stream`: marks[0] before the
 * chunk-table kernel, marks[1] before the intra-chunk kernel, marks[2]
 * before the inter-chunk state pass and marks[3] after it, so that the
 * elapsed time between consecutive marks is one stage's duration.  A NULL
 * `marks` or a NULL entry returns KDA_ERR_INVALID_ARGUMENT with nothing
 * enqueued; a failed event record returns KDA_ERR_LAUNCH.
 */
kda_status kda_chunk_prefill_marked(kda_dtype io, const void* q, const void* k,
                                    const void* v, const float* a, const float* b,
                                    const float* A_log, const float* dt_bias,
                                    float lower_bound, const int32_t* cu_seqlens,
                                    int32_t N, int64_t T, int32_t H, int32_t K,
                                    int32_t V, int32_t chunk, float scale,
                                    const float* h0, float* ht, void* o,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream, void* const* marks);

/*
 * How a prefill call of these sizes is scheduled (the kernels it launches
 * depend on the sizes only, not on the sequence lengths), so that a profiler
 * trace can be matched to the call:
 *   n_waves         > 1: the chain of chunks is cut into that many waves; the
 *                   intra-chunk kernel of wave p runs beside the state pass
 *                   of wave p - 1 (on a second stream unless the call is
 *                   kda_chunk_prefill_marked or kda_chunk_prefill_noalloc);
 *   segment_chunks  chunks per segment of a cut chain (0: not cut);
 *   uses_maps       1: middle segments are first run as affine maps, then
 *                   chained by a scan kernel and re-run from their starts;
 *   intra_launches, state_launches: launches of the intra-chunk kernel and of
 *                   the state-pass kernel; other_launches: the chunk-table
 *                   kernel and, with maps, the scan kernel.
 * Sizes the prefill entry points reject return the status they would.
 */
typedef struct {
  int32_t n_waves;
  int32_t segment_chunks;
  int32_t uses_maps;
  int32_t intra_launches;
  int32_t state_launches;
  int32_t other_launches;
} kda_prefill_schedule;

kda_status kda_chunk_prefill_schedule(int64_t T, int32_t N, int32_t H, int32_t K,
                                      int32_t V, int32_t chunk,
                                      kda_prefill_schedule* out);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* KDA_PROFILE_H_ */
