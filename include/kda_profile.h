/*
 * kda_profile.h -- timing hook of libkda for benchmarks and profilers.  It is
 * not part of the computation's interface (include/kda.h); it records HIP
 * events around the prefill's kernels so that each kernel can be timed on
 * the stream it runs on.
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

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* KDA_PROFILE_H_ */
