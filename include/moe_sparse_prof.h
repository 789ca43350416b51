/*
 * moe_sparse_prof.h -- measurement hooks of libmoesparse, kept apart from the
 * method's calls in moe_sparse.h.  Benchmarks use them to time the dominant
 * kernel of a layer call on the stream it is launched on; nothing else in the
 * library depends on them.
 *
 * Conventions are those of moe_sparse.h (device pointers owned by the caller,
 * host-detectable errors returned before any HIP call, nothing printed).
 */
#ifndef MOE_SPARSE_PROF_H
#define MOE_SPARSE_PROF_H

#include "moe_sparse.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * moe_sparse_expert_ffn with two events that time the expert projection
 * kernel (gate, score, mask, up) on hip_stream.  The kernel is dispatched by
 * hipExtLaunchKernelGGL with ev_begin / ev_end as its start and stop events,
 * so they take the kernel's own begin and end times (events recorded around
 * a plain launch would also count its dispatch).  Where the projection is
 * two launches (rows wider than 2048 bf16 elements with MFMA experts: the
 * GEMV and the MFMA launch), ev_begin goes with the first and ev_end with the
 * second; in MOE_TOPK mode they span its score pass, selection and masked
 * pass.  On the one-launch path (batches of one token, and small batches of
 * layers whose experts' gates hold at most 16 MiB each) they time the kernel
 * that also runs routing and the down projection.  ev_begin / ev_end are
 * hipEvent_t handles (for example from moe_timer_create), either may be
 * NULL.  This call is for eager timing; capture moe_sparse_expert_ffn in a
 * graph instead.  Results, errors and workspace are exactly those of
 * moe_sparse_expert_ffn.
 */
moe_status moe_sparse_expert_ffn_profiled(const moe_shape *shape, int32_t mode, const moe_ffn_args *args,
                                          void *ev_begin, void *ev_end, void *hip_stream);

/* A hipEvent_t with timing enabled, destroyed by moe_timer_destroy;
 * moe_timer_elapsed_ms waits for `end` and returns the milliseconds between
 * two recorded events. */
moe_status moe_timer_create(void **event);
moe_status moe_timer_destroy(void *event);
moe_status moe_timer_elapsed_ms(void *begin, void *end, float *ms);

#ifdef __cplusplus
}
#endif

#endif /* MOE_SPARSE_PROF_H */
