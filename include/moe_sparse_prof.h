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
 * moe_sparse_expert_ffn with two events recorded on hip_stream around the
 * expert projection kernel (gate, score, mask, up).  On the one-launch path
 * (batches of one token, and small batches of layers whose experts' gates
 * hold at most 16 MiB each) they bracket the kernel that also runs routing
 * and the down projection.  ev_begin / ev_end are hipEvent_t handles (for
 * example from moe_timer_create), either may be NULL.  Results, errors and
 * workspace are exactly those of moe_sparse_expert_ffn.
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
