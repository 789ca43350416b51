// Top-K softmax routing of one token by one wavefront, shared by the routing
// kernel and the single-launch decode path.  The router itself is unchanged
// by the method (gist.science page of arXiv 2605.08575, Technical Summary,
// Methodology: router logic preserved).
#pragma once

#include "moe_internal.h"
#include "wave_reduce.h"

namespace moe {

// Weight of a chosen expert with exp value ev: its softmax probability
// ev / denom, or renormalised over the K chosen, ev / sel_sum (the same
// quotient of probabilities with denom cancelled).  A NaN denominator (a NaN
// or +inf logit) makes every probability NaN, and so every weight.
__device__ __forceinline__ float slot_weight(float ev, float sel_sum, float denom, int renorm)
{
    if (!renorm) return ev / denom;
    return isnan(denom) ? denom : ev / sel_sum;
}

// Routes token t with one wavefront, KP logits per lane (E <= 64 * KP): lane
// k < K ends with the expert id and the weight of slot k.
template <int KP>
__device__ __forceinline__ void route_token_kp(const float *__restrict__ logits, int t, int E, int K, int renorm,
                                               int &id, float &wt)
{
    const int lane = threadIdx.x & (kWave - 1);
    const float *l = logits + (size_t)t * E;
    float v[KP];        // ranking value (NaN ranks as -inf)
    float raw[KP];      // logit as given
    uint32_t avail = 0; // bit i: expert lane + 64 i is present and not yet chosen
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        const int e = lane + kWave * i;
        raw[i] = e < E ? l[e] : 0.f;
        v[i] = (e < E && !isnan(raw[i])) ? raw[i] : -INFINITY;
        if (e < E) avail |= 1u << i;
    }
    // maximum over the non-NaN logits, for a range-safe softmax
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < KP; ++i)
        if ((avail >> i) & 1u) m = fmaxf(m, v[i]);
    m = wave_max(m);
    float denom = 0.f;
#pragma unroll
    for (int i = 0; i < KP; ++i)
        if ((avail >> i) & 1u) denom += expf(raw[i] - m);
    denom = wave_sum_all(denom);

    float chosen_e = 0.f;  // lane k keeps exp(l - m) of slot k, and its expert
    int chosen_id = 0;
    float sel_sum = 0.f;
    for (int k = 0; k < K; ++k) {
        // lane-local best available expert (ascending ids: ties keep the lower)
        float bv = -INFINITY;
        int bid = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            if (((avail >> i) & 1u) && (bid == 0x7fffffff || v[i] > bv)) {
                bv = v[i];
                bid = lane + kWave * i;
            }
        }
        // wavefront arg-max: the largest value, then the lowest id holding it
        const float top = wave_max(bid == 0x7fffffff ? -INFINITY : bv);
        const int win = wave_min((bid != 0x7fffffff && bv == top) ? bid : 0x7fffffff);
        if ((win & (kWave - 1)) == lane) avail &= ~(1u << (win / kWave));
        // exp of the chosen logit: its ranking value is the logit itself unless
        // the logit is NaN, and then the denominator is NaN and so is every weight
        const float ev = expf(top - m);
        if (lane == k) {
            chosen_e = ev;
            chosen_id = win;
        }
        sel_sum += ev;
    }
    id = chosen_id;
    wt = slot_weight(chosen_e, sel_sum, denom, renorm);
}

// Routes token t with one wavefront (E <= 512): lane k < K ends with the
// expert id and the weight of slot k.  E decides how many logits a lane holds.
__device__ __forceinline__ void route_token(const float *__restrict__ logits, int t, int E, int K, int renorm,
                                            int &id, float &wt)
{
    if (E <= kWave) route_token_kp<1>(logits, t, E, K, renorm, id, wt);
    else if (E <= 2 * kWave) route_token_kp<2>(logits, t, E, K, renorm, id, wt);
    else if (E <= 4 * kWave) route_token_kp<4>(logits, t, E, K, renorm, id, wt);
    else route_token_kp<kMaxExperts / kWave>(logits, t, E, K, renorm, id, wt);
}

}  // namespace moe
