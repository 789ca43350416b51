// Top-K softmax routing of one token by one wavefront, shared by the routing
// kernel and the single-launch decode path.  The router itself is unchanged
// by the method (gist.science page of arXiv 2605.08575, Technical Summary,
// Methodology: router logic preserved).
//
// The expert ids are found without K rounds of wavefront arg-max: each logit
// becomes an unsigned key in ranking order, and a bitwise search over ballots
// finds the K-th largest key (one step per key bit, each two compares per
// logit and a popcount; it stops early once exactly K keys lie at or above
// the prefix, which real-valued logits reach after a dozen bits or so).  The
// keys above it and the lowest-id ties at it are the chosen set; they are
// compacted into LDS as (key, inverted id) words, whose order is the slot
// order, and each one's slot is the number of words above it.  The weights
// need the ids' logits, not the reverse, so a caller that only needs the ids
// (to fetch an expert's rows) stops there.
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

// Token t's logits, KP per lane (expert lane + 64 i): as given, and as
// ranking values (NaN ranks as -inf); bit i of avail: expert lane + 64 i < E.
template <int KP>
struct TokenLogits {
    float raw[KP];
    float v[KP];
    uint32_t avail;
};

template <int KP>
__device__ __forceinline__ TokenLogits<KP> load_logits(const float *__restrict__ logits, int t, int E)
{
    const int lane = threadIdx.x & (kWave - 1);
    const float *l = logits + (size_t)t * E;
    TokenLogits<KP> g;
    g.avail = 0u;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        const int e = lane + kWave * i;
        g.raw[i] = e < E ? l[e] : 0.f;
        g.v[i] = (e < E && !isnan(g.raw[i])) ? g.raw[i] : -INFINITY;
        if (e < E) g.avail |= 1u << i;
    }
    return g;
}

// Unsigned key in the order of a ranking value (equal values, -0 and +0
// included, get equal keys).  Every value's key is at least that of -inf,
// 0x007fffff, so 0 marks an absent expert.
__device__ __forceinline__ uint32_t rank_key(float v)
{
    const uint32_t b = v == 0.f ? 0u : __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// LDS words per wavefront that select_topk needs: the chosen experts in id
// order, then in slot order.
constexpr int kSelWords = 2 * kMaxK;

// The K (1 <= K <= kMaxK, K <= E) largest ranking values, descending, ties to
// the lower id: lane k < K ends with the id of slot k and its ranking value.
// sel: this wavefront's kSelWords words of LDS.
template <int KP>
__device__ __forceinline__ void select_topk(const TokenLogits<KP> &g, int K, uint64_t *sel, int &id, float &vsel)
{
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t key[KP];
#pragma unroll
    for (int i = 0; i < KP; ++i) key[i] = ((g.avail >> i) & 1u) ? rank_key(g.v[i]) : 0u;

    // the K-th largest key: the largest x with at least K keys >= x, bit by
    // bit; a prefix with exactly K keys at or above it already separates them
    uint32_t kth = 0u;
#pragma unroll
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = kth | (1u << b);
        int n = 0;
#pragma unroll
        for (int i = 0; i < KP; ++i) n += __popcll(__ballot(key[i] >= cand));
        if (n >= K) {
            kth = cand;
            if (n == K) break;
        }
    }
    // chosen: the keys above kth, then the ties at it in ascending id order
    int above = 0;
#pragma unroll
    for (int i = 0; i < KP; ++i) above += __popcll(__ballot(key[i] > kth));
    const int need = K - above;  // ties taken (all of them when the search stopped early)
    int before = 0;  // ties, then chosen experts, at lower ids
    int nch = 0;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        const uint64_t eq = __ballot(key[i] == kth);
        const int pos = before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0u));
        const bool ch = key[i] > kth || (key[i] == kth && pos < need);
        before += __popcll(eq);
        // compacted in id order; a larger word ranks first (larger key, then lower id)
        const uint64_t cm = __ballot(ch);
        const int ci = nch + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(cm >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)cm, 0u));
        if (ch) sel[ci] = ((uint64_t)key[i] << 32) | (uint32_t)(~(uint32_t)(lane + kWave * i));
        nch += __popcll(cm);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane j < K: the slot of chosen word j is the number of chosen words above
    // it (eight words per round of LDS reads; words past K are not counted)
    const uint64_t mine = sel[lane < K ? lane : 0];
    int slot = 0;
    for (int c0 = 0; c0 < K; c0 += 8) {
        uint64_t o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o[u] = sel[c0 + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) slot += (c0 + u < K && o[u] > mine) ? 1 : 0;
    }
    if (lane < K) sel[kMaxK + slot] = mine;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint64_t w = sel[kMaxK + (lane < K ? lane : 0)];
    const uint32_t kk = (uint32_t)(w >> 32);
    id = lane < K ? (int)~(uint32_t)w : 0;
    // the ranking value back from its key (+0 for a zero of either sign, which
    // gives the same exponential)
    vsel = lane < K ? __uint_as_float((kk & 0x80000000u) ? (kk & 0x7fffffffu) : ~kk) : 0.f;
}

// Softmax weight of slot k in lane k < K (vsel: the slot's ranking value).
// The maximum is over the non-NaN logits (range-safe exponentials); the
// renormalising sum adds the chosen exponentials in slot order.
template <int KP>
__device__ __forceinline__ float slot_weights(const TokenLogits<KP> &g, int K, int renorm, float vsel)
{
    const int lane = threadIdx.x & (kWave - 1);
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < KP; ++i)
        if ((g.avail >> i) & 1u) m = fmaxf(m, g.v[i]);
    m = wave_max(m);
    float denom = 0.f;
#pragma unroll
    for (int i = 0; i < KP; ++i)
        if ((g.avail >> i) & 1u) denom += expf(g.raw[i] - m);
    denom = wave_sum_all(denom);
    // a chosen NaN logit ranks as -inf, so its exponential is 0; the
    // denominator is NaN then and so is every weight
    const float ev = lane < K ? expf(vsel - m) : 0.f;
    float sel_sum = 0.f;
    for (int k = 0; k < K; ++k) sel_sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ev), k));
    return slot_weight(ev, sel_sum, denom, renorm);
}

template <int KP>
__device__ __forceinline__ void route_token_kp(const float *__restrict__ logits, int t, int E, int K, int renorm,
                                               uint64_t *sel, int &id, float &wt)
{
    const TokenLogits<KP> g = load_logits<KP>(logits, t, E);
    float vsel;
    select_topk<KP>(g, K, sel, id, vsel);
    wt = slot_weights<KP>(g, K, renorm, vsel);
}

template <int KP>
__device__ __forceinline__ int route_ids_kp(const float *__restrict__ logits, int t, int E, int K, uint64_t *sel)
{
    const TokenLogits<KP> g = load_logits<KP>(logits, t, E);
    int id;
    float vsel;
    select_topk<KP>(g, K, sel, id, vsel);
    return id;
}

// Routes token t with one wavefront (E <= 512, sel: its kSelWords words of
// LDS): lane k < K ends with the expert id and the weight of slot k.  E
// decides how many logits a lane holds.
__device__ __forceinline__ void route_token(const float *__restrict__ logits, int t, int E, int K, int renorm,
                                            uint64_t *sel, int &id, float &wt)
{
    if (E <= kWave) route_token_kp<1>(logits, t, E, K, renorm, sel, id, wt);
    else if (E <= 2 * kWave) route_token_kp<2>(logits, t, E, K, renorm, sel, id, wt);
    else if (E <= 4 * kWave) route_token_kp<4>(logits, t, E, K, renorm, sel, id, wt);
    else route_token_kp<kMaxExperts / kWave>(logits, t, E, K, renorm, sel, id, wt);
}

// The expert ids alone (lane k < K: slot k), as route_token finds them.
__device__ __forceinline__ int route_token_ids(const float *__restrict__ logits, int t, int E, int K, uint64_t *sel)
{
    if (E <= kWave) return route_ids_kp<1>(logits, t, E, K, sel);
    if (E <= 2 * kWave) return route_ids_kp<2>(logits, t, E, K, sel);
    if (E <= 4 * kWave) return route_ids_kp<4>(logits, t, E, K, sel);
    return route_ids_kp<kMaxExperts / kWave>(logits, t, E, K, sel);
}

}  // namespace moe
