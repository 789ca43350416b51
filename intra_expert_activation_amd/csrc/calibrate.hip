// Threshold calibration: exact order statistic of |SiLU(gate)| scores.
//
// gist.science page of arXiv 2605.08575, Technical Summary, Results: models
// are run at a target intra-expert sparsity.  The threshold for sparsity q is
// v[floor(q*N)] of the ascending scores v, so floor(q*N) scores fall below it.
//
// Non-negative IEEE floats order like their bit patterns read as unsigned
// integers (NaN with the sign bit clear after |.| sorts above +inf), so the
// selection is an exact radix select: four passes over 8-bit digits, most
// significant first; each pass histograms the digit of the candidates that
// match the prefix found so far and keeps the bin holding the wanted rank.
// One workgroup per population: 0 = routed pairs, 1 = shared experts, then one
// per expert when per-expert thresholds are requested.
#include <math.h>

#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(1024) void k_select(SelectParams p)
{
    __shared__ unsigned int s_hist[256];
    __shared__ unsigned int s_prefix;
    __shared__ unsigned long long s_rank;

    const int pop = blockIdx.x;
    size_t begin = 0, N = 0;
    if (pop == 0) {
        begin = 0;
        N = (size_t)p.A * p.I;
    } else if (pop == 1) {
        begin = (size_t)p.A * p.I;
        N = (size_t)p.S * p.T * p.Is;
    } else {
        const int xe = pop - 2;
        const bool shared = xe >= p.E;
        const int Ie = shared ? p.Is : p.I;
        const int off = p.offsets[xe];
        begin = shared ? (size_t)p.A * p.I + (size_t)(off - p.A) * Ie : (size_t)off * Ie;
        N = (size_t)p.counts[xe] * Ie;
    }
    float result;
    const double kappa_d = floor((double)p.q * (double)N);
    if (N == 0) {
        result = 0.f;  // no population (unused: the finalize step falls back by the pair count)
    } else if (p.q == 0.f) {
        result = 0.f;
    } else if (kappa_d >= (double)N) {
        result = INFINITY;
    } else {
        const unsigned int *v = reinterpret_cast<const unsigned int *>(p.scores + begin);
        if (threadIdx.x == 0) {
            s_prefix = 0u;
            s_rank = (unsigned long long)kappa_d;
        }
        for (int d = 3; d >= 0; --d) {
            for (int i = threadIdx.x; i < 256; i += blockDim.x) s_hist[i] = 0u;
            __syncthreads();
            const unsigned int prefix = s_prefix;
            const int shift = 8 * d;
            for (size_t i = threadIdx.x; i < N; i += blockDim.x) {
                const unsigned int key = v[i] & 0x7fffffffu;
                if (d == 3 || (key >> (shift + 8)) == prefix)
                    atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                unsigned long long k = s_rank, cum = 0;
                int digit = 255;
                for (int b = 0; b < 256; ++b) {
                    if (cum + s_hist[b] > k) {
                        digit = b;
                        break;
                    }
                    cum += s_hist[b];
                }
                s_rank = k - cum;
                s_prefix = (prefix << 8) | (unsigned int)digit;
            }
            __syncthreads();
        }
        result = __uint_as_float(s_prefix);
    }
    if (threadIdx.x == 0) p.taus[pop] = result;
}

// tau_out[e]: routed experts take the routed population's value (or their own
// when per_expert, falling back to the routed value when the expert has no
// calibration pair); shared experts take the shared population's value (or
// their own; a shared expert has a pair for every token).  An expert's own
// order statistic is kept even when it is NaN (NaN scores order after
// +infinity, so a high q over a population holding NaN scores selects one):
// only the pair count, never the value, decides the fallback.
__global__ void k_select_finalize(const float *taus, const int32_t *counts, int E, int S, int per_expert,
                                  float *tau_out)
{
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E + S) return;
    float t = (e < E) ? taus[0] : taus[1];
    if (per_expert && counts[e] > 0) t = taus[2 + e];
    tau_out[e] = t;
}

hipError_t launch_select(const Plan &pl, const SelectParams &sp, float *tau_out, hipStream_t st)
{
    const int pops = 2 + (sp.per_expert ? sp.EX : 0);
    hipLaunchKernelGGL(k_select, dim3(pops), dim3(1024), 0, st, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_select_finalize, dim3((sp.EX + 255) / 256), dim3(256), 0, st, sp.taus, sp.counts,
                       sp.E, sp.S, sp.per_expert, tau_out);
    return hipGetLastError();
}

}  // namespace moe
