// Per-pair top-k neuron selection: the alternative to the threshold pass.
//
// gist.science page of arXiv 2605.08575, Technical Summary, Methodology,
// Activation Masking: the method masks with one elementwise threshold pass
// instead of selecting the top-k activations per token.  This kernel is that
// alternative, so that the two can be measured side by side: for every
// (token, slot) pair the `budget` neurons with the largest |a_j| are active.
// A NaN score ranks first, equal scores go to the lower neuron index.
//
// Unlike the threshold, a selection needs every score of the pair before any
// neuron is decided, so the layer runs the gate of every pair first (the
// projection's score mode), then this kernel, then the projection again with
// these masks (up and h only).
//
// One workgroup per grouped pair.  |a| read as an unsigned integer (sign bit
// cleared) orders like |a|, with NaN above +inf, so the budget-th largest key
// comes from an exact radix select: four passes over 8-bit digits, most
// significant first, each a 256-bin histogram of the keys that match the
// digits found so far, and a wavefront scan of the bins from the top.  The
// keys equal to the selected one are then ranked by neuron index (each thread
// owns a contiguous run of rows; a block scan orders the runs) and the lowest
// ones fill the budget.
#include "moe_internal.h"
#include "wave_reduce.h"

namespace moe {

constexpr int kTopkThreads = 256;

__device__ __forceinline__ uint32_t score_key(float a) { return __float_as_uint(a) & 0x7fffffffu; }

__global__ __launch_bounds__(kTopkThreads) void k_topk_select(TopkParams p)
{
    __shared__ uint32_t s_mask[kMaxRows / 32];
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_prefix;
    __shared__ int s_rank;
    __shared__ int s_wsum[kTopkThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;

    const int pr = blockIdx.x;  // grouped pair
    const int t = p.pair_tok[pr], slot = p.pair_slot[pr];
    const int xe = slot < p.K ? p.ids[(size_t)t * p.K + slot] : p.E + slot - p.K;
    const bool shared = xe >= p.E;
    const int Ie = shared ? p.Is : p.I;
    const int n = p.counts[xe], off = p.offsets[xe];
    // row r of this pair's scores is a[r * n] (per-expert blocks [rows][n])
    const float *a = p.a + (shared ? (size_t)p.A * p.I + (size_t)(off - p.A) * Ie : (size_t)off * Ie) + (pr - off);
    const int budget = min(p.budget, Ie);

    for (int w = tid; w < p.W; w += kTopkThreads) s_mask[w] = 0u;
    const int R = (Ie + kTopkThreads - 1) / kTopkThreads;  // contiguous rows per thread
    const int rb = min(Ie, tid * R), re = min(Ie, rb + R);

    uint32_t kstar = 0u;  // the budget-th largest key
    int need = 0;         // keys equal to kstar that are active (the lowest rows)
    if (budget > 0 && budget < Ie) {
        if (tid == 0) {
            s_prefix = 0u;
            s_rank = budget - 1;  // 0-indexed rank from the top
        }
        for (int d = 3; d >= 0; --d) {
            for (int i = tid; i < 256; i += kTopkThreads) s_hist[i] = 0u;
            __syncthreads();
            const uint32_t prefix = s_prefix;
            const int shift = 8 * d;
            for (int r = rb; r < re; ++r) {
                const uint32_t key = score_key(a[(size_t)r * n]);
                if (d == 3 || (key >> (shift + 8)) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (wave == 0) {
                // lane l holds bins 255 - 4l down to 252 - 4l (the scan runs from the top)
                uint32_t hb[4];
                int c = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    hb[j] = s_hist[255 - 4 * lane - j];
                    c += (int)hb[j];
                }
                const int incl = wave_incl_scan_dpp(c);
                const int k = s_rank;
                const uint64_t past = __ballot(incl > k);  // lanes whose bins reach rank k
                const int first = __ffsll((long long)past) - 1;
                if (lane == first) {
                    int cum = incl - c;
                    int digit = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (cum + (int)hb[j] > k) {
                            digit = 255 - 4 * lane - j;
                            break;
                        }
                        cum += (int)hb[j];
                    }
                    s_rank = k - cum;
                    s_prefix = (prefix << 8) | (uint32_t)digit;
                }
            }
            __syncthreads();
        }
        kstar = s_prefix;
        need = s_rank + 1;
    }

    // rank of this thread's first key equal to kstar among all of them, by row
    int ceq = 0;
    if (need > 0)
        for (int r = rb; r < re; ++r) ceq += score_key(a[(size_t)r * n]) == kstar ? 1 : 0;
    const int incl = wave_incl_scan_dpp(ceq);
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int eq = incl - ceq;
    for (int w = 0; w < wave; ++w) eq += s_wsum[w];

    for (int r = rb; r < re; ++r) {
        bool on;
        if (budget >= Ie) {
            on = true;
        } else if (budget <= 0) {
            on = false;
        } else {
            const uint32_t key = score_key(a[(size_t)r * n]);
            on = key > kstar || (key == kstar && eq++ < need);
        }
        if (on) atomicOr(&s_mask[r >> 5], 1u << (r & 31));
    }
    __syncthreads();
    for (int w = tid; w < p.W; w += kTopkThreads) p.pmask[(size_t)pr * p.W + w] = s_mask[w];
}

hipError_t launch_topk_select(const Plan &pl, const TopkParams &tp, hipStream_t st)
{
    if (pl.P <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_topk_select, dim3((unsigned)pl.P), dim3(kTopkThreads), 0, st, tp);
    return hipGetLastError();
}

}  // namespace moe
