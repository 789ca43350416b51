// Down projection over an expert's active neurons, and the top-K weighted
// combine.
//
// gist.science page of arXiv 2605.08575, Technical Summary, Methodology,
// "Fused Up-Down Projection": only active neurons' weights are gathered.  With
// the down matrix stored neuron-major, an active neuron is one contiguous row
// of H elements and an inactive one is never read.
//
// k_down: one workgroup per (touched expert, column tile, split).  It expands
// the expert's union bit words into an ascending row list in LDS (popcount
// prefix), takes its split of that list, and accumulates
//     o[pair, cols] += h[row][pair] * w_down[row][cols]
// for every pair of the expert in register tiles of TB tokens.  The 4
// wavefronts take interleaved rows of the split and are summed through LDS in
// a fixed order; splits land in separate partial buffers that the combine
// kernel adds in a fixed order, so no floating-point atomics are used and the
// result is bitwise reproducible.
#include "moe_internal.h"

namespace moe {

template <class Tr, int UR, int TB>
struct DownBatch {
    typename Tr::V w[UR];
    float h[UR][TB];
};

// Loads of the wavefront's next UR rows of the split: this lane's 16-byte
// vector of each down row and the tile's h values of each row.
template <class Tr, int UR, int TB, int MODE>
__device__ __forceinline__ void load_down_batch(DownBatch<Tr, UR, TB> &bt, const typename Tr::V *Wd,
                                                const float *hb, const uint16_t *list, int i0, int hi,
                                                int n, int t0, int nt, int rowV)
{
#pragma unroll
    for (int u = 0; u < UR; ++u) {
        const int i = i0 + 4 * u;
        const int j = (i < hi) ? ((MODE == MOE_DENSE) ? i : (int)list[i]) : -1;
        bt.w[u] = (j >= 0) ? Wd[(size_t)j * rowV] : Tr::zero();
#pragma unroll
        for (int t = 0; t < TB; ++t) bt.h[u][t] = (j >= 0 && t < nt) ? hb[(size_t)j * n + t0 + t] : 0.f;
    }
}

template <class Tr, int UR, int TB>
__device__ __forceinline__ void fma_down_batch(const DownBatch<Tr, UR, TB> &bt, float (&acc)[TB][Tr::kEpl])
{
#pragma unroll
    for (int u = 0; u < UR; ++u) {
        float wf[Tr::kEpl];
        Tr::unpack(bt.w[u], wf);
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int e = 0; e < Tr::kEpl; ++e) acc[t][e] = fmaf(bt.h[u][t], wf[e], acc[t][e]);
    }
}

template <class Tr, int TB, int MODE>
__global__ __launch_bounds__(256) void k_down(DownParams p)
{
    using V = typename Tr::V;
    constexpr int EPL = Tr::kEpl;
    constexpr int UR = 4;  // rows per batch per wavefront; two batches in flight
    extern __shared__ uint16_t s_list[];  // the expert's union rows, ascending
    __shared__ float s_red[2][TB][kWave * EPL];
    __shared__ int s_wpre[4];

    const int per_e = p.NCT * p.NSPLIT;
    const int s = blockIdx.x / per_e;
    const int rem = blockIdx.x - s * per_e;
    const int ct = rem / p.NSPLIT;
    const int sp = rem - ct * p.NSPLIT;
    if (s >= p.hdr[0]) return;
    const int xe = p.touched[s];
    const bool shared = xe >= p.E;
    const int Ie = shared ? p.Is : p.I;
    const int n = p.counts[xe];
    if (n >= p.nm) return;  // this expert takes the MFMA path
    const int off = p.offsets[xe];
    const int rowV = p.NCT * kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int cv = ct * kWave + lane;  // this lane's vector of each row
    const size_t mat = (size_t)(shared ? xe - p.E : xe) * Ie * rowV;
    const V *Wd = reinterpret_cast<const V *>(shared ? p.swd : p.wd) + mat + cv;
    const float *hb = p.h + (shared ? (size_t)p.A * p.I + (size_t)(off - p.A) * Ie : (size_t)off * Ie);

    // ---- union row list -----------------------------------------------------
    int U;
    if (MODE == MOE_DENSE) {
        U = Ie;
    } else {
        const int nw = Ie / 32;
        const uint32_t *uw = p.union_words + (size_t)xe * p.W;
        // popcount prefix over the words: thread i owns words [i*per, i*per+per)
        const int per = (nw + blockDim.x - 1) / blockDim.x;
        const int w_begin = threadIdx.x * per;
        int cnt = 0;
        for (int i = 0; i < per; ++i)
            if (w_begin + i < nw) cnt += __popc(uw[w_begin + i]);
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += o;
        }
        if (lane == kWave - 1) s_wpre[wave] = incl;
        __syncthreads();
        int wbase = 0;
        for (int i = 0; i < wave; ++i) wbase += s_wpre[i];
        U = s_wpre[0] + s_wpre[1] + s_wpre[2] + s_wpre[3];
        int pos = wbase + incl - cnt;
        for (int i = 0; i < per; ++i) {
            const int wd = w_begin + i;
            if (wd >= nw) break;
            uint32_t bits = uw[wd];
            while (bits) {
                const int b = __ffs(bits) - 1;
                bits &= bits - 1;
                s_list[pos++] = (uint16_t)(wd * 32 + b);
            }
        }
        __syncthreads();
    }
    if (ct == 0 && sp == 0) {
        if (p.union_idx)
            for (int i = threadIdx.x; i < U; i += blockDim.x)
                p.union_idx[(size_t)xe * p.Imax + i] = (MODE == MOE_DENSE) ? i : (int)s_list[i];
        if (p.union_cnt && threadIdx.x == 0) p.union_cnt[xe] = U;
    }

    const int lo = (int)(((long long)U * sp) / p.NSPLIT);
    const int hi = (int)(((long long)U * (sp + 1)) / p.NSPLIT);
    const int mine = hi - lo - wave > 0 ? (hi - lo - wave + 3) / 4 : 0;  // rows of this wavefront
    const int nb = (mine + UR - 1) / UR;

    for (int t0 = 0; t0 < n; t0 += TB) {
        const int nt = min(TB, n - t0);
        float acc[TB][EPL];
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[t][e] = 0.f;

        // rows lo + wave + 4 i of the split, batches of UR, two in flight
        DownBatch<Tr, UR, TB> A, B;
        if (nb > 0) load_down_batch<Tr, UR, TB, MODE>(A, Wd, hb, s_list, lo + wave, hi, n, t0, nt, rowV);
#pragma unroll 1
        for (int b = 0; b < nb; b += 2) {
            if (b + 1 < nb)
                load_down_batch<Tr, UR, TB, MODE>(B, Wd, hb, s_list, lo + wave + 4 * UR * (b + 1), hi, n, t0, nt, rowV);
            fma_down_batch<Tr, UR, TB>(A, acc);
            if (b + 1 >= nb) break;
            if (b + 2 < nb)
                load_down_batch<Tr, UR, TB, MODE>(A, Wd, hb, s_list, lo + wave + 4 * UR * (b + 2), hi, n, t0, nt, rowV);
            fma_down_batch<Tr, UR, TB>(B, acc);
        }

        // wavefront sums in a fixed order: (w0 + w2) + (w1 + w3)
        if (wave >= 2) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
#pragma unroll
                for (int e = 0; e < EPL; ++e) s_red[wave - 2][t][lane * EPL + e] = acc[t][e];
        }
        __syncthreads();
        if (wave < 2) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[t][e] += s_red[wave][t][lane * EPL + e];
        }
        __syncthreads();
        if (wave == 1) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
#pragma unroll
                for (int e = 0; e < EPL; ++e) s_red[0][t][lane * EPL + e] = acc[t][e];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                if (t >= nt) break;
                float o[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[e] = acc[t][e] + s_red[0][t][lane * EPL + e];
                float *dst = p.partial + ((size_t)sp * p.P + off + t0 + t) * p.H + (size_t)cv * EPL;
#pragma unroll
                for (int e = 0; e < EPL; e += 4)
                    *reinterpret_cast<float4 *>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
            }
        }
        __syncthreads();  // s_red is rewritten by the next tile
    }
}

template <class Tr, int TB>
static hipError_t launch_down_t(const Plan &pl, const DownParams &dp, int mode, hipStream_t st)
{
    const dim3 grid(pl.max_touched * pl.NCT * pl.NSPLIT), block(256);
    const size_t lds = (size_t)pl.Imax * sizeof(uint16_t);
    if (mode == MOE_DENSE) hipLaunchKernelGGL((k_down<Tr, TB, MOE_DENSE>), grid, block, 0, st, dp);
    else hipLaunchKernelGGL((k_down<Tr, TB, MOE_SPARSE>), grid, block, lds, st, dp);
    return hipGetLastError();
}

template <class Tr>
static hipError_t launch_down_tr(const Plan &pl, const DownParams &dp, int mode, hipStream_t st)
{
    switch (pl.TT) {
    case 1: return launch_down_t<Tr, 1>(pl, dp, mode, st);
    case 2: return launch_down_t<Tr, 2>(pl, dp, mode, st);
    case 4: return launch_down_t<Tr, 4>(pl, dp, mode, st);
    case 8: return launch_down_t<Tr, 8>(pl, dp, mode, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_down(const Plan &pl, const DownParams &dp, int mode, hipStream_t st)
{
    if (pl.T <= 0) return hipSuccess;
    return pl.dtype == MOE_BF16 ? launch_down_tr<BF16>(pl, dp, mode, st)
                                : launch_down_tr<F32>(pl, dp, mode, st);
}

// ---------------------------------------------------------------------------
// k_combine: y[t] = sum_{k<K} w[t,k] * o[pos(t,k)] + sum_{s<S} o[pos(t,K+s)],
// with o the sum of the NSPLIT partials (one partial for an expert on the MFMA
// path).  A workgroup covers one token and 256
// columns: 64 column quads x 4 thread groups; group g adds the terms
// (slot, split) with (slot * NSPLIT + split) % 4 == g, and the 4 group sums
// meet in LDS in a fixed order (so the result is deterministic).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(CombineParams p)
{
    __shared__ float4 s_acc[3][64];
    const int t = blockIdx.x;
    const int q = threadIdx.x & 63;  // column quad within the block
    const int g = threadIdx.x >> 6;  // term group
    const int c4 = blockIdx.y * 64 + q;
    const int H4 = p.H / 4;
    const bool live = c4 < H4;
    const int nterms = p.slots * p.NSPLIT;
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
        for (int i = g; i < nterms; i += 4) {
            const int k = i / p.NSPLIT, sp = i - k * p.NSPLIT;
            const int e = (k < p.K) ? p.topk_ids[(size_t)t * p.K + k] : p.E + (k - p.K);
            if (sp > 0 && p.counts[e] >= p.nm) continue;  // MFMA experts write split 0 only
            const int pr = p.pos[(size_t)t * p.slots + k];
            const float wk = (k < p.K) ? p.topk_w[(size_t)t * p.K + k] : 1.f;
            const float4 v = reinterpret_cast<const float4 *>(p.partial + ((size_t)sp * p.P + pr) * p.H)[c4];
            y.x = fmaf(wk, v.x, y.x);
            y.y = fmaf(wk, v.y, y.y);
            y.z = fmaf(wk, v.z, y.z);
            y.w = fmaf(wk, v.w, y.w);
        }
    }
    if (g > 0) s_acc[g - 1][q] = y;
    __syncthreads();
    if (g == 0 && live) {
        const float4 a = s_acc[0][q], b = s_acc[1][q], c = s_acc[2][q];
        y.x = (y.x + a.x) + (b.x + c.x);
        y.y = (y.y + a.y) + (b.y + c.y);
        y.z = (y.z + a.z) + (b.z + c.z);
        y.w = (y.w + a.w) + (b.w + c.w);
        reinterpret_cast<float4 *>(p.y + (size_t)t * p.H)[c4] = y;
    }
}

hipError_t launch_combine(const Plan &pl, const CombineParams &cp, hipStream_t st)
{
    if (pl.T <= 0) return hipSuccess;
    const int H4 = pl.H / 4;
    hipLaunchKernelGGL(k_combine, dim3(pl.T, (H4 + 63) / 64), dim3(256), 0, st, cp);
    return hipGetLastError();
}

}  // namespace moe
