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
#include <type_traits>

#include "mfma_body.h"
#include "moe_internal.h"

namespace moe {

constexpr int kDownRowChunk = 256;  // rows of h staged in LDS at a time

// Loads of the wavefront's next UR rows: this lane's 16-byte vector of each
// down row (rows past `hi` read as zero).
template <class Tr, int UR, int MODE>
__device__ __forceinline__ void load_down_rows(typename Tr::V (&w)[UR], const typename Tr::V *Wd,
                                               const uint16_t *list, int i0, int hi, int rowV)
{
#pragma unroll
    for (int u = 0; u < UR; ++u) {
        const int i = i0 + 4 * u;
        const int j = (i < hi) ? ((MODE == MOE_DENSE) ? i : (int)list[i]) : -1;
        w[u] = (j >= 0) ? Wd[(size_t)j * rowV] : Tr::zero();
    }
}

// acc[t][:] += h[row][t] * w[row][:] for the batch; h comes from LDS (one
// broadcast read per 4 tokens), rows past the chunk contribute zero weights.
template <class Tr, int UR, int TB>
__device__ __forceinline__ void fma_down_rows(const typename Tr::V (&w)[UR], const float *s_h, int r0,
                                              float (&acc)[TB][Tr::kEpl])
{
#pragma unroll
    for (int u = 0; u < UR; ++u) {
        float wf[Tr::kEpl];
        Tr::unpack(w[u], wf);
        const float *hr = s_h + (size_t)(r0 + 4 * u) * TB;
        float hv[TB];
#pragma unroll
        for (int t = 0; t < TB; t += (TB >= 4 ? 4 : TB)) {
            if constexpr (TB >= 4) {
                const float4 q = *reinterpret_cast<const float4 *>(hr + t);
                hv[t] = q.x; hv[t + 1] = q.y; hv[t + 2] = q.z; hv[t + 3] = q.w;
            } else {
#pragma unroll
                for (int k = 0; k < TB; ++k) hv[k] = hr[k];
            }
        }
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int e = 0; e < Tr::kEpl; ++e) acc[t][e] = fmaf(hv[t], wf[e], acc[t][e]);
    }
}

// One token tile of TB tokens (nt valid): the split's rows of this column tile.
// The tile's h values of the split's rows are staged in LDS, kDownRowChunk
// rows at a time ([row][TB], zero past nt and past the split).
template <class Tr, int TB, int TBMAX, int MODE>
__device__ __forceinline__ void down_tile(const DownParams &p, float (&s_red)[2][TBMAX][kWave * Tr::kEpl],
                                          float *s_h, const uint16_t *s_list, const typename Tr::V *Wd,
                                          const float *hb, int n, int off, int t0, int nt, int lo, int hi,
                                          int sp, int cv, int rowV, int lane, int wave)
{
    constexpr int EPL = Tr::kEpl;
    constexpr int UR = 4;  // rows per batch per wavefront; two batches in flight
    float acc[TB][EPL];
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[t][e] = 0.f;

    for (int c0 = lo; c0 < hi; c0 += kDownRowChunk) {
        const int c1 = min(hi, c0 + kDownRowChunk);
        // stage h[row][t] for rows c0..c1 (padded to a multiple of 4 * UR rows)
        const int rows = ((c1 - c0 + 4 * UR - 1) / (4 * UR)) * (4 * UR);
        for (int q = threadIdx.x; q < rows * TB; q += blockDim.x) {
            const int r = q / TB, t = q - r * TB;
            const int i = c0 + r;
            float v = 0.f;
            if (i < c1 && t < nt) {
                const int j = (MODE == MOE_DENSE) ? i : (int)s_list[i];
                v = hb[(size_t)j * n + t0 + t];
            }
            s_h[q] = v;
        }
        __syncthreads();
        // rows c0 + wave + 4 i of the chunk, batches of UR, two in flight
        const int mine = c1 - c0 - wave > 0 ? (c1 - c0 - wave + 3) / 4 : 0;
        const int nb = (mine + UR - 1) / UR;
        typename Tr::V A[UR], B[UR];
        if (nb > 0) load_down_rows<Tr, UR, MODE>(A, Wd, s_list, c0 + wave, c1, rowV);
#pragma unroll 1
        for (int b = 0; b < nb; b += 2) {
            if (b + 1 < nb) load_down_rows<Tr, UR, MODE>(B, Wd, s_list, c0 + wave + 4 * UR * (b + 1), c1, rowV);
            fma_down_rows<Tr, UR, TB>(A, s_h, wave + 4 * UR * b, acc);
            if (b + 1 >= nb) break;
            if (b + 2 < nb) load_down_rows<Tr, UR, MODE>(A, Wd, s_list, c0 + wave + 4 * UR * (b + 2), c1, rowV);
            fma_down_rows<Tr, UR, TB>(B, s_h, wave + 4 * UR * (b + 1), acc);
        }
        __syncthreads();  // s_h is rewritten by the next chunk
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

template <int TBMAX, int EPL>
struct DownLds {
    float red[2][TBMAX][kWave * EPL];
    float h[kDownRowChunk * TBMAX];
    int wpre[4];
};

// The GEMV down projection of workgroup `bid`: (expert, column tile, split).
template <class Tr, int TBMAX, int MODE>
__device__ __forceinline__ void down_gemv(const DownParams &p, DownLds<TBMAX, Tr::kEpl> &D, int bid)
{
    using V = typename Tr::V;
    extern __shared__ uint16_t s_list[];  // the expert's union rows, ascending (dynamic LDS)
    auto &s_red = D.red;
    float *s_h = D.h;
    auto &s_wpre = D.wpre;

    const int per_e = p.NCT * p.NSPLIT;
    const int s = bid / per_e;
    const int rem = bid - s * per_e;
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
    // token tiles: the smallest of 1, 2, 4, 8 covering what is left (capped)
    for (int t0 = 0; t0 < n;) {
        const int r = n - t0;
        if (TBMAX >= 8 && r > 4) {
            down_tile<Tr, (TBMAX >= 8 ? 8 : 1), TBMAX, MODE>(p, s_red, s_h, s_list, Wd, hb, n, off, t0, min(r, 8),
                                                             lo, hi, sp, cv, rowV, lane, wave);
            t0 += 8;
        } else if (TBMAX >= 4 && r > 2) {
            down_tile<Tr, (TBMAX >= 4 ? 4 : 1), TBMAX, MODE>(p, s_red, s_h, s_list, Wd, hb, n, off, t0, min(r, 4),
                                                             lo, hi, sp, cv, rowV, lane, wave);
            t0 += 4;
        } else if (TBMAX >= 2 && r > 1) {
            down_tile<Tr, (TBMAX >= 2 ? 2 : 1), TBMAX, MODE>(p, s_red, s_h, s_list, Wd, hb, n, off, t0, 2, lo, hi,
                                                             sp, cv, rowV, lane, wave);
            t0 += 2;
        } else {
            down_tile<Tr, 1, TBMAX, MODE>(p, s_red, s_h, s_list, Wd, hb, n, off, t0, 1, lo, hi, sp, cv, rowV, lane,
                                          wave);
            t0 += 1;
        }
    }
}

// (256 threads, at least 3 wavefronts per SIMD: 3 workgroups per CU)
template <class Tr, int TBMAX, int MODE>
__global__ __launch_bounds__(256, 3) void k_down(DownParams p)
{
    __shared__ DownLds<TBMAX, Tr::kEpl> D;
    down_gemv<Tr, TBMAX, MODE>(p, D, blockIdx.x);
}

// bf16 layers: one launch runs the GEMV down workgroups [0, gemv_blocks) and
// the MFMA down tiles (the rest; gemv_blocks is a multiple of 8).
template <int TBMAX, int MODE>
__global__ __launch_bounds__(256, 3) void k_down_bf16(DownParams p, MfmaParams mp, int gemv_blocks)
{
    __shared__ union {
        DownLds<TBMAX, BF16::kEpl> gemv;
        MfmaDownLds mfma;
    } S;
    if ((int)blockIdx.x < gemv_blocks) down_gemv<BF16, TBMAX, MODE>(p, S.gemv, blockIdx.x);
    else mfma_down_body<MODE>(mp, S.mfma, blockIdx.x - gemv_blocks, gridDim.x - gemv_blocks);
}

static int round8_down(long long v) { return (int)((v + 7) / 8 * 8); }

template <class Tr, int TB, int MODE>
static hipError_t launch_down_m(const Plan &pl, const DownParams &dp, const MfmaParams &mp, hipStream_t st)
{
    const size_t lds = MODE == MOE_DENSE ? 0 : (size_t)pl.Imax * sizeof(uint16_t);
    if constexpr (std::is_same<Tr, BF16>::value) {
        if (pl.use_mfma) {  // the merged kernel carries the MFMA tiles' LDS; only when they can exist
            const int gemv = round8_down((long long)pl.max_touched * pl.NCT * pl.NSPLIT);
            const int grid = gemv + round8_down((long long)pl.max_items * (pl.H / kTC));
            hipLaunchKernelGGL((k_down_bf16<TB, MODE>), dim3(grid), dim3(256), lds, st, dp, mp, gemv);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_down<Tr, TB, MODE>), dim3(pl.max_touched * pl.NCT * pl.NSPLIT), dim3(256), lds, st, dp);
    return hipGetLastError();
}

template <class Tr, int TB>
static hipError_t launch_down_t(const Plan &pl, const DownParams &dp, const MfmaParams &mp, int mode, hipStream_t st)
{
    if (mode == MOE_DENSE) return launch_down_m<Tr, TB, MOE_DENSE>(pl, dp, mp, st);
    return launch_down_m<Tr, TB, MOE_SPARSE>(pl, dp, mp, st);
}

template <class Tr>
static hipError_t launch_down_tr(const Plan &pl, const DownParams &dp, const MfmaParams &mp, int mode, hipStream_t st)
{
    switch (pl.TT) {
    case 1: return launch_down_t<Tr, 1>(pl, dp, mp, mode, st);
    case 2: return launch_down_t<Tr, 2>(pl, dp, mp, mode, st);
    case 4: return launch_down_t<Tr, 4>(pl, dp, mp, mode, st);
    case 8: return launch_down_t<Tr, 8>(pl, dp, mp, mode, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_down(const Plan &pl, const DownParams &dp, const MfmaParams &mp, int mode, hipStream_t st)
{
    if (pl.T <= 0) return hipSuccess;
    return pl.dtype == MOE_BF16 ? launch_down_tr<BF16>(pl, dp, mp, mode, st)
                                : launch_down_tr<F32>(pl, dp, mp, mode, st);
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
