// Expert projection: dense gate GEMV, SiLU score, threshold mask, wavefront
// ballot of the active neurons, and the up projection of the active rows only.
//
// gist.science page of arXiv 2605.08575, Technical Summary, Methodology:
//   Gate Projection    every gate row of a selected expert is read (dense);
//   Activation Masking one elementwise threshold pass over the scores;
//   Fused Up-Down      only active neurons' up rows are fetched.
// The down projection of the active rows is the next kernel (down.hip).
//
// Work decomposition.  One workgroup (4 wavefronts) owns R consecutive neuron
// rows of one touched expert and loops over that expert's tokens in register
// tiles of TT tokens.  A lane owns a fixed set of columns of every row
// (NS 16-byte vectors, 64 lanes interleaved), so its slice of each token's
// hidden state is loaded once per tile and kept in registers while rows
// stream through.  Row dot products are finished with a wavefront reduction.
//   phase G  all R gate rows: g, a = SiLU(g), m = NOT(|a| < tau); a goes to LDS,
//            m to LDS bit words (the mask), their OR over the tile's tokens to
//            the tile's active-row words;
//   phase U  the active rows only: u = x . w_up, h = m ? a*u : 0.
// h is written to a per-expert block [rows][n_e] (n_e = the expert's pairs);
// rows inactive for the whole tile get h = 0 without touching w_up.  Every
// workgroup owns whole 32-bit mask words (R is a multiple of 32), so masks and
// the per-expert union are written without atomics.
#include "moe_internal.h"

namespace moe {

template <class Tr, int NS, int TT, int MODE>
__global__ __launch_bounds__(256) void k_proj(ProjParams p)
{
    using V = typename Tr::V;
    constexpr int UR = (16 / NS) > 8 ? 8 : ((16 / NS) < 1 ? 1 : (16 / NS));  // rows in flight per wavefront
    constexpr int kWords = kMaxRowsPerChunk / 32;

    __shared__ float s_a[TT][kMaxRowsPerChunk];
    __shared__ uint32_t s_mask[TT][kWords];
    __shared__ uint32_t s_act[kWords];
    __shared__ uint32_t s_union[kWords];
    __shared__ int s_list[kMaxRowsPerChunk];
    __shared__ int s_nact;

    const int s = blockIdx.x / p.C;
    const int c = blockIdx.x - s * p.C;
    if (s >= p.hdr[0]) return;
    const int xe = p.touched[s];
    const bool shared = xe >= p.E;
    const int Ie = shared ? p.Is : p.I;
    const int r0 = c * p.R;
    if (r0 >= Ie) return;
    const int nr = min(p.R, Ie - r0);  // multiple of 32
    const int n = p.counts[xe];
    const int off = p.offsets[xe];
    const int rowV = NS * kWave;       // 16-byte vectors per row (= H / epl)
    const size_t mat = (size_t)(shared ? xe - p.E : xe) * Ie * rowV;
    const V *Wg = reinterpret_cast<const V *>(shared ? p.swg : p.wg) + mat;
    const V *Wu = reinterpret_cast<const V *>(shared ? p.swu : p.wu) + mat;
    const V *X = reinterpret_cast<const V *>(p.x);
    float *hb = p.h + (shared ? (size_t)p.A * p.I + (size_t)(off - p.A) * Ie : (size_t)off * Ie);
    const float tau = (MODE == MOE_SPARSE) ? p.tau[xe] : 0.f;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwords = nr / 32;

    if (threadIdx.x < kWords) s_union[threadIdx.x] = 0u;

    for (int t0 = 0; t0 < n; t0 += TT) {
        const int nt = min(TT, n - t0);
        __syncthreads();  // LDS of the previous tile is no longer read
        if (threadIdx.x < TT * kWords) (&s_mask[0][0])[threadIdx.x] = 0u;
        if (threadIdx.x < kWords) s_act[threadIdx.x] = 0u;

        // this lane's columns of the tile's hidden states
        V xr[TT][NS];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const int tok = (t < nt) ? p.pair_tok[off + t0 + t] : -1;
#pragma unroll
            for (int v = 0; v < NS; ++v)
                xr[t][v] = (tok >= 0) ? X[(size_t)tok * rowV + v * kWave + lane] : Tr::zero();
        }
        __syncthreads();

        // ---- phase G: gate rows r = wave + 4 i -------------------------------
        for (int rb = wave; rb < nr; rb += 4 * UR) {
            V wv[UR][NS];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int r = rb + 4 * u;
#pragma unroll
                for (int v = 0; v < NS; ++v)
                    wv[u][v] = (r < nr) ? Wg[(size_t)(r0 + r) * rowV + v * kWave + lane] : Tr::zero();
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int r = rb + 4 * u;
                if (r >= nr) break;
                float g[TT];
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    float acc = 0.f;
#pragma unroll
                    for (int v = 0; v < NS; ++v) acc = Tr::dot(wv[u][v], xr[t][v], acc);
                    g[t] = wave_sum(acc);
                }
                if (MODE == kModeScore) {
#pragma unroll
                    for (int t = 0; t < TT; ++t)
                        if (lane == t && t < nt) hb[(size_t)(r0 + r) * n + t0 + t] = fabsf(silu(g[t]));
                } else {
                    uint32_t mb = 0;
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        const float a = silu(g[t]);
                        const bool m = (t < nt) && (MODE == MOE_DENSE || !(fabsf(a) < tau));
                        mb |= (m ? 1u : 0u) << t;
                        if (lane == t) s_a[t][r] = a;
                    }
                    if (lane < TT && ((mb >> lane) & 1u)) atomicOr(&s_mask[lane][r >> 5], 1u << (r & 31));
                    if (lane == 0 && mb) atomicOr(&s_act[r >> 5], 1u << (r & 31));
                }
            }
        }
        if (MODE == kModeScore) continue;
        __syncthreads();

        // ---- compact the tile's active rows (ascending) ----------------------
        if (wave == 0) {
            int base = 0;
            for (int r = lane; r < ((nr + kWave - 1) / kWave) * kWave; r += kWave) {
                const bool act = (r < nr) && ((s_act[r >> 5] >> (r & 31)) & 1u);
                const uint64_t b = __ballot(act);
                if (act) s_list[base + __popcll(b & lanemask_lt())] = r;
                base += __popcll(b);
            }
            if (lane == 0) s_nact = base;
        }
        // rows inactive for every token of the tile: h = 0, w_up not read
        for (int i = threadIdx.x; i < nr * nt; i += blockDim.x) {
            const int r = i / nt, t = i - r * nt;
            if (!((s_act[r >> 5] >> (r & 31)) & 1u)) hb[(size_t)(r0 + r) * n + t0 + t] = 0.f;
        }
        __syncthreads();
        const int nact = s_nact;

        // ---- phase U: up rows of the active neurons only ---------------------
        for (int ib = wave; ib < nact; ib += 4 * UR) {
            V wv[UR][NS];
            int rr[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int i = ib + 4 * u;
                rr[u] = (i < nact) ? s_list[i] : -1;
#pragma unroll
                for (int v = 0; v < NS; ++v)
                    wv[u][v] = (rr[u] >= 0) ? Wu[(size_t)(r0 + rr[u]) * rowV + v * kWave + lane] : Tr::zero();
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int r = rr[u];
                if (r < 0) break;
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    float acc = 0.f;
#pragma unroll
                    for (int v = 0; v < NS; ++v) acc = Tr::dot(wv[u][v], xr[t][v], acc);
                    const float uu = wave_sum(acc);
                    if (lane == t && t < nt) {
                        const bool m = (s_mask[t][r >> 5] >> (r & 31)) & 1u;
                        // a select, not a multiply: an inactive neuron contributes exactly 0
                        hb[(size_t)(r0 + r) * n + t0 + t] = m ? s_a[t][r] * uu : 0.f;
                    }
                }
            }
        }

        // ---- masks of the tile's (token, slot) rows, and the union ---------
        if (p.mask_bits) {
            for (int i = threadIdx.x; i < nt * nwords; i += blockDim.x) {
                const int t = i / nwords, wd = i - t * nwords;
                const int pr = off + t0 + t;
                const size_t row = (size_t)p.pair_tok[pr] * p.slots + p.pair_slot[pr];
                p.mask_bits[row * p.W + (r0 >> 5) + wd] = s_mask[t][wd];
            }
            // words past this expert's last row (experts narrower than Imax)
            const int wtail = p.W - Ie / 32;
            if (c == 0 && wtail > 0) {
                for (int i = threadIdx.x; i < nt * wtail; i += blockDim.x) {
                    const int t = i / wtail, wd = Ie / 32 + (i - t * wtail);
                    const int pr = off + t0 + t;
                    const size_t row = (size_t)p.pair_tok[pr] * p.slots + p.pair_slot[pr];
                    p.mask_bits[row * p.W + wd] = 0u;
                }
            }
        }
        if (threadIdx.x < nwords) s_union[threadIdx.x] |= s_act[threadIdx.x];
    }
    if (MODE == kModeScore) return;
    __syncthreads();
    if (threadIdx.x < nwords) p.union_words[(size_t)xe * p.W + (r0 >> 5) + threadIdx.x] = s_union[threadIdx.x];
}

// ---------------------------------------------------------------------------
template <class Tr, int NS, int TT>
static hipError_t launch_proj_t(const Plan &pl, const ProjParams &pp, int mode, hipStream_t st)
{
    const dim3 grid(pl.max_touched * pl.C), block(256);
    if (mode == MOE_SPARSE) hipLaunchKernelGGL((k_proj<Tr, NS, TT, MOE_SPARSE>), grid, block, 0, st, pp);
    else if (mode == MOE_DENSE) hipLaunchKernelGGL((k_proj<Tr, NS, TT, MOE_DENSE>), grid, block, 0, st, pp);
    else hipLaunchKernelGGL((k_proj<Tr, NS, TT, kModeScore>), grid, block, 0, st, pp);
    return hipGetLastError();
}

template <class Tr, int NS>
static hipError_t launch_proj_ns(const Plan &pl, const ProjParams &pp, int mode, hipStream_t st)
{
    // the register tile holds TT * NS vectors of x; keep it at <= 32
    switch (pl.TT) {
    case 1: return launch_proj_t<Tr, NS, 1>(pl, pp, mode, st);
    case 2: if constexpr (NS <= 16) return launch_proj_t<Tr, NS, 2>(pl, pp, mode, st); break;
    case 4: if constexpr (NS <= 8) return launch_proj_t<Tr, NS, 4>(pl, pp, mode, st); break;
    case 8: if constexpr (NS <= 4) return launch_proj_t<Tr, NS, 8>(pl, pp, mode, st); break;
    }
    return hipErrorInvalidValue;
}

template <class Tr>
static hipError_t launch_proj_tr(const Plan &pl, const ProjParams &pp, int mode, hipStream_t st)
{
    switch (pl.NS) {
    case 1: return launch_proj_ns<Tr, 1>(pl, pp, mode, st);
    case 2: return launch_proj_ns<Tr, 2>(pl, pp, mode, st);
    case 4: return launch_proj_ns<Tr, 4>(pl, pp, mode, st);
    case 8: return launch_proj_ns<Tr, 8>(pl, pp, mode, st);
    case 16: return launch_proj_ns<Tr, 16>(pl, pp, mode, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_proj(const Plan &pl, const ProjParams &pp, int mode, hipStream_t st)
{
    if (pl.T <= 0) return hipSuccess;
    return pl.dtype == MOE_BF16 ? launch_proj_tr<BF16>(pl, pp, mode, st)
                                : launch_proj_tr<F32>(pl, pp, mode, st);
}

}  // namespace moe
