// Expert projection: dense gate GEMV, SiLU score, threshold mask, ballot of
// the active neurons, and the up projection of the active rows only.
//
// gist.science page of arXiv 2605.08575, Technical Summary, Methodology:
//   Gate Projection    every gate row of a selected expert is read (dense);
//   Activation Masking one elementwise threshold pass over the scores;
//   Fused Up-Down      only active neurons' up rows are fetched.
// The down projection of the active rows is the next kernel (down.hip).
//
// Work decomposition (gfx950).  A workgroup owns 32 consecutive neuron rows of
// one touched expert -- one 32-bit mask word -- and every token of that
// expert, in tiles of TT tokens.  Its NW wavefronts split each row's columns
// (K-split): wavefront w reads the w-th 1/NW of every row (NSW 16-byte vectors
// per lane, contiguous 1 KB blocks), so it keeps only its slice of the token
// tile's hidden states in registers.  Rows stream in batches of UR with the
// next batch's loads issued before the current batch is reduced (software
// pipelining), and the UR x TT partial dot products of a batch are summed
// across the 64 lanes by one transposed reduction (wave_reduce.h).  The NW
// partials of each (row, token) meet in LDS and are added in a fixed order.
//   gate  all 32 rows -> g, a = SiLU(g), m = NOT(|a| < tau), mask word per
//         token, active-row word (OR over the tile's tokens);
//   up    the active rows only -> u, h = m ? a*u : 0 (a select: an inactive
//         neuron contributes exactly 0).
// h goes to a per-expert block [rows][n_e]; rows inactive for every token of
// the tile get h = 0 without reading w_up.  Mask words and the per-expert
// union word are written whole, without atomics; only the union sizes are
// summed, by integer atomics (order-independent).
#include <type_traits>

#include "gemv_rows.h"
#include "mfma_body.h"
#include "moe_internal.h"
#include "wave_reduce.h"

namespace moe {

// Gate and up rows with nontemporal loads: each row is read by one workgroup.
// An expert's second token tile re-reads them, but keeping the weight stream
// out of the caches measured faster overall (the rest of the call finds its
// data there).
constexpr bool kProjStream = true;

// LDS of one workgroup, sized for the largest token tile.
template <int NW, int TTMAX>
struct ProjLds {
    float part[NW][kChunk][TTMAX];  // per-wavefront partial dots
    float a[kChunk][TTMAX];         // scores of the tile
    uint32_t mask[TTMAX];           // mask word per token of the tile
    uint32_t act;                   // rows active for some token of the tile
};

// One token tile of TT tokens (nt <= TT valid): gate, scores, masks, up, h.
// Returns the tile's active-row word.
template <class Tr, int NW, int NSW, int TT, int TTMAX, int MODE>
__device__ __forceinline__ uint32_t proj_tile(const ProjParams &p, ProjLds<NW, TTMAX> &L,
                                              const typename Tr::V *X, const typename Tr::V *Wg,
                                              const typename Tr::V *Wu, float *hb, int n, int off, int t0,
                                              int nt, int r0, int c, int Ie, float tau, int lane, int wave)
{
    using V = typename Tr::V;
    // rows per batch: at most 32 partial sums per reduction and 4 vectors of
    // weights per lane per batch (two batches are in flight)
    constexpr int UR_T = 32 / TT < 1 ? 1 : 32 / TT;
    constexpr int UR_V = 4 / NSW < 1 ? 1 : 4 / NSW;
    constexpr int UR = UR_T < UR_V ? UR_T : UR_V;
    constexpr int M = UR * TT;        // values per reduction
    constexpr int NB = kChunk / UR;   // batches per 32 rows (even)
    static_assert(NB % 2 == 0, "ping-pong needs an even batch count");
    constexpr int rowV = NW * NSW * kWave;
    auto &s_part = *reinterpret_cast<float(*)[NW][kChunk][TT]>(&L.part);  // TT-wide view
    const int kidx = xreduce_index<M>(lane);
    const bool owner = xreduce_owner<M>(lane);

    // Two batches in flight (ping-pong).  The steady-state loops always issue
    // the next batch before reducing the current one, with no conditional
    // load inside (a load under a branch makes the compiler wait for every
    // load in flight where the paths join); the last batches are peeled.  The
    // scheduling barriers keep each batch's loads ahead of the other batch's
    // arithmetic.
    V bufA[UR][NSW], bufB[UR][NSW];
    if constexpr (MODE != kModeMasked)
        load_rows<Tr, UR, NSW, kProjStream>(bufA, Wg, 0, rowV);  // weights first: they do not wait for the tokens

    // this wavefront's slice of the tile's hidden states
    V xr[TT][NSW];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const int tok = p.pair_tok[off + t0 + min(t, nt - 1)];  // past nt: a valid token, dots unused
#pragma unroll
        for (int k = 0; k < NSW; ++k) xr[t][k] = X[(size_t)tok * rowV + k * kWave];
    }
    if (threadIdx.x < TT) L.mask[threadIdx.x] = 0u;
    if (threadIdx.x == 0) L.act = 0u;

    // ---- gate: 32 rows in NB batches -----------------------------------------
    if constexpr (MODE != kModeMasked) {
        int b = 0;
#pragma unroll 1
        for (; b + 2 < NB; b += 2) {
            load_rows<Tr, UR, NSW, kProjStream>(bufB, Wg, (b + 1) * UR, rowV);
            __builtin_amdgcn_sched_barrier(0);
            reduce_batch<Tr, UR, NSW, TT, NW>(bufA, xr, s_part, wave, b * UR, lane, kidx, owner);
            __builtin_amdgcn_sched_barrier(0);
            load_rows<Tr, UR, NSW, kProjStream>(bufA, Wg, (b + 2) * UR, rowV);
            __builtin_amdgcn_sched_barrier(0);
            reduce_batch<Tr, UR, NSW, TT, NW>(bufB, xr, s_part, wave, (b + 1) * UR, lane, kidx, owner);
            __builtin_amdgcn_sched_barrier(0);
        }
        load_rows<Tr, UR, NSW, kProjStream>(bufB, Wg, (b + 1) * UR, rowV);
        __builtin_amdgcn_sched_barrier(0);
        reduce_batch<Tr, UR, NSW, TT, NW>(bufA, xr, s_part, wave, b * UR, lane, kidx, owner);
        reduce_batch<Tr, UR, NSW, TT, NW>(bufB, xr, s_part, wave, (b + 1) * UR, lane, kidx, owner);
    }
    __syncthreads();

    // ---- scores, masks, active rows -----------------------------------------
    for (int i = threadIdx.x; i < kChunk * TT; i += NW * kWave) {
        const int r = i / TT, t = i - r * TT;
        if constexpr (MODE == kModeMasked) {  // the scores and masks of an earlier pass
            if (t < nt) {
                L.a[r][t] = hb[(size_t)r * n + t0 + t];
                if ((p.pmask[(size_t)(off + t0 + t) * p.W + (r0 >> 5)] >> r) & 1u) {
                    atomicOr(&L.mask[t], 1u << r);
                    atomicOr(&L.act, 1u << r);
                }
            }
            continue;
        }
        float g = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) g += s_part[w][r][t];
        const float a = silu(g);
        if (MODE == kModeScore) {
            if (t < nt) hb[(size_t)r * n + t0 + t] = a;  // signed: |a| is the score
        } else {
            L.a[r][t] = a;
            const bool m = (t < nt) && (MODE == MOE_DENSE || !(fabsf(a) < tau));
            if (m) {
                atomicOr(&L.mask[t], 1u << r);
                atomicOr(&L.act, 1u << r);
            }
        }
    }
    __syncthreads();
    if (MODE == kModeScore) return 0u;
    const uint32_t act = __builtin_amdgcn_readfirstlane(L.act);
    const int nact = __popc(act);

    // ---- up: active rows only, in ascending order ----------------------------
    if (nact > 0) {
        const int nbu = (nact + UR - 1) / UR;
        const int last = 31 - __clz(act);
        uint32_t rest = act;  // rows not yet issued (scalar)
        load_active_rows<Tr, UR, NSW, kProjStream>(bufA, Wu, rest, last, rowV);
        int b = 0;
#pragma unroll 1
        for (; b + 2 < nbu; b += 2) {
            load_active_rows<Tr, UR, NSW, kProjStream>(bufB, Wu, rest, last, rowV);
            __builtin_amdgcn_sched_barrier(0);
            reduce_batch<Tr, UR, NSW, TT, NW>(bufA, xr, s_part, wave, b * UR, lane, kidx, owner);
            __builtin_amdgcn_sched_barrier(0);
            load_active_rows<Tr, UR, NSW, kProjStream>(bufA, Wu, rest, last, rowV);
            __builtin_amdgcn_sched_barrier(0);
            reduce_batch<Tr, UR, NSW, TT, NW>(bufB, xr, s_part, wave, (b + 1) * UR, lane, kidx, owner);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (b + 1 < nbu) {
            load_active_rows<Tr, UR, NSW, kProjStream>(bufB, Wu, rest, last, rowV);
            __builtin_amdgcn_sched_barrier(0);
            reduce_batch<Tr, UR, NSW, TT, NW>(bufA, xr, s_part, wave, b * UR, lane, kidx, owner);
            reduce_batch<Tr, UR, NSW, TT, NW>(bufB, xr, s_part, wave, (b + 1) * UR, lane, kidx, owner);
        } else {
            reduce_batch<Tr, UR, NSW, TT, NW>(bufA, xr, s_part, wave, b * UR, lane, kidx, owner);
        }
    }
    __syncthreads();

    // ---- h for every row of the tile, masks ----------------------------------
    for (int i = threadIdx.x; i < kChunk * nt; i += NW * kWave) {
        const int r = i / nt, t = i - r * nt;
        float hv = 0.f;
        if ((act >> r) & 1u) {
            const int slot = __popc(act & ((1u << r) - 1u));  // rank among active rows
            float u = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) u += s_part[w][slot][t];
            const bool m = (L.mask[t] >> r) & 1u;
            hv = m ? L.a[r][t] * u : 0.f;
        }
        hb[(size_t)r * n + t0 + t] = hv;
    }
    if (p.mask_bits && threadIdx.x < nt) {
        const int t = threadIdx.x;
        const int pr = off + t0 + t;
        const size_t row = (size_t)p.pair_tok[pr] * p.slots + p.pair_slot[pr];
        p.mask_bits[row * p.W + (r0 >> 5)] = L.mask[t];
        if (c == 0)
            for (int wd = Ie / 32; wd < p.W; ++wd) p.mask_bits[row * p.W + wd] = 0u;
    }
    __syncthreads();  // LDS is rewritten by the next tile
    return act;
}

// The GEMV projection of workgroup `bid`: one 32-row chunk of one expert.
template <class Tr, int NW, int NSW, int TTMAX, int MODE>
__device__ __forceinline__ void proj_gemv(const ProjParams &p, ProjLds<NW, TTMAX> &L, int bid)
{
    using V = typename Tr::V;
    const int r = bid / p.C;  // rank of the expert in the longest-first order
    const int c = bid - r * p.C;
    // r < max_touched <= E + S: the entry is in bounds, and it is read together
    // with the count of touched experts (ranks past it hold stale entries)
    const int ntouched = p.hdr[0];
    const int4 ord = reinterpret_cast<const int4 *>(p.order)[r];
    if (r >= ntouched) return;
    const int s = ord.x >> 16;  // touched slot
    const int xe = ord.x & 0xffff;
    const bool shared = xe >= p.E;
    const int Ie = shared ? p.Is : p.I;
    const int r0 = c * kChunk;
    if (r0 >= Ie) return;
    const int n = ord.y;
    if (n >= p.nm) return;  // this expert takes the MFMA path
    const int off = ord.z;
    constexpr int rowV = NW * NSW * kWave;  // 16-byte vectors per row (H / epl)
    const size_t mat = (size_t)(shared ? xe - p.E : xe) * Ie * rowV;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int vbase = wave * NSW * kWave + lane;  // this lane's first vector of a row
    const V *Wg = reinterpret_cast<const V *>(shared ? p.swg : p.wg) + mat + (size_t)r0 * rowV + vbase;
    const V *Wu = reinterpret_cast<const V *>(shared ? p.swu : p.wu) + mat + (size_t)r0 * rowV + vbase;
    const V *X = reinterpret_cast<const V *>(p.x) + vbase;
    float *hb = p.h + (shared ? (size_t)p.A * p.I + (size_t)(off - p.A) * Ie : (size_t)off * Ie)
                + (size_t)r0 * n;
    const float tau = (MODE == MOE_SPARSE) ? p.tau[xe] : 0.f;

    // token tiles: the smallest of 1, 2, 4, 8 covering what is left (capped at
    // TTMAX), so an expert's rows are streamed once whenever n <= TTMAX
    uint32_t uni = 0;
    for (int t0 = 0; t0 < n;) {
        const int rem = n - t0;
        if (TTMAX >= 8 && rem > 4) {
            uni |= proj_tile<Tr, NW, NSW, (TTMAX >= 8 ? 8 : 1), TTMAX, MODE>(
                p, L, X, Wg, Wu, hb, n, off, t0, min(rem, 8), r0, c, Ie, tau, lane, wave);
            t0 += 8;
        } else if (TTMAX >= 4 && rem > 2) {
            uni |= proj_tile<Tr, NW, NSW, (TTMAX >= 4 ? 4 : 1), TTMAX, MODE>(
                p, L, X, Wg, Wu, hb, n, off, t0, min(rem, 4), r0, c, Ie, tau, lane, wave);
            t0 += 4;
        } else if (TTMAX >= 2 && rem > 1) {
            uni |= proj_tile<Tr, NW, NSW, (TTMAX >= 2 ? 2 : 1), TTMAX, MODE>(
                p, L, X, Wg, Wu, hb, n, off, t0, 2, r0, c, Ie, tau, lane, wave);
            t0 += 2;
        } else {
            uni |= proj_tile<Tr, NW, NSW, 1, TTMAX, MODE>(p, L, X, Wg, Wu, hb, n, off, t0, 1, r0, c, Ie, tau,
                                                          lane, wave);
            t0 += 1;
        }
    }
    if (MODE != kModeScore && threadIdx.x == 0) {
        p.union_words[(size_t)xe * p.W + (r0 >> 5)] = uni;
        atomicAdd(&p.ucount[s], __popc(uni));  // by touched slot; integer: order-independent
    }
}

template <class Tr, int NW, int NSW, int TTMAX, int MODE>
__global__ __launch_bounds__(NW * 64) void k_proj(ProjParams p)
{
    __shared__ ProjLds<NW, TTMAX> L;
    proj_gemv<Tr, NW, NSW, TTMAX, MODE>(p, L, blockIdx.x);
}

// bf16 layers with 256-thread GEMV workgroups: one launch runs the MFMA tiles
// (workgroups [0, mfma_blocks)) and the GEMV chunks (the rest).  The MFMA
// tiles come first so that their arithmetic overlaps the GEMV chunks' weight
// streaming instead of trailing it; mfma_blocks is a multiple of 8, so they
// keep their XCD order.
template <int NSW, int TTMAX, int MODE>
__global__ __launch_bounds__(256, 3) void k_proj_bf16(ProjParams p, MfmaParams mp, int mfma_blocks)
{
    __shared__ union {
        ProjLds<4, TTMAX> gemv;
        MfmaProjLds mfma;
    } S;
    if ((int)blockIdx.x >= mfma_blocks) {
        proj_gemv<BF16, 4, NSW, TTMAX, MODE>(p, S.gemv, blockIdx.x - mfma_blocks);
    } else {
        if constexpr (MODE == MOE_SPARSE || MODE == MOE_DENSE) mfma_proj_body<MODE>(mp, S.mfma, blockIdx.x);
    }
}

// ---------------------------------------------------------------------------
static int round8(long long v) { return (int)((v + 7) / 8 * 8); }

template <class Tr, int NW, int NSW, int TT, int MODE>
static hipError_t launch_proj_m(const Plan &pl, const ProjParams &pp, const MfmaParams &mp, hipStream_t st,
                                const KernelEvents &ev)
{
    const bool mfma = (MODE == MOE_SPARSE || MODE == MOE_DENSE) && pl.use_mfma;
    // one 16-byte vector per lane per row only: with more, the merged kernel's
    // GEMV body does not fit 3 workgroups per CU, and the MFMA tiles get a
    // launch of their own
    if constexpr (std::is_same<Tr, BF16>::value && NW == 4 && NSW == 1) {
        if (mfma) {  // the merged kernel carries the MFMA tiles' LDS; only when they can exist
            const int mfma_blocks = round8((long long)pl.max_pairs * pl.NT);
            const int grid = mfma_blocks + pl.max_touched * pl.C;
            launch_timed(k_proj_bf16<NSW, TT, MODE>, dim3(grid), dim3(256), st, ev.begin, ev.end, pp, mp,
                         mfma_blocks);
            return hipGetLastError();
        }
    }
    {
        // with a second (MFMA) launch, the stop event goes with that one
        launch_timed(k_proj<Tr, NW, NSW, TT, MODE>, dim3(pl.max_touched * pl.C), dim3(NW * kWave), st, ev.begin,
                     mfma ? nullptr : ev.end, pp);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || !mfma) return e;
        return launch_proj_mfma(pl, mp, MODE, st, nullptr, ev.end);
    }
}

template <class Tr, int NW, int NSW, int TT>
static hipError_t launch_proj_t(const Plan &pl, const ProjParams &pp, const MfmaParams &mp, int mode, hipStream_t st,
                                const KernelEvents &ev)
{
    if (mode == MOE_SPARSE) return launch_proj_m<Tr, NW, NSW, TT, MOE_SPARSE>(pl, pp, mp, st, ev);
    if (mode == MOE_DENSE) return launch_proj_m<Tr, NW, NSW, TT, MOE_DENSE>(pl, pp, mp, st, ev);
    if (mode == kModeMasked) return launch_proj_m<Tr, NW, NSW, TT, kModeMasked>(pl, pp, mp, st, ev);
    return launch_proj_m<Tr, NW, NSW, TT, kModeScore>(pl, pp, mp, st, ev);
}

template <class Tr, int NW, int NSW>
static hipError_t launch_proj_ns(const Plan &pl, const ProjParams &pp, const MfmaParams &mp, int mode, hipStream_t st,
                                 const KernelEvents &ev)
{
    switch (pl.TT) {  // the largest token tile
    case 1: return launch_proj_t<Tr, NW, NSW, 1>(pl, pp, mp, mode, st, ev);
    case 2: return launch_proj_t<Tr, NW, NSW, 2>(pl, pp, mp, mode, st, ev);
    case 4: return launch_proj_t<Tr, NW, NSW, 4>(pl, pp, mp, mode, st, ev);
    case 8: if constexpr (NSW <= 2) return launch_proj_t<Tr, NW, NSW, 8>(pl, pp, mp, mode, st, ev); break;
    }
    return hipErrorInvalidValue;
}

template <class Tr>
static hipError_t launch_proj_tr(const Plan &pl, const ProjParams &pp, const MfmaParams &mp, int mode, hipStream_t st,
                                 const KernelEvents &ev)
{
    // NS 16-byte vectors per lane per row, split over up to 4 wavefronts
    switch (pl.NS) {
    case 1: return launch_proj_ns<Tr, 1, 1>(pl, pp, mp, mode, st, ev);
    case 2: return launch_proj_ns<Tr, 2, 1>(pl, pp, mp, mode, st, ev);
    case 4: return launch_proj_ns<Tr, 4, 1>(pl, pp, mp, mode, st, ev);
    case 8: return launch_proj_ns<Tr, 4, 2>(pl, pp, mp, mode, st, ev);
    case 16: return launch_proj_ns<Tr, 4, 4>(pl, pp, mp, mode, st, ev);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_proj(const Plan &pl, const ProjParams &pp, const MfmaParams &mp, int mode, hipStream_t st,
                       const KernelEvents *ev)
{
    if (pl.T <= 0) return hipSuccess;
    const KernelEvents none{};
    const KernelEvents &e = ev ? *ev : none;
    return pl.dtype == MOE_BF16 ? launch_proj_tr<BF16>(pl, pp, mp, mode, st, e)
                                : launch_proj_tr<F32>(pl, pp, mp, mode, st, e);
}

}  // namespace moe
