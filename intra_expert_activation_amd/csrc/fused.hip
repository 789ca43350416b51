// One-launch decode path for small batches (single tokens, and up to
// kFusedMaxT tokens of layers with small experts).
//
// gist.science page of arXiv 2605.08575, Technical Summary, Methodology:
// the gate projection is dense, the threshold mask is one elementwise pass,
// and only the active neurons' up and down rows are fetched (Fused Up-Down).
// Here the whole chain runs inside one workgroup per (pair, 32-row chunk),
// with no grouping and no h round trip through memory:
//   route  every wavefront selects the pair's token's top K itself (each
//          workgroup of a token finds the same ids; the hidden states load
//          meanwhile), so the first gate rows wait on no barrier; the
//          weights are stored by one extra workgroup per token;
//   gate   the chunk's 32 gate rows, SiLU, threshold, mask word;
//   up     the active rows only -> h = a * u, kept in LDS;
//   down   the active rows' down weights, h-weighted, summed in registers
//          over the chunk -> one fp32 partial output row of H columns.
// A second launch (k_fcombine) adds each token's partial rows with the routing
// weights and builds the per-expert unions from the mask words.
//
// With one token per batch every expert serves exactly one pair, so the
// grouping and the separate down launch (its schedule and row lists are a
// chain of dependent memory round trips) cost more than they organise.  With a
// few tokens an expert chosen by several of them has its rows read once per
// pair, mostly from cache while those workgroups run together.  The partial
// rows add 4 * H bytes per 32 neuron rows and pair: 1/16 of the gate bytes,
// written and read once.
#include "gemv_rows.h"
#include "moe_internal.h"
#include "route.h"
#include "wave_reduce.h"

namespace moe {

template <int NW>
struct FusedLds {
    float part[NW][kChunk][1];  // per-wavefront partial dots (gate, then up)
    float a[kChunk];            // scores
    float h[kChunk];            // h of the active rows, by rank
    uint64_t sel[NW][kSelWords];  // each wavefront's top-K selection words
    uint32_t act;               // active rows of the chunk
};

// acc += h[rank] * (row of buf) for the batch's rows that exist (rank < nact);
// the extra rows repeat the last active row and are skipped.
template <class Tr, int UR, int NSW>
__device__ __forceinline__ void down_batch(const typename Tr::V (&buf)[UR][NSW], const float *sh, int rank0,
                                           int nact, float (&acc)[NSW][Tr::kEpl])
{
#pragma unroll
    for (int u = 0; u < UR; ++u) {
        const int rank = rank0 + u;
        const float hv = sh[rank < kChunk ? rank : kChunk - 1];
        if (rank < nact) {
#pragma unroll
            for (int k = 0; k < NSW; ++k) {
                float f[Tr::kEpl];
                Tr::unpack(buf[u][k], f);
#pragma unroll
                for (int i = 0; i < Tr::kEpl; ++i) acc[k][i] = fmaf(hv, f[i], acc[k][i]);
            }
        }
    }
}

// NT: nontemporal weight loads, for single-token batches (every expert then
// serves one pair, so no other workgroup reads its rows).
template <class Tr, int NW, int NSW, int MODE, bool NT>
__global__ __launch_bounds__(NW * 64) void k_fused(FusedParams p)
{
    using V = typename Tr::V;
    constexpr int epl = Tr::kEpl;
    // rows per batch: 8 vectors of weights per lane per batch, two batches in
    // flight (one token leaves the registers for twice the projection's
    // batches: the gate's 32 rows take two memory round trips instead of four)
    constexpr int UR = 8 / NSW < 1 ? 1 : 8 / NSW;
    constexpr int NB = kChunk / UR;
    static_assert(NB % 2 == 0, "ping-pong needs an even batch count");
    constexpr int rowV = NW * NSW * kWave;  // 16-byte vectors per row
    __shared__ FusedLds<NW> L;

    if ((int)blockIdx.x >= p.P * p.C) {  // the routing outputs of one token
        const int tt = blockIdx.x - p.P * p.C;
        if (threadIdx.x < kWave) {
            int id;
            float wt;
            route_token(p.logits, tt, p.E, p.K, p.renorm, L.sel[0], id, wt);
            if ((int)threadIdx.x < p.K) {
                p.ids[(size_t)tt * p.K + threadIdx.x] = id;
                p.w[(size_t)tt * p.K + threadIdx.x] = wt;
            }
        }
        return;
    }
    const int pair = blockIdx.x / p.C;
    const int c = blockIdx.x - pair * p.C;
    const int t = pair / p.slots;
    const int slot = pair - t * p.slots;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int vbase = wave * NSW * kWave + lane;  // this lane's first vector of a row

    // the token's hidden states (this wavefront's slice) do not wait for the routing
    V xr[1][NSW];
#pragma unroll
    for (int k = 0; k < NSW; ++k) xr[0][k] = reinterpret_cast<const V *>(p.x)[(size_t)t * rowV + vbase + k * kWave];

    int xe = p.E + slot - p.K;  // a shared expert, or else the routed one:
    if (slot < p.K) xe = __builtin_amdgcn_readlane(route_token_ids(p.logits, t, p.E, p.K, L.sel[wave]), slot);
    const bool shared = xe >= p.E;
    const int Ie = shared ? p.Is : p.I;
    const int r0 = c * kChunk;

    float acc[NSW][epl];
#pragma unroll
    for (int k = 0; k < NSW; ++k)
#pragma unroll
        for (int i = 0; i < epl; ++i) acc[k][i] = 0.f;
    uint32_t act = 0u;

    if (r0 < Ie) {  // chunks past a narrower expert's rows only store zeros
        const size_t mat = (size_t)(shared ? xe - p.E : xe) * Ie * rowV + (size_t)r0 * rowV + vbase;
        const V *Wg = reinterpret_cast<const V *>(shared ? p.swg : p.wg) + mat;
        const V *Wu = reinterpret_cast<const V *>(shared ? p.swu : p.wu) + mat;
        const V *Wd = reinterpret_cast<const V *>(shared ? p.swd : p.wd) + mat;
        const float tau = (MODE == MOE_SPARSE) ? p.tau[xe] : 0.f;
        const int kidx = xreduce_index<UR>(lane);
        const bool owner = xreduce_owner<UR>(lane);

        // ---- gate: 32 rows, two batches in flight, last two peeled -----------
        V bufA[UR][NSW], bufB[UR][NSW];
        load_rows<Tr, UR, NSW, NT>(bufA, Wg, 0, rowV);
        {
            int b = 0;
#pragma unroll 1
            for (; b + 2 < NB; b += 2) {
                load_rows<Tr, UR, NSW, NT>(bufB, Wg, (b + 1) * UR, rowV);
                __builtin_amdgcn_sched_barrier(0);
                reduce_batch<Tr, UR, NSW, 1, NW>(bufA, xr, L.part, wave, b * UR, lane, kidx, owner);
                __builtin_amdgcn_sched_barrier(0);
                load_rows<Tr, UR, NSW, NT>(bufA, Wg, (b + 2) * UR, rowV);
                __builtin_amdgcn_sched_barrier(0);
                reduce_batch<Tr, UR, NSW, 1, NW>(bufB, xr, L.part, wave, (b + 1) * UR, lane, kidx, owner);
                __builtin_amdgcn_sched_barrier(0);
            }
            load_rows<Tr, UR, NSW, NT>(bufB, Wg, (b + 1) * UR, rowV);
            __builtin_amdgcn_sched_barrier(0);
            reduce_batch<Tr, UR, NSW, 1, NW>(bufA, xr, L.part, wave, b * UR, lane, kidx, owner);
            reduce_batch<Tr, UR, NSW, 1, NW>(bufB, xr, L.part, wave, (b + 1) * UR, lane, kidx, owner);
        }
        __syncthreads();

        // ---- scores and the mask word ----------------------------------------
        if (wave == 0) {
            bool m = false;
            if (lane < kChunk) {
                float g = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) g += L.part[w][lane][0];
                const float a = silu(g);
                L.a[lane] = a;
                m = MODE == MOE_DENSE || !(fabsf(a) < tau);
            }
            const uint64_t bits = __ballot(m);
            if (lane == 0) L.act = (uint32_t)bits;
        }
        __syncthreads();
        act = __builtin_amdgcn_readfirstlane(L.act);
        const int nact = __popc(act);

        if (nact > 0) {
            const int last = 31 - __clz(act);
            const int nb = (nact + UR - 1) / UR;
            // ---- up: the active rows, ascending -------------------------------
            {
                uint32_t rest = act;
                load_active_rows<Tr, UR, NSW, NT>(bufA, Wu, rest, last, rowV);
                int b = 0;
#pragma unroll 1
                for (; b + 2 < nb; b += 2) {
                    load_active_rows<Tr, UR, NSW, NT>(bufB, Wu, rest, last, rowV);
                    __builtin_amdgcn_sched_barrier(0);
                    reduce_batch<Tr, UR, NSW, 1, NW>(bufA, xr, L.part, wave, b * UR, lane, kidx, owner);
                    __builtin_amdgcn_sched_barrier(0);
                    load_active_rows<Tr, UR, NSW, NT>(bufA, Wu, rest, last, rowV);
                    __builtin_amdgcn_sched_barrier(0);
                    reduce_batch<Tr, UR, NSW, 1, NW>(bufB, xr, L.part, wave, (b + 1) * UR, lane, kidx, owner);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (b + 1 < nb) {
                    load_active_rows<Tr, UR, NSW, NT>(bufB, Wu, rest, last, rowV);
                    __builtin_amdgcn_sched_barrier(0);
                    reduce_batch<Tr, UR, NSW, 1, NW>(bufA, xr, L.part, wave, b * UR, lane, kidx, owner);
                    reduce_batch<Tr, UR, NSW, 1, NW>(bufB, xr, L.part, wave, (b + 1) * UR, lane, kidx, owner);
                } else {
                    reduce_batch<Tr, UR, NSW, 1, NW>(bufA, xr, L.part, wave, b * UR, lane, kidx, owner);
                }
            }
            // the first down rows do not depend on h: issue them before the barrier
            uint32_t rest = act;
            load_active_rows<Tr, UR, NSW, NT>(bufA, Wd, rest, last, rowV);
            __syncthreads();
            if (wave == 0 && lane < kChunk && ((act >> lane) & 1u)) {
                const int rank = __popc(act & ((1u << lane) - 1u));
                float u = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) u += L.part[w][rank][0];
                L.h[rank] = L.a[lane] * u;  // every row of act is active for the pair's one token
            }
            __syncthreads();

            // ---- down: the same rows of w_down, h-weighted --------------------
            int b = 0;
#pragma unroll 1
            for (; b + 2 < nb; b += 2) {
                load_active_rows<Tr, UR, NSW, NT>(bufB, Wd, rest, last, rowV);
                __builtin_amdgcn_sched_barrier(0);
                down_batch<Tr, UR, NSW>(bufA, L.h, b * UR, nact, acc);
                __builtin_amdgcn_sched_barrier(0);
                load_active_rows<Tr, UR, NSW, NT>(bufA, Wd, rest, last, rowV);
                __builtin_amdgcn_sched_barrier(0);
                down_batch<Tr, UR, NSW>(bufB, L.h, (b + 1) * UR, nact, acc);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (b + 1 < nb) {
                load_active_rows<Tr, UR, NSW, NT>(bufB, Wd, rest, last, rowV);
                __builtin_amdgcn_sched_barrier(0);
                down_batch<Tr, UR, NSW>(bufA, L.h, b * UR, nact, acc);
                down_batch<Tr, UR, NSW>(bufB, L.h, (b + 1) * UR, nact, acc);
            } else {
                down_batch<Tr, UR, NSW>(bufA, L.h, b * UR, nact, acc);
            }
        }
    }

    // ---- the chunk's partial output row and mask word ------------------------
    float *dst = p.partial + ((size_t)pair * p.C + c) * p.H;
#pragma unroll
    for (int k = 0; k < NSW; ++k) {
        float4 *d4 = reinterpret_cast<float4 *>(dst + (size_t)(vbase + k * kWave) * epl);
#pragma unroll
        for (int q = 0; q < epl / 4; ++q)
            d4[q] = make_float4(acc[k][4 * q], acc[k][4 * q + 1], acc[k][4 * q + 2], acc[k][4 * q + 3]);
    }
    if (threadIdx.x == 0) {
        p.mw[(size_t)pair * p.W + c] = act;
        if (p.mask_bits) p.mask_bits[(size_t)pair * p.W + c] = act;
    }
}

// ---------------------------------------------------------------------------
// k_fcombine.  Workgroups [0, T * H / 64): y of one token over 64 columns.
// Its 16 thread groups take the token's partial rows (slot, chunk) in a fixed
// interleave, each adding w_slot * row (w = 1 for a shared expert), with the
// loads of 16 rows per thread in flight together (one memory round trip for up
// to 256 rows), and the group sums meet in LDS in a fixed order, so y is
// reproducible bit for bit.
// Workgroups after those (only when a union output is requested): one per
// expert, OR of its pairs' mask words, then the union size and the ascending
// list of its active neurons.  For one token (at most kFcSlots1 slots) the
// slot ids and every slot's mask words load together and the expert's slot is
// picked in registers.
// ---------------------------------------------------------------------------
constexpr int kFcCols = 64;
constexpr int kFcSlots1 = 16;  // single-token unions: slots whose mask words load at once

__global__ __launch_bounds__(256) void k_fcombine(FusedParams p)
{
    const int tid = threadIdx.x;
    const int tiles = p.H / kFcCols;
    const int nyb = p.T * tiles;
    if ((int)blockIdx.x < nyb) {
        __shared__ float4 s_acc[16][16];
        const int t = blockIdx.x / tiles;
        const int ct = blockIdx.x - t * tiles;
        const int q = tid & 15;  // float4 of the 64 columns
        const int g = tid >> 4;  // thread group
        const int col = ct * kFcCols + q * 4;
        const int R = p.slots * p.C;  // partial rows of the token, (slot, chunk) order
        const float *src = p.partial + (size_t)t * R * p.H + col;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        constexpr int kRows = 16;  // rows per thread whose loads are in flight together
        for (int i0 = g; i0 < R; i0 += 16 * kRows) {
            float4 v[kRows];
            float wv[kRows];
#pragma unroll
            for (int j = 0; j < kRows; ++j) {  // indices clamped, extras unused
                const int i = min(i0 + 16 * j, R - 1);
                const int slot = i / p.C;
                v[j] = *reinterpret_cast<const float4 *>(src + (size_t)i * p.H);
                const float ws = p.w[(size_t)t * p.K + min(slot, p.K - 1)];
                wv[j] = slot < p.K ? ws : 1.f;
            }
#pragma unroll
            for (int j = 0; j < kRows; ++j)
                if (i0 + 16 * j < R) {
                    acc.x = fmaf(wv[j], v[j].x, acc.x);
                    acc.y = fmaf(wv[j], v[j].y, acc.y);
                    acc.z = fmaf(wv[j], v[j].z, acc.z);
                    acc.w = fmaf(wv[j], v[j].w, acc.w);
                }
        }
        s_acc[g][q] = acc;
        __syncthreads();
        if (g == 0) {
            float4 r = s_acc[0][q];
#pragma unroll
            for (int gg = 1; gg < 16; ++gg) {
                r.x += s_acc[gg][q].x;
                r.y += s_acc[gg][q].y;
                r.z += s_acc[gg][q].z;
                r.w += s_acc[gg][q].w;
            }
            *reinterpret_cast<float4 *>(p.y + (size_t)t * p.H + col) = r;
        }
        return;
    }

    // ---- union of expert e -------------------------------------------------
    __shared__ int s_pairs[kFusedMaxT];  // a token has an expert in at most one slot
    __shared__ int s_np;
    __shared__ int s_wt[4];
    const int e = blockIdx.x - nyb;
    const int w0 = 2 * tid;  // words [w0, w0 + 2) of this thread (W <= 512)
    uint32_t u0 = 0u, u1 = 0u;
    if (p.T == 1 && p.slots <= kFcSlots1) {
        // one token: expert e is in at most one slot, and the mask words are
        // stored by slot, so every slot's words load with the ids (one round
        // trip instead of a search and then the words)
        uint32_t v0[kFcSlots1], v1[kFcSlots1];
        int sid[kFcSlots1];
#pragma unroll
        for (int j = 0; j < kFcSlots1; ++j) {
            v0[j] = v1[j] = 0u;
            sid[j] = -1;
            if (j < p.slots) {
                sid[j] = j < p.K ? p.ids[j] : p.E + (j - p.K);
                if (w0 < p.W) v0[j] = p.mw[(size_t)j * p.W + w0];
                if (w0 + 1 < p.W) v1[j] = p.mw[(size_t)j * p.W + w0 + 1];
            }
        }
#pragma unroll
        for (int j = 0; j < kFcSlots1; ++j)
            if (sid[j] == e) {
                u0 |= v0[j];
                u1 |= v1[j];
            }
    } else {
        if (tid == 0) s_np = 0;
        __syncthreads();
        if (e < p.E) {
            for (int a = tid; a < p.T * p.K; a += blockDim.x)
                if (p.ids[a] == e) {  // the OR below does not depend on the order
                    const int at = atomicAdd(&s_np, 1);
                    if (at < kFusedMaxT) s_pairs[at] = (a / p.K) * p.slots + a % p.K;
                }
        } else {
            for (int t = tid; t < p.T; t += blockDim.x) s_pairs[t] = t * p.slots + p.K + (e - p.E);
            if (tid == 0) s_np = p.T;
        }
        __syncthreads();
        const int np = min(s_np, kFusedMaxT);
        for (int j = 0; j < np; ++j) {
            const uint32_t *m = p.mw + (size_t)s_pairs[j] * p.W;
            if (w0 < p.W) u0 |= m[w0];
            if (w0 + 1 < p.W) u1 |= m[w0 + 1];
        }
    }
    const int cnt = __popc(u0) + __popc(u1);
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int incl = wave_incl_scan_dpp(cnt);
    if (lane == kWave - 1) s_wt[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        base += w < wave ? s_wt[w] : 0;
        total += s_wt[w];
    }
    if (p.union_cnt && tid == 0) p.union_cnt[e] = total;
    if (p.union_idx) {
        int pos = base + incl - cnt;
        int32_t *out = p.union_idx + (size_t)e * p.Imax;
        for (uint32_t b = u0; b; b &= b - 1) out[pos++] = w0 * 32 + __ffs(b) - 1;
        for (uint32_t b = u1; b; b &= b - 1) out[pos++] = (w0 + 1) * 32 + __ffs(b) - 1;
    }
}

// ---------------------------------------------------------------------------
template <class Tr, int NW, int NSW, bool NT>
static hipError_t launch_fused_nt(const Plan &pl, const FusedParams &fp, int mode, const KernelEvents &ev,
                                  hipStream_t st)
{
    const dim3 grid((unsigned)(pl.P * pl.C + pl.T));  // + one routing-store workgroup per token
    if (mode == MOE_DENSE)
        launch_timed(k_fused<Tr, NW, NSW, MOE_DENSE, NT>, grid, dim3(NW * kWave), st, ev.begin, ev.end, fp);
    else
        launch_timed(k_fused<Tr, NW, NSW, MOE_SPARSE, NT>, grid, dim3(NW * kWave), st, ev.begin, ev.end, fp);
    return hipGetLastError();
}

template <class Tr, int NW, int NSW>
static hipError_t launch_fused_ns(const Plan &pl, const FusedParams &fp, int mode, const KernelEvents &ev,
                                  hipStream_t st)
{
    return pl.T == 1 ? launch_fused_nt<Tr, NW, NSW, true>(pl, fp, mode, ev, st)
                     : launch_fused_nt<Tr, NW, NSW, false>(pl, fp, mode, ev, st);
}

template <class Tr>
static hipError_t launch_fused_tr(const Plan &pl, const FusedParams &fp, int mode, const KernelEvents &ev,
                                  hipStream_t st)
{
    switch (pl.NS) {  // as the expert projection: NS vectors per lane per row over up to 4 wavefronts
    case 1: return launch_fused_ns<Tr, 1, 1>(pl, fp, mode, ev, st);
    case 2: return launch_fused_ns<Tr, 2, 1>(pl, fp, mode, ev, st);
    case 4: return launch_fused_ns<Tr, 4, 1>(pl, fp, mode, ev, st);
    case 8: return launch_fused_ns<Tr, 4, 2>(pl, fp, mode, ev, st);
    case 16: return launch_fused_ns<Tr, 4, 4>(pl, fp, mode, ev, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fused(const Plan &pl, const FusedParams &fp, int mode, const KernelEvents *ev, hipStream_t st)
{
    if (pl.T <= 0) return hipSuccess;
    if (pl.T > kFusedMaxT || pl.C != pl.W || pl.H % kFcCols != 0) return hipErrorInvalidValue;
    const KernelEvents none{};
    const KernelEvents &e = ev ? *ev : none;
    hipError_t err = pl.dtype == MOE_BF16 ? launch_fused_tr<BF16>(pl, fp, mode, e, st)
                                          : launch_fused_tr<F32>(pl, fp, mode, e, st);
    if (err != hipSuccess) return err;
    const int unions = (fp.union_idx || fp.union_cnt) ? pl.EX : 0;
    hipLaunchKernelGGL(k_fcombine, dim3((unsigned)(pl.T * (pl.H / kFcCols) + unions)), dim3(256), 0, st, fp);
    return hipGetLastError();
}

}  // namespace moe
