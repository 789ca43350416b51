// Down projection over an expert's active neurons, and the top-K weighted
// combine.
//
// gist.science page of arXiv 2605.08575, Technical Summary, Methodology,
// "Fused Up-Down Projection": only active neurons' weights are gathered.  With
// the down matrix stored neuron-major, an active neuron is one contiguous row
// of H elements and an inactive one is never read.
//
// k_down (GEMV experts, n_e below the MFMA threshold) accumulates
//     o[pair, cols] += h[row][pair] * w_down[row][cols]
// over the union rows of each expert.  The work is a sequence of groups, one
// per (touched expert, token tile of up to 8 of its pairs, 1024-column tile),
// each as long as the expert's union; the sequence is cut into equal
// contiguous shares of at most kDownChunk rows, one per workgroup (workgroup
// g takes shares g, g + GD, ...; its 4 wavefronts stream the same rows, 256
// columns each).  So an expert with a large union (or many pairs) is spread
// over several workgroups instead of setting the kernel's length, and the
// workgroups never wait for one another.  A group cut into pieces leaves one
// partial sum per piece (at most KMAX); the combine kernel adds the pieces
// and the K slots in a fixed order, so no floating-point atomics are used and
// the result is bitwise reproducible.  Every workgroup derives the same
// schedule from the per-slot union sizes.  Outputs are indexed by (token,
// slot): piece k of pair (t, slot) is row t * slots + slot of partial slice
// k, and the last piece of a group stores the group's piece count for the
// combine.
#include <atomic>
#include <type_traits>

#include "mfma_body.h"
#include "moe_internal.h"
#include "wave_reduce.h"

namespace moe {

constexpr int kDownTok = 8;      // pairs per token tile (one pass over the rows each)
constexpr int kMinShare = 32;    // smallest share of a workgroup (union rows)

// A wavefront's lanes own 4 consecutive columns each (8-byte vectors of bf16,
// 16-byte vectors of fp32), so a wavefront covers 256 columns and the 4
// wavefronts of a workgroup cover 1024 adjacent columns (2 KB of a bf16 row)
// and stream the same rows; the groups of an expert's column tiles are
// adjacent in the schedule, so the rest of each row is read at about the same
// time by the neighbouring workgroups.  Reading a row's pieces together keeps
// the DRAM pages open: reading the 512-byte pieces of a row at different times
// measured 4.7-5.9 TB/s against 6.0-6.4 TB/s for whole rows.
constexpr int kDownCols = 4 * kWave * 4;  // columns per workgroup column tile

struct DownBF16 {
    using V = uint2;
    static constexpr int kEpl = 4;
    static __device__ __forceinline__ void unpack(V w, float (&f)[4]) {
        f[0] = __uint_as_float(w.x << 16);
        f[1] = __uint_as_float(w.x & 0xffff0000u);
        f[2] = __uint_as_float(w.y << 16);
        f[3] = __uint_as_float(w.y & 0xffff0000u);
    }
};
template <class Tr> struct DownVec { using type = F32; };
template <> struct DownVec<BF16> { using type = DownBF16; };

// Orders a wavefront's LDS writes before its own later LDS reads (no
// workgroup barrier: the list regions are wave-private).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// Writes the neuron indices at positions [a, b) of an expert's ascending union
// list (the set bits of its nw union words; bit i of word w = neuron 32 w + i)
// to list[0 .. b - a).  Lane l holds words l, l + 64, ...; the neurons are
// visited 64 at a time (lane i takes neuron 64 kb + i), and a ballot with a
// masked popcount gives each set bit its position, so the list comes out in
// ascending order without a per-bit loop.  A prefix sum of the words'
// popcounts finds the word holding position a, so the visit starts there
// (not at word 0) and stops once position b is reached.
constexpr int kMaxWordsPerLane = kMaxRows / 32 / kWave;  // 8

// The ballot walk over word pairs [2 kk0, ...) of one register of words,
// starting at union position base; returns the position after the walk.
__device__ __forceinline__ int union_walk(uint32_t words, int wbase, int nw, int kk0, int base, int a, int b,
                                          uint16_t *list, int lane, uint64_t below)
{
    for (int kk = kk0; kk < kWave / 2; ++kk) {
        const int w0 = wbase + 2 * kk;  // the block's first word
        if (w0 >= nw || base >= b) break;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)words, 2 * kk);
        const uint32_t hi = w0 + 1 < nw ? (uint32_t)__builtin_amdgcn_readlane((int)words, 2 * kk + 1) : 0u;
        const bool bit = (((lane < 32) ? lo : hi) >> (lane & 31)) & 1u;
        const uint64_t m = __ballot(bit);
        const int pos = base + __popcll(m & below);
        if (bit && pos >= a && pos < b) list[pos - a] = (uint16_t)(w0 * 32 + lane);
        base += __popcll(m);
    }
    return base;
}

// The same for nw <= 64 with lane l's word already loaded (0 past nw).
__device__ __forceinline__ void wave_union_list_1(uint32_t word, int nw, int a, int b, uint16_t *list, int lane)
{
    const int c = __popc(word);
    const int ex = wave_incl_scan_dpp(c) - c;  // set bits before this word
    // the last word whose prefix is <= a holds position a (a < b <= total)
    const uint64_t le = __ballot(lane < nw && ex <= a);
    const int w0 = 63 - __clzll((long long)le);
    const int kk0 = w0 >> 1;
    const int base = __builtin_amdgcn_readlane(ex, 2 * kk0);
    union_walk(word, 0, nw, kk0, base, a, b, list, lane, lanemask_lt());
    wave_lds_sync();
}

__device__ __forceinline__ void wave_union_list(const uint32_t *uw, int nw, int a, int b, uint16_t *list,
                                                int lane)
{
    uint32_t words[kMaxWordsPerLane];
    int ex[kMaxWordsPerLane];
#pragma unroll
    for (int r = 0; r < kMaxWordsPerLane; ++r) words[r] = (r * kWave + lane < nw) ? uw[r * kWave + lane] : 0u;
    int run = 0;
#pragma unroll
    for (int r = 0; r < kMaxWordsPerLane; ++r) {
        const int c = __popc(words[r]);
        const int incl = wave_incl_scan_dpp(c);
        ex[r] = run + incl - c;
        run += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    const uint64_t below = lanemask_lt();
    int base = -1;  // set when the walk has started
#pragma unroll
    for (int r = 0; r < kMaxWordsPerLane; ++r) {
        if (r * kWave >= nw) break;
        int kk0 = 0;
        if (base < 0) {
            // does position a lie in this register's words (or before the next's)?
            const uint64_t le = __ballot(r * kWave + lane < nw && ex[r] <= a);
            const int nr = min(kWave, nw - r * kWave);  // words in this register
            if (le == 0) continue;  // (cannot happen for r = 0)
            const int wl = 63 - __clzll((long long)le);
            const bool later = r + 1 < kMaxWordsPerLane && (r + 1) * kWave < nw &&
                               __builtin_amdgcn_readfirstlane(ex[r + 1 < kMaxWordsPerLane ? r + 1 : r]) <= a;
            if (wl == nr - 1 && later) continue;  // a lies in a later register's words
            kk0 = wl >> 1;
            base = __builtin_amdgcn_readlane(ex[r], 2 * kk0);
        }
        if (base >= b) break;
        base = union_walk(words[r], r * kWave, nw, kk0, base, a, b, list, lane, below);
    }
    wave_lds_sync();
}

// One batch of UR rows of a wavefront's list: this lane's vector of each down
// row, and h[row][token] of the batch spread over NH registers (entry
// u * TB + t in lane (u * TB + t) % 64 of register (u * TB + t) / 64), so the
// h values travel with the weights they scale.
template <class Tr, int TB, int UR>
struct DownBatch {
    static constexpr int NH = (UR * TB + kWave - 1) / kWave;
    typename Tr::V w[UR];
    float h[NH];    // as loaded; zeroed at use where hok is false
    bool hok[NH];
};

template <class Tr, int TB, int UR, int MODE>
__device__ __forceinline__ void down_issue(DownBatch<Tr, TB, UR> &bt, const typename Tr::V *Wd, int rowV,
                                           const float *hb, int n, int t0, int nt, const uint16_t *list, int a,
                                           int L, int i0, int lane)
{
    constexpr int NH = DownBatch<Tr, TB, UR>::NH;
    // Every load is unconditional, from an in-bounds address: entries past L
    // re-read the list's last row (L >= 1 here) and tokens past nt the last
    // valid token.  Their h is zeroed, so such a row adds h * w = 0 (weights
    // are finite); the weights themselves are not masked, since the compiler
    // would turn that select into a branch around the load, and a load under a
    // branch makes it wait for every load in flight where the paths join.
    // h first: it is consumed first, so waiting for it leaves the batch's
    // weight loads in flight.  Its zeroing happens at use (selecting here would
    // wait for the load).
#pragma unroll
    for (int q = 0; q < NH; ++q) {
        const int e = q * kWave + lane;
        const int ih = i0 + e / TB, t = e % TB;
        const int ihc = min(ih, L - 1);
        const int jh = (MODE == MOE_DENSE) ? a + ihc : (int)list[ihc];
        bt.h[q] = hb[(size_t)jh * n + t0 + min(t, nt - 1)];
        bt.hok[q] = e < UR * TB && ih < L && t < nt;
    }
    const int iw = min(i0 + (lane & (UR - 1)), L - 1);
    const int jw = (MODE == MOE_DENSE) ? a + iw : (int)list[iw];
    // Wd is the wavefront-uniform start of the column tile: row j's vectors
    // are Wd + j * rowV + lane
#pragma unroll
    for (int u = 0; u < UR; ++u) {
        const int j = __builtin_amdgcn_readlane(jw, u);
        bt.w[u] = load_stream(Wd + (size_t)j * rowV + lane);  // read once per call: nontemporal
    }
}

// acc[t][:] += h[row][t] * w[row][:] over the batch's rows; h is broadcast
// from its lane by v_readlane (UR * TB <= 64: one register).
template <class Tr, int TB, int UR>
__device__ __forceinline__ void down_fma(const DownBatch<Tr, TB, UR> &bt, float (&acc)[TB][Tr::kEpl])
{
    static_assert(UR * TB <= kWave, "one register of h per batch");
    const float h = bt.hok[0] ? bt.h[0] : 0.f;
#pragma unroll
    for (int u = 0; u < UR; ++u) {
        float wf[Tr::kEpl];
        Tr::unpack(bt.w[u], wf);
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const float hs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), u * TB + t));
#pragma unroll
            for (int c = 0; c < Tr::kEpl; ++c) acc[t][c] = fmaf(hs, wf[c], acc[t][c]);
        }
    }
}

// Streams the wavefront's L list rows into acc: batches of UR rows, two in
// flight.  The steady-state loop always issues the next batch before
// consuming the current one (no conditional loads inside, so each wait is for
// exactly one batch); the last one or two batches are peeled.  The scheduling
// barriers keep each batch's loads ahead of the other batch's arithmetic (left
// alone, the scheduler sinks the loads below it to shorten live ranges).
template <class Tr, int TB, int MODE>
__device__ __forceinline__ void down_stream(const typename Tr::V *Wd, int rowV, const float *hb, int n, int t0,
                                            int nt, const uint16_t *list, int a, int L, float (&acc)[TB][Tr::kEpl],
                                            int lane)
{
    // rows per batch: 16 registers of weights per batch (two batches in
    // flight) and one register of h
    constexpr int UR = sizeof(typename Tr::V) < 16 ? 8 : 4;
    static_assert(UR * TB <= kWave, "one register of h per batch");
    const int nb = (L + UR - 1) / UR;
    if (nb == 0) return;
    DownBatch<Tr, TB, UR> A, B;
    down_issue<Tr, TB, UR, MODE>(A, Wd, rowV, hb, n, t0, nt, list, a, L, 0, lane);
    int k = 0;
#pragma unroll 1
    for (; k + 2 < nb; k += 2) {
        down_issue<Tr, TB, UR, MODE>(B, Wd, rowV, hb, n, t0, nt, list, a, L, (k + 1) * UR, lane);
        __builtin_amdgcn_sched_barrier(0);
        down_fma<Tr, TB, UR>(A, acc);
        __builtin_amdgcn_sched_barrier(0);
        down_issue<Tr, TB, UR, MODE>(A, Wd, rowV, hb, n, t0, nt, list, a, L, (k + 2) * UR, lane);
        __builtin_amdgcn_sched_barrier(0);
        down_fma<Tr, TB, UR>(B, acc);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (k + 1 < nb) {
        down_issue<Tr, TB, UR, MODE>(B, Wd, rowV, hb, n, t0, nt, list, a, L, (k + 1) * UR, lane);
        __builtin_amdgcn_sched_barrier(0);
        down_fma<Tr, TB, UR>(A, acc);
        down_fma<Tr, TB, UR>(B, acc);
    } else {
        down_fma<Tr, TB, UR>(A, acc);
    }
}

constexpr int kMaxPieces = 16;  // pieces listed before streaming starts

struct DownPiece {
    int s, tile, ctg, a, b, k, lofs, pad;
};

struct DownLds {
    int start[kMaxExperts];   // exclusive prefix of the work over touched slots
    int uc[kMaxExperts];      // union size per touched slot (0: not on this path)
    int xe[kMaxExperts];      // expert of each touched slot
    int n[kMaxExperts];       // its pair count
    int off[kMaxExperts];     // its first grouped pair
    int wsum[4], wmax[4];
    uint16_t list[4][kDownChunk];             // per wavefront: the pieces' rows
    DownPiece piece[4][kMaxPieces];           // per wavefront: the pieces
};

// One piece: union positions [a, b) (at most kDownChunk) of expert xe, token
// tile `tile`, workgroup column tile ctg, whose rows are list[0 .. b - a).  The
// wavefront streams its 256 columns of each row and writes them to partial
// piece k.
template <class Tr, int TB, int MODE>
__device__ __forceinline__ void down_piece(const DownParams &p, const uint16_t *list, int xe, int n, int off,
                                           int tile, int ctg, int a, int b, int k, bool last, int lane, int wave)
{
    using V = typename Tr::V;
    constexpr int EPL = Tr::kEpl;                    // 4 columns per lane
    const int rowV = p.H / EPL;                      // vectors per row
    const int v0 = ctg * (kDownCols / EPL) + wave * kWave;  // this wavefront's first vector
    if (v0 >= rowV) return;                          // narrow layers: no columns here
    const bool shared = xe >= p.E;
    const int Ie = shared ? p.Is : p.I;
    const int t0 = tile * kDownTok;
    const int nt = min(n - t0, kDownTok);
    const size_t mat = (size_t)(shared ? xe - p.E : xe) * Ie * rowV;
    const V *Wd = reinterpret_cast<const V *>(shared ? p.swd : p.wd) + mat + v0;
    const float *hb = p.h + (shared ? (size_t)p.A * p.I + (size_t)(off - p.A) * Ie : (size_t)off * Ie);
    // lane t < nt: the output row (t * slots + slot) of the tile's pair t
    const int pr = off + t0 + min(lane, nt - 1);
    const int orow = p.pair_tok[pr] * p.slots + p.pair_slot[pr];

    float acc[TB][EPL];
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int c = 0; c < EPL; ++c) acc[t][c] = 0.f;
    down_stream<Tr, TB, MODE>(Wd, rowV, hb, n, t0, nt, list, a, b - a, acc, lane);

    // piece 0 at the pair's (token, slot) row, later pieces at its compact row
    const int prow = k == 0 ? orow : p.P + (k - 1) * p.G + p.cidx[orow];
    float *dst = p.partial + (size_t)(v0 + lane) * EPL;
#pragma unroll
    for (int t = 0; t < TB; ++t)
        if (t < nt) {
            const int r = __builtin_amdgcn_readlane(prow, t);
#pragma unroll
            for (int c = 0; c < EPL; c += 4)
                *reinterpret_cast<float4 *>(dst + (size_t)r * p.H + c) =
                    make_float4(acc[t][c], acc[t][c + 1], acc[t][c + 2], acc[t][c + 3]);
        }
    // the group's last piece records how many pieces it has
    if (last && wave == 0 && lane < nt) p.npc[(size_t)orow * p.NCT + ctg] = k + 1;
}

// Block-wide exclusive scan of v (one value per thread), with the total and
// the maximum of m over the workgroup.
__device__ __forceinline__ int block_excl_scan(DownLds &D, int v, int m, int &total, int &mx, int lane, int wave)
{
    const int incl = wave_incl_scan(v, lane);
    int wm = m;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) wm = max(wm, __shfl_xor(wm, d, kWave));
    if (lane == kWave - 1) D.wsum[wave] = incl;
    if (lane == 0) D.wmax[wave] = wm;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wave; ++i) base += D.wsum[i];
    total = D.wsum[0] + D.wsum[1] + D.wsum[2] + D.wsum[3];
    mx = max(max(D.wmax[0], D.wmax[1]), max(D.wmax[2], D.wmax[3]));
    __syncthreads();
    return base + incl - v;
}

// The GEMV down projection of workgroup g (of p.GD).
template <class Tr, int MODE>
__device__ __forceinline__ void down_gemv(const DownParams &p, DownLds &D, int g)
{
    using DV = typename DownVec<Tr>::type;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wavefront
    const int EX = p.E + p.S;
    const int ntouched = p.hdr[0];

    // ---- schedule: work per touched slot = union size x token tiles ---------
    // thread i covers slots 2i and 2i + 1 (E + S <= 512)
    int wl[2], ul[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int s = 2 * threadIdx.x + r;
        wl[r] = ul[r] = 0;
        // slot-ordered experts, pair counts, offsets and union sizes: one round
        // of independent loads, issued with the load of the touched count (the
        // index is clamped into the arrays; slots past the count are not used)
        const int sc = min(s, EX - 1);
        const int xe = p.touched[sc];
        const int n = p.slot_n[sc];
        const int of = p.slot_off[sc];
        const int uc = MODE == MOE_DENSE ? 0 : p.ucount[sc];
        if (s < ntouched) {
            const int Iw = xe >= p.E ? p.Is : p.I;
            D.xe[s] = xe;
            D.n[s] = n;
            D.off[s] = of;
            if (n < p.nm) {
                const int U = (MODE == MOE_DENSE) ? Iw : uc;
                ul[r] = U;
                wl[r] = U * ((n + kDownTok - 1) / kDownTok);
                if (g == 0) {
                    if (p.union_cnt) p.union_cnt[xe] = U;
                    // no active row: no piece, the pairs' outputs are zero
                    if (U == 0)
                        for (int i = 0; i < n; ++i) {
                            const int orow = p.pair_tok[of + i] * p.slots + p.pair_slot[of + i];
                            for (int c = 0; c < p.NCT; ++c) p.npc[(size_t)orow * p.NCT + c] = 0;
                        }
                }
            }
        }
    }
    int total, umax;
    const int ex = block_excl_scan(D, wl[0] + wl[1], max(ul[0], ul[1]), total, umax, lane, wave);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int s = 2 * threadIdx.x + r;
        D.start[s] = ex + (r ? wl[0] : 0);
        D.uc[s] = ul[r];
    }
    const long long wtot = (long long)p.NCT * total;
    // GD workgroup shares of at most kDownChunk rows (one list build per
    // piece), none below kMinShare, and no group cut into more than KMAX
    // pieces (KMAX - 1 >= Imax / kDownChunk keeps that bound under kDownChunk)
    long long share = (wtot + p.GD - 1) / p.GD;
    share = max(share, (long long)kMinShare);
    share = min(share, (long long)kDownChunk);
    share = max(share, (long long)((umax + p.KMAX - 2) / (p.KMAX - 1)));
    __syncthreads();

    // ---- workgroup shares vg = g + j GD: [vg share, (vg + 1) share) ---------
    // Each round lists up to kMaxPieces pieces (from LDS only), loads all their
    // union words at once and builds their row lists before any weight is
    // streamed (and before any store: a load consumed after a store waits for
    // the store to complete), then streams them.
    uint16_t *list = D.list[wave];
    DownPiece *pc = D.piece[wave];
    const int nwmax = p.Imax / 32;
    for (long long vg = g; vg * share < wtot; vg += p.GD) {
        long long pos = vg * share;
        const long long end = min(pos + share, wtot);
        while (pos < end) {
            int np = 0, lofs = 0;
            while (pos < end && np < kMaxPieces) {
                // the last slot whose range starts at or before pos (slots with
                // no work start where the next one does, so they are skipped)
                int lo = 0, hi = ntouched;  // invariant: NCT * start[lo] <= pos
                while (hi - lo > 1) {
                    const int mid = (lo + hi) / 2;
                    if ((long long)p.NCT * D.start[mid] <= pos) lo = mid;
                    else hi = mid;
                }
                const int s = lo;
                const int U = D.uc[s];
                const long long sbase = (long long)p.NCT * D.start[s];
                const int gi = (int)((pos - sbase) / U);  // group within the slot: tile * NCT + ctg
                const int tile = gi / p.NCT, ctg = gi - tile * p.NCT;
                const long long gstart = sbase + (long long)gi * U;
                const int a = (int)(pos - gstart);
                const int b = (int)(min(end, gstart + U) - gstart);
                if (lane == 0) pc[np] = DownPiece{s, tile, ctg, a, b, (int)(vg - gstart / share), lofs, 0};
                ++np;
                lofs += b - a;
                pos = gstart + b;
            }
            wave_lds_sync();
            if (MODE != MOE_DENSE) {
                if (nwmax <= kWave) {
                    // one union word per lane: every piece's words in flight at once
                    uint32_t wv[kMaxPieces];
#pragma unroll
                    for (int j = 0; j < kMaxPieces; ++j) {
                        wv[j] = 0u;
                        if (j < np) {
                            const int xe = __builtin_amdgcn_readfirstlane(D.xe[pc[j].s]);
                            const int nw = (xe >= p.E ? p.Is : p.I) / 32;
                            if (lane < nw) wv[j] = p.union_words[(size_t)xe * p.W + lane];
                        }
                    }
#pragma unroll
                    for (int j = 0; j < kMaxPieces; ++j)
                        if (j < np) {
                            const int xe = __builtin_amdgcn_readfirstlane(D.xe[pc[j].s]);
                            const int nw = (xe >= p.E ? p.Is : p.I) / 32;
                            wave_union_list_1(wv[j], nw, __builtin_amdgcn_readfirstlane(pc[j].a),
                                              __builtin_amdgcn_readfirstlane(pc[j].b),
                                              list + __builtin_amdgcn_readfirstlane(pc[j].lofs), lane);
                        }
                } else {
                    for (int j = 0; j < np; ++j) {
                        const int xe = __builtin_amdgcn_readfirstlane(D.xe[pc[j].s]);
                        const int nw = (xe >= p.E ? p.Is : p.I) / 32;
                        wave_union_list(p.union_words + (size_t)xe * p.W, nw, __builtin_amdgcn_readfirstlane(pc[j].a),
                                        __builtin_amdgcn_readfirstlane(pc[j].b),
                                        list + __builtin_amdgcn_readfirstlane(pc[j].lofs), lane);
                    }
                }
            }
            for (int j = 0; j < np; ++j) {
                // uniform piece fields (LDS values are not known to be uniform)
                const int s = __builtin_amdgcn_readfirstlane(pc[j].s);
                const int xe = __builtin_amdgcn_readfirstlane(D.xe[s]);
                const int n = __builtin_amdgcn_readfirstlane(D.n[s]);
                const int of = __builtin_amdgcn_readfirstlane(D.off[s]);
                const int tile = __builtin_amdgcn_readfirstlane(pc[j].tile);
                const int ctg = __builtin_amdgcn_readfirstlane(pc[j].ctg);
                const int a = __builtin_amdgcn_readfirstlane(pc[j].a);
                const int b = __builtin_amdgcn_readfirstlane(pc[j].b);
                const int k = __builtin_amdgcn_readfirstlane(pc[j].k);
                const int lo = __builtin_amdgcn_readfirstlane(pc[j].lofs);
                const bool last = b == __builtin_amdgcn_readfirstlane(D.uc[s]);
                const int nt = min(n - tile * kDownTok, kDownTok);
                if (nt > 4) down_piece<DV, 8, MODE>(p, list + lo, xe, n, of, tile, ctg, a, b, k, last, lane, wave);
                else if (nt > 2) down_piece<DV, 4, MODE>(p, list + lo, xe, n, of, tile, ctg, a, b, k, last, lane, wave);
                else if (nt > 1) down_piece<DV, 2, MODE>(p, list + lo, xe, n, of, tile, ctg, a, b, k, last, lane, wave);
                else down_piece<DV, 1, MODE>(p, list + lo, xe, n, of, tile, ctg, a, b, k, last, lane, wave);
            }
            // the union list output, after the round's streaming
            if (wave == 0 && p.union_idx)
                for (int j = 0; j < np; ++j) {
                    if (__builtin_amdgcn_readfirstlane(pc[j].tile) != 0 || __builtin_amdgcn_readfirstlane(pc[j].ctg) != 0) continue;
                    const int xe = __builtin_amdgcn_readfirstlane(D.xe[pc[j].s]);
                    const int a = __builtin_amdgcn_readfirstlane(pc[j].a);
                    const int b = __builtin_amdgcn_readfirstlane(pc[j].b);
                    const int lo = __builtin_amdgcn_readfirstlane(pc[j].lofs);
                    for (int i = lane; i < b - a; i += kWave)
                        p.union_idx[(size_t)xe * p.Imax + a + i] = (MODE == MOE_DENSE) ? a + i : (int)list[lo + i];
                }
            wave_lds_sync();  // the next round rewrites the lists and pieces
        }
    }
}

// (256 threads, at least 3 wavefronts per SIMD; the launcher sizes GD to the
// workgroups the device holds at once)
template <class Tr, int MODE>
__global__ __launch_bounds__(256, 3) void k_down(DownParams p)
{
    __shared__ DownLds D;
    down_gemv<Tr, MODE>(p, D, blockIdx.x);
}

// bf16 layers: one launch runs the GEMV down workgroups [0, GD) and the MFMA
// down tiles (the rest; GD is a multiple of 8).
template <int MODE>
__global__ __launch_bounds__(256, 3) void k_down_bf16(DownParams p, MfmaParams mp)
{
    __shared__ union {
        DownLds gemv;
        MfmaDownLds mfma;
    } S;
    if ((int)blockIdx.x < p.GD) down_gemv<BF16, MODE>(p, S.gemv, blockIdx.x);
    else mfma_down_body<MODE>(mp, S.mfma, blockIdx.x - p.GD);
}

static int round8_down(long long v) { return (int)((v + 7) / 8 * 8); }

// Workgroups of kernel KF (256 threads) the current device holds at once.
// The query is cached per kernel and device; calls from several host threads
// may race to fill an entry, which is harmless because every thread computes
// the same value and the entry is read and written atomically.
template <auto KF>
static int resident_blocks()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KF, 256, 0) != hipSuccess || per_cu < 1) per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    const int r = per_cu * cus;
    if (dev < 64) cache[dev].store(r, std::memory_order_relaxed);
    return r;
}

// GEMV down workgroups: the plan's bound, at most what is resident at once,
// a multiple of 8 (the MFMA tiles after them keep their XCD order)
static int down_groups(const Plan &pl, int resident)
{
    int gd = pl.GD < resident ? pl.GD : resident;
    gd = gd / 8 * 8;
    return gd < 8 ? 8 : gd;
}

template <class Tr, int MODE>
static hipError_t launch_down_m(const Plan &pl, const DownParams &dp_in, const MfmaParams &mp, hipStream_t st)
{
    DownParams dp = dp_in;
    if constexpr (std::is_same<Tr, BF16>::value) {
        if (pl.use_mfma) {  // the merged kernel carries the MFMA tiles' LDS; only when they can exist
            dp.GD = down_groups(pl, resident_blocks<k_down_bf16<MODE>>());
            const int grid = dp.GD + round8_down((long long)pl.max_items * (pl.H / kTC) * pl.NKS);
            hipLaunchKernelGGL((k_down_bf16<MODE>), dim3(grid), dim3(256), 0, st, dp, mp);
            return hipGetLastError();
        }
    }
    dp.GD = down_groups(pl, resident_blocks<k_down<Tr, MODE>>());
    hipLaunchKernelGGL((k_down<Tr, MODE>), dim3(dp.GD), dim3(256), 0, st, dp);
    return hipGetLastError();
}

template <class Tr>
static hipError_t launch_down_tr(const Plan &pl, const DownParams &dp, const MfmaParams &mp, int mode, hipStream_t st)
{
    if (mode == MOE_DENSE) return launch_down_m<Tr, MOE_DENSE>(pl, dp, mp, st);
    return launch_down_m<Tr, MOE_SPARSE>(pl, dp, mp, st);
}

hipError_t launch_down(const Plan &pl, const DownParams &dp, const MfmaParams &mp, int mode, hipStream_t st)
{
    if (pl.T <= 0) return hipSuccess;
    return pl.dtype == MOE_BF16 ? launch_down_tr<BF16>(pl, dp, mp, mode, st)
                                : launch_down_tr<F32>(pl, dp, mp, mode, st);
}

// ---------------------------------------------------------------------------
// k_combine: y[t] = sum_{k<K} w[t,k] * o[t,k] + sum_{s<S} o[t,K+s].
// o of a GEMV expert's pair is the sum, in piece order, of the partial sums of
// the pieces its group (token tile, column tile) was cut into (npc of them:
// piece 0 at the pair's (token, slot) row, the others at its compact row);
// an MFMA expert's pair has one piece per segment of its neuron tiles (piece 0
// as above, the others by (token, slot) row after the GEMV pieces).  A
// workgroup covers one token and one 256-column tile: 64 column quads x 4 thread groups; group g adds the slots k with k % 4 == g,
// and the 4 group sums meet in LDS in a fixed order (so the result is
// deterministic).
// ---------------------------------------------------------------------------
// NB: slots per thread group whose loads are issued together (1, 2 or 4).
// Each slot's weight, piece count, compact row and first piece depend on
// (t, slot) alone, so a batch needs one memory latency for those.  PF: pieces
// per slot whose loads are issued together; the next PF - 1 pieces of every
// slot of the batch then take one more latency (a load past the slot's piece
// count repeats its first piece's address and is not added), and any further
// pieces one each.  Pieces are added in piece order, so the sum is the same for
// every PF.
// Row of piece k >= 1 of the pair at (token, slot) row orow: a GEMV expert's
// pair at its compact row crow, an MFMA expert's pair (crow -1) by segment.
__device__ __forceinline__ size_t piece_row(const CombineParams &p, int k, int crow, int orow)
{
    return crow >= 0 ? (size_t)p.P + (size_t)(k - 1) * p.G + crow : p.mbase + (size_t)(k - 1) * p.P + orow;
}

template <int NB, int PF>
__device__ __forceinline__ void combine_body(const CombineParams &p, float4 (&s_acc)[3][64])
{
    const int t = blockIdx.x;
    const int ct = blockIdx.y;
    const int q = threadIdx.x & 63;  // column quad within the tile
    const int g = threadIdx.x >> 6;  // slot group
    const int c4 = ct * 64 + q;
    const int ctg = c4 / (kDownCols / 4);  // the down kernel's column tile of these columns
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = g; k0 < p.slots; k0 += 4 * NB) {
        int np[NB], crow[NB], orow[NB];
        float wk[NB];
        float4 o[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int k = min(k0 + 4 * j, p.slots - 1);
            orow[j] = t * p.slots + k;
            const float rw = p.topk_w[(size_t)t * p.K + min(k, p.K - 1)];
            wk[j] = (k < p.K) ? rw : 1.f;
            np[j] = p.npc[(size_t)orow[j] * p.NCT + ctg];
            crow[j] = p.cidx[orow[j]];  // -1 for an MFMA expert's pair
            o[j] = reinterpret_cast<const float4 *>(p.partial + (size_t)orow[j] * p.H)[c4];
        }
        float4 ex[NB][PF > 1 ? PF - 1 : 1];
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int kk = 1; kk < PF; ++kk) {
                const size_t row = kk < np[j] ? piece_row(p, kk, crow[j], orow[j]) : (size_t)orow[j];
                ex[j][kk - 1] = reinterpret_cast<const float4 *>(p.partial + row * p.H)[c4];
            }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if (k0 + 4 * j >= p.slots) break;
            float4 v = np[j] > 0 ? o[j] : make_float4(0.f, 0.f, 0.f, 0.f);  // no piece: o = 0
#pragma unroll
            for (int kk = 1; kk < PF; ++kk)
                if (kk < np[j]) {
                    v.x += ex[j][kk - 1].x;
                    v.y += ex[j][kk - 1].y;
                    v.z += ex[j][kk - 1].z;
                    v.w += ex[j][kk - 1].w;
                }
            for (int kk = PF > 1 ? PF : 1; kk < np[j]; ++kk) {
                const float4 w = reinterpret_cast<const float4 *>(p.partial + piece_row(p, kk, crow[j], orow[j]) * p.H)[c4];
                v.x += w.x;
                v.y += w.y;
                v.z += w.z;
                v.w += w.w;
            }
            y.x = fmaf(wk[j], v.x, y.x);
            y.y = fmaf(wk[j], v.y, y.y);
            y.z = fmaf(wk[j], v.z, y.z);
            y.w = fmaf(wk[j], v.w, y.w);
        }
    }
    if (g > 0) s_acc[g - 1][q] = y;
    __syncthreads();
    if (g == 0) {
        const float4 a = s_acc[0][q], b = s_acc[1][q], c = s_acc[2][q];
        y.x = (y.x + a.x) + (b.x + c.x);
        y.y = (y.y + a.y) + (b.y + c.y);
        y.z = (y.z + a.z) + (b.z + c.z);
        y.w = (y.w + a.w) + (b.w + c.w);
        reinterpret_cast<float4 *>(p.y + (size_t)t * p.H)[c4] = y;
    }
}

template <int PF>
__global__ __launch_bounds__(256) void k_combine(CombineParams p)
{
    __shared__ float4 s_acc[3][64];
    if (p.slots <= 4) combine_body<1, PF>(p, s_acc);
    else if (p.slots <= 8) combine_body<2, PF>(p, s_acc);
    else combine_body<4, PF>(p, s_acc);
}

// Small grids (decode batches) issue 6 pieces of a slot together; large grids
// (prefill, where most slots have one piece) keep the registers for occupancy.
constexpr int kCombPrefetchMaxBlocks = 2048;

hipError_t launch_combine(const Plan &pl, const CombineParams &cp, hipStream_t st)
{
    if (pl.T <= 0) return hipSuccess;
    const dim3 grid((unsigned)pl.T, (unsigned)(pl.H / 256));
    if ((long long)pl.T * (pl.H / 256) <= kCombPrefetchMaxBlocks)
        hipLaunchKernelGGL(k_combine<6>, grid, dim3(256), 0, st, cp);
    else
        hipLaunchKernelGGL(k_combine<1>, grid, dim3(256), 0, st, cp);
    return hipGetLastError();
}

}  // namespace moe
