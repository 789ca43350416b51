// Routing (softmax + top-K) and token-to-expert grouping (histogram, prefix
// sum, stable permutation) for the routed MoE layer.
//
// The router itself is unchanged by the method (gist.science page of arXiv
// 2605.08575, Technical Summary, Methodology: router logic preserved); the
// grouping is what lets every expert process its tokens as one batch.
#include "moe_internal.h"
#include "route.h"
#include "wave_reduce.h"

namespace moe {

// ---------------------------------------------------------------------------
// k_route: one wavefront per token.  Each lane holds up to 8 logits (E <= 512).
// The experts are picked in descending logit order (ties to the lower id) by
// a ballot search for the K-th largest logit; softmax weights are
// exp(l - max) / sum exp(l - max).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_route(const float *__restrict__ logits, int T, int E, int K,
                                               int renorm, int32_t *__restrict__ ids, float *__restrict__ w)
{
    __shared__ uint64_t s_sel[4][kSelWords];
    const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (t >= T) return;
    int id;
    float wt;
    route_token(logits, t, E, K, renorm, s_sel[threadIdx.x / kWave], id, wt);
    const int lane = threadIdx.x & (kWave - 1);
    if (lane < K) {
        ids[(size_t)t * K + lane] = id;
        w[(size_t)t * K + lane] = wt;
    }
}

hipError_t launch_route(const float *logits, int T, int E, int K, int renorm, int32_t *ids,
                        float *w, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    const int waves = 4;
    hipLaunchKernelGGL(k_route, dim3((T + waves - 1) / waves), dim3(waves * kWave), 0, stream,
                       logits, T, E, K, renorm, ids, w);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// k_group: one workgroup of 16 wavefronts.  Routed assignments a = t*K + k are
// ordered by expert, and within an expert by a (a stable counting sort):
//   pass 1  each wavefront counts its contiguous segment per expert;
//   scan    per-expert totals, per-wavefront bases, exclusive prefix over
//           experts, the ascending list of touched experts;
//   pass 2  each wavefront re-walks its segment and scatters.
// Lanes holding the same expert are found with one ballot per id bit; their
// leader updates the per-wavefront counter with an LDS atomic and shares the
// old value, so the rank inside a 64-assignment chunk is a popcount.
// The S shared experts follow the routed pairs: pair A + s*T + t.
// ---------------------------------------------------------------------------
constexpr int kGroupWaves = 16;

__device__ __forceinline__ uint64_t peers_of(int e, bool valid)
{
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 9; ++b) {  // ids < 512
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return valid ? m : 0ull;
}

constexpr int kIdBatch = 8;

// The ids of chunks b0, b0 + 64, ... (kIdBatch of them) for this lane; loads
// past a_end repeat the last id (unconditional loads, never used).
__device__ __forceinline__ void load_id_batch(const int32_t *ids, int b0, int a_end, int lane, int (&ev)[kIdBatch])
{
#pragma unroll
    for (int j = 0; j < kIdBatch; ++j) ev[j] = ids[min(b0 + j * kWave + lane, a_end - 1)];
}

// Groups the routed pairs [rb, re) (the whole batch, or one block of it).
// With blockcnt (per-block expert counts of nblk blocks of kGroupBlock pairs,
// this being block myblk), an expert's pairs from earlier blocks come first;
// without it the range is the whole batch.  Only the writer workgroup stores
// the per-expert metadata (counts, offsets, touched lists, MFMA work items)
// and the shared experts' pairs; every workgroup derives the same offsets.
__device__ __forceinline__ void group_body(const GroupParams &p, const int32_t *ids, int rb, int re,
                                           const int32_t *blockcnt, int nblk, int myblk, bool writer)
{
    __shared__ int s_cnt[kGroupWaves][kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_before[kMaxExperts];  // this expert's pairs in earlier blocks
    __shared__ int s_tot[kMaxExperts];     // pairs per expert (the whole batch)
    __shared__ int s_mb[kMaxExperts];      // pairs of MFMA experts before this expert (grouped order)
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid / kWave;
    const int EX = p.E + p.S;

    for (int i = tid; i < kGroupWaves * kMaxExperts; i += blockDim.x) (&s_cnt[0][0])[i] = 0;
    __syncthreads();

    const int chunks = (re - rb + kWave - 1) / kWave;
    const int per_wave = (chunks + kGroupWaves - 1) / kGroupWaves;
    const int a_begin = rb + wv * per_wave * kWave;
    const int a_end = min(re, rb + (wv + 1) * per_wave * kWave);

    // pass 1: per-wavefront counts (the ids of kIdBatch chunks are loaded at
    // once: one memory latency per batch instead of one per chunk; the first
    // batch stays in registers for pass 2)
    int ev0[kIdBatch];
    if (a_begin < a_end) load_id_batch(ids, a_begin, a_end, lane, ev0);
    for (int b0 = a_begin; b0 < a_end; b0 += kIdBatch * kWave) {
        int ev[kIdBatch];
        if (b0 == a_begin) {
#pragma unroll
            for (int j = 0; j < kIdBatch; ++j) ev[j] = ev0[j];
        } else {
            load_id_batch(ids, b0, a_end, lane, ev);
        }
#pragma unroll
        for (int j = 0; j < kIdBatch; ++j) {
            const int base = b0 + j * kWave;
            if (base >= a_end) break;
            const bool valid = base + lane < a_end;
            const int e = valid ? ev[j] : 0;
            const uint64_t peers = peers_of(e, valid);
            if (valid && (__ffsll((long long)peers) - 1) == lane) atomicAdd(&s_cnt[wv][e], __popcll(peers));
        }
    }
    __syncthreads();

    // per-expert totals; s_cnt becomes the per-wavefront base inside the expert
    for (int e = tid; e < EX; e += blockDim.x) {
        int run = 0, before = 0;
        if (e < p.E) {
            for (int w2 = 0; w2 < kGroupWaves; ++w2) {
                const int c = s_cnt[w2][e];
                s_cnt[w2][e] = run;
                run += c;
            }
            if (blockcnt) {  // the whole batch's count, and the earlier blocks' share
                int tot = 0;
                for (int b = 0; b < nblk; ++b) {
                    const int c = blockcnt[(size_t)b * p.E + e];
                    tot += c;
                    before += b < myblk ? c : 0;
                }
                run = tot;
            }
        } else {
            run = p.T;  // a shared expert serves every token
        }
        s_off[e] = run;  // total for now
        s_tot[e] = run;
        s_before[e] = before;
    }
    __syncthreads();
    if (wv == 0) {
        // exclusive prefix over experts: lane l owns experts [8l, 8l+8)
        constexpr int kPer = kMaxExperts / kWave;
        int loc[kPer];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            loc[i] = e < EX ? s_off[e] : 0;
            sum += loc[i];
        }
        const int incl = wave_incl_scan_dpp(sum);
        int run = incl - sum;
        int ntouched_before = 0;
        // pairs of the MFMA experts before each expert: a GEMV expert's pairs
        // take the compact rows [offset - that, ...) of the down pieces
        int msum = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) msum += (lane * kPer + i < EX && loc[i] >= p.nm) ? loc[i] : 0;
        int mrun = wave_incl_scan_dpp(msum) - msum;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            if (e < EX) s_mb[e] = mrun;
            mrun += (e < EX && loc[i] >= p.nm) ? loc[i] : 0;
        }
        // touched list needs the counts in ascending expert order
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            if (e < EX) {
                if (writer) {
                    p.counts[e] = loc[i];
                    p.offsets[e] = run;
                    if (p.ucount) p.ucount[e] = 0;
                }
                s_off[e] = run;
            }
            run += loc[i];
            ntouched_before += (e < EX && loc[i] > 0) ? 1 : 0;
        }
        if (lane == kWave - 1) {
            if (writer) p.offsets[EX] = run;
            s_off[EX] = run;
        }
      if (writer) {
        // touched experts, ascending: exclusive prefix of per-lane touched counts
        const int tincl = wave_incl_scan_dpp(ntouched_before);
        int tpos = tincl - ntouched_before;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            if (e < EX) {
                if (loc[i] > 0) {
                    p.slot_n[tpos] = loc[i];
                    p.slot_off[tpos] = s_off[e];
                    p.touched[tpos++] = e;
                }
                else if (p.union_cnt) p.union_cnt[e] = 0;
            }
        }
        if (lane == kWave - 1) {
            p.hdr[0] = tincl;
        }
        // MFMA work items: (expert, 64-token tile) of every expert with at
        // least nm pairs, ascending expert then tile
        int tiles = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            if (e < EX && loc[i] >= p.nm) tiles += (loc[i] + kMfmaTokens - 1) / kMfmaTokens;
        }
        const int iincl = wave_incl_scan_dpp(tiles);
        // and the projection's item pairs (two adjacent token tiles of one
        // expert, or its last tile alone): (first item index << 1) | has second
        int npairs = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            if (e < EX && loc[i] >= p.nm) npairs += ((loc[i] + kMfmaTokens - 1) / kMfmaTokens + 1) / 2;
        }
        const int pincl = wave_incl_scan_dpp(npairs);
        int ipos = iincl - tiles, ppos = pincl - npairs;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            if (e < EX && loc[i] >= p.nm) {
                const int nt = (loc[i] + kMfmaTokens - 1) / kMfmaTokens;
                for (int tl = 0; tl < nt; ++tl) {
                    if ((tl & 1) == 0) p.pairs[ppos++] = (ipos << 1) | (tl + 1 < nt ? 1 : 0);
                    p.items[ipos++] = (e << 16) | tl;
                }
            }
        }
        if (lane == kWave - 1) {
            p.hdr[1] = iincl;
            p.hdr[2] = pincl;
        }
      }
    } else if (wv == 1 && writer && p.order) {
        // The order in which the GEMV projection takes the touched experts:
        // by descending pair count (16 or more share the first class), ties
        // by slot.  Longest first keeps the experts that need two token tiles
        // (more than 8 pairs) from starting last and trailing the grid.  A
        // stable counting sort over 16 classes, in this wavefront while
        // wavefront 0 writes the metadata: a lane's class counts are packed
        // three to an int, 10 bits each (a class holds at most 512 experts,
        // so no field carries into the next), and summed across the lanes by
        // prefix scans.  Each entry also carries the expert's pair count and
        // first grouped pair, so a projection workgroup finds its work with
        // one load.
        constexpr int kPer = kMaxExperts / kWave;
        constexpr int kCls = 16;
        constexpr int kWords = (kCls + 2) / 3;
        int cls[kPer];
        int cnt[kWords];
#pragma unroll
        for (int j = 0; j < kWords; ++j) cnt[j] = 0;
        int ntl = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            const int n = e < EX ? s_tot[e] : 0;
            cls[i] = n <= 0 ? -1 : (n >= kCls ? 0 : kCls - n);
            if (n > 0) {
                ++ntl;
#pragma unroll
                for (int j = 0; j < kWords; ++j) cnt[j] += (cls[i] / 3 == j) ? 1 << (10 * (cls[i] % 3)) : 0;
            }
        }
        int slot = wave_incl_scan_dpp(ntl) - ntl;  // slot of this lane's first touched expert
        int lsum = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) lsum += (lane * kPer + i < EX) ? s_tot[lane * kPer + i] : 0;
        int first = wave_incl_scan_dpp(lsum) - lsum;  // first grouped pair of this lane's first expert
        int pos[kWords];  // next position of each class for this lane, packed
        int run = 0;      // experts in the classes before (uniform)
#pragma unroll
        for (int j = 0; j < kWords; ++j) {
            const int incl = wave_incl_scan_dpp(cnt[j]);
            const int tot = __builtin_amdgcn_readlane(incl, kWave - 1);
            int base = 0;
#pragma unroll
            for (int f = 0; f < 3; ++f)
                if (3 * j + f < kCls) {
                    base |= run << (10 * f);
                    run += (tot >> (10 * f)) & 1023;
                }
            pos[j] = base + incl - cnt[j];
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = cls[i];
            if (c >= 0) {
                const int sh = 10 * (c % 3);
                int w = 0;
#pragma unroll
                for (int j = 0; j < kWords; ++j) w = (c / 3 == j) ? pos[j] : w;
                const int e = lane * kPer + i;
                reinterpret_cast<int4 *>(p.order)[(w >> sh) & 1023] = make_int4((slot << 16) | e, s_tot[e], first, 0);
#pragma unroll
                for (int j = 0; j < kWords; ++j) pos[j] += (c / 3 == j) ? 1 << sh : 0;
                ++slot;
            }
            first += (lane * kPer + i < EX) ? s_tot[lane * kPer + i] : 0;
        }
    }
    __syncthreads();
    // union words of the MFMA experts are built with atomic ORs: clear them
    if (writer && p.union_words)
        for (int i = tid; i < EX * p.W; i += blockDim.x) {
            const int e = i / p.W;
            if (s_off[e + 1] - s_off[e] >= p.nm) p.union_words[i] = 0u;
        }

    // pass 2: stable scatter of the routed pairs
    for (int b0 = a_begin; b0 < a_end; b0 += kIdBatch * kWave) {
        int ev[kIdBatch];
        if (b0 == a_begin) {
#pragma unroll
            for (int j = 0; j < kIdBatch; ++j) ev[j] = ev0[j];
        } else {
            load_id_batch(ids, b0, a_end, lane, ev);
        }
#pragma unroll
        for (int j = 0; j < kIdBatch; ++j) {
            const int base = b0 + j * kWave;
            if (base >= a_end) break;
            const int a = base + lane;
            const bool valid = a < a_end;
            const int e = valid ? ev[j] : 0;
            const uint64_t peers = peers_of(e, valid);
            const int leader = valid ? (__ffsll((long long)peers) - 1) : lane;
            int old = 0;
            if (valid && leader == lane) old = atomicAdd(&s_cnt[wv][e], __popcll(peers));
            old = __shfl(old, leader, kWave);
            if (valid) {
                const int rank = __popcll(peers & lanemask_lt());
                const int pos = s_off[e] + s_before[e] + old + rank;
                const int t = a / p.K, k = a - t * p.K;
                p.pair_tok[pos] = t;
                p.pair_slot[pos] = k;
                if (p.cidx) p.cidx[t * p.slots + k] = (s_off[e + 1] - s_off[e] >= p.nm) ? -1 : pos - s_mb[e];
            }
        }
    }
    // shared experts: pair A + s*T + t
    if (writer)
    for (int i = tid; i < p.S * p.T; i += blockDim.x) {
        const int s = i / p.T, t = i - s * p.T;
        const int pos = p.A + i;
        p.pair_tok[pos] = t;
        p.pair_slot[pos] = p.K + s;
        if (p.cidx) p.cidx[t * p.slots + p.K + s] = (p.T >= p.nm) ? -1 : pos - s_mb[p.E + s];
    }
}

__global__ __launch_bounds__(1024) void k_group(GroupParams p) { group_body(p, p.ids, 0, p.A, nullptr, 0, 0, true); }

// Large batches: the grouping over blocks of kGroupBlock pairs, one workgroup
// each.  k_group_count stores each block's per-expert counts; k_group_scatter
// places each block's pairs after the same expert's pairs of earlier blocks
// (the same stable order as one workgroup over the whole batch), and its
// block 0 stores the per-expert metadata.
__global__ __launch_bounds__(256) void k_group_count(GroupParams p)
{
    __shared__ int s_h[kMaxExperts];
    for (int e = threadIdx.x; e < p.E; e += blockDim.x) s_h[e] = 0;
    __syncthreads();
    const int rb = blockIdx.x * kGroupBlock, re = min(p.A, rb + kGroupBlock);
    for (int a = rb + threadIdx.x; a < re; a += blockDim.x) atomicAdd(&s_h[p.ids[a]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < p.E; e += blockDim.x) p.blockcnt[(size_t)blockIdx.x * p.E + e] = s_h[e];
}

__global__ __launch_bounds__(1024) void k_group_scatter(GroupParams p)
{
    const int b = blockIdx.x;
    group_body(p, p.ids, b * kGroupBlock, min(p.A, (b + 1) * kGroupBlock), p.blockcnt, gridDim.x, b, b == 0);
}

// Routing (many workgroups, one wavefront per token) then grouping (one
// workgroup).  Routing inside the grouping workgroup was slower at every
// batch size measured (1 to 64 tokens, with 1 to 64 lanes per token): one
// compute unit routes the batch, and the grouping alone costs about as much
// as the second launch saves.
hipError_t launch_route_group(const float *logits, int renorm, int32_t *ids, float *w, const GroupParams &gp,
                              hipStream_t stream)
{
    if (gp.T <= 0) return hipSuccess;
    const hipError_t e = launch_route(logits, gp.T, gp.E, gp.K, renorm, ids, w, stream);
    if (e != hipSuccess) return e;
    if (gp.A > kGroupBlock && gp.blockcnt) {
        const int nb = (gp.A + kGroupBlock - 1) / kGroupBlock;
        hipLaunchKernelGGL(k_group_count, dim3(nb), dim3(256), 0, stream, gp);
        hipLaunchKernelGGL(k_group_scatter, dim3(nb), dim3(kGroupWaves * kWave), 0, stream, gp);
    } else {
        hipLaunchKernelGGL(k_group, dim3(1), dim3(kGroupWaves * kWave), 0, stream, gp);
    }
    return hipGetLastError();
}

}  // namespace moe
