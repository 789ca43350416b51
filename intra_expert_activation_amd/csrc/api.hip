// Exported C ABI of libmoesparse: argument validation, the launch plan, the
// workspace layout and the kernel sequence of each call.
//
// Every check that can fail on the host runs before the first HIP call, so a
// bad call is reported without touching a device.  No call allocates memory,
// synchronises the host or issues a memset (zeroing, where needed, is done by
// kernels), so calls can be captured in a HIP graph.
#include <limits.h>
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "moe_internal.h"
#include "moe_sparse_prof.h"

namespace moe {

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

moe_status make_plan(const moe_shape *s, int mode, int calib_tokens, Plan *p)
{
    if (!s || !p) return MOE_ERR_INVALID_ARG;
    const bool calib = calib_tokens > 0;
    if (!calib && mode != MOE_SPARSE && mode != MOE_DENSE && mode != MOE_TOPK) return MOE_ERR_INVALID_ARG;
    const int T = calib ? calib_tokens : s->T;
    if (T < 0 || s->H <= 0 || s->E <= 0 || s->I <= 0 || s->K <= 0 || s->K > s->E || s->S < 0)
        return MOE_ERR_INVALID_ARG;
    if (s->S > 0 && s->I_shared <= 0) return MOE_ERR_INVALID_ARG;
    if (s->x_dtype != MOE_F32 && s->x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (s->w_dtype != MOE_F32 && s->w_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (s->renormalize != 0 && s->renormalize != 1) return MOE_ERR_INVALID_ARG;
    if (s->K > kMaxK) return MOE_ERR_UNSUPPORTED;
    // the kernels take hidden states and weights of one element type
    if (s->x_dtype != s->w_dtype) return MOE_ERR_UNSUPPORTED;

    memset(p, 0, sizeof *p);
    p->T = T;
    p->H = s->H;
    p->E = s->E;
    p->I = s->I;
    p->K = s->K;
    p->S = s->S;
    p->Is = s->S > 0 ? s->I_shared : 0;
    p->dtype = s->w_dtype;
    p->renorm = s->renormalize;
    p->epl = s->w_dtype == MOE_BF16 ? 8 : 4;
    if (p->H % (kWave * p->epl) != 0) return MOE_ERR_UNSUPPORTED;
    p->NS = p->H / (kWave * p->epl);
    if (p->NS != 1 && p->NS != 2 && p->NS != 4 && p->NS != 8 && p->NS != 16) return MOE_ERR_UNSUPPORTED;
    if (p->I % 32 != 0 || p->I > kMaxRows) return MOE_ERR_UNSUPPORTED;
    if (p->S > 0 && (p->Is % 32 != 0 || p->Is > kMaxRows)) return MOE_ERR_UNSUPPORTED;
    if (p->E + p->S > kMaxExperts) return MOE_ERR_UNSUPPORTED;
    // sizes that index device buffers must fit the kernels' int arithmetic
    const long long P_ll = (long long)T * (s->K + s->S);
    if (P_ll > INT_MAX / 64) return MOE_ERR_UNSUPPORTED;

    p->Imax = (p->S > 0 && p->Is > p->I) ? p->Is : p->I;
    p->W = p->Imax / 32;
    p->slots = p->K + p->S;
    p->A = T * p->K;
    p->P = T * p->slots;
    p->EX = p->E + p->S;
    p->max_touched = T > 0 ? (p->A < p->E ? p->A : p->E) + p->S : 0;

    // rows per projection workgroup: the smallest multiple of 32 that keeps the
    // grid at or below ~2048 workgroups (8 per CU on 256 CUs)
    // the projection kernel gives each workgroup one 32-row mask word
    p->R = 32;
    p->C = p->Imax / 32;

    // largest token tile: the kernels pick 1, 2, 4 or 8 per tile to cover an
    // expert's remaining pairs, so its rows stream once when n_e <= TT.  At
    // most 8 (the dot products of larger tiles outrun the weight stream) and
    // at most 16 vectors of hidden states per lane (a wavefront holds NS/4 of
    // a row); no expert has more than T pairs.
    const int nsw = p->NS <= 4 ? 1 : p->NS / 4;
    const int tt_cap = 16 / nsw < 8 ? 16 / nsw : 8;
    p->TT = 1;
    while (p->TT < T && p->TT < tt_cap) p->TT *= 2;

    // down projection: workgroup column tiles of 1024 columns (2 KB of a bf16
    // row).  Up to GD workgroups (the launcher lowers it to
    // what the device holds resident at once) each take an equal share of the
    // (expert tile, column tile, union row) work; a group is cut into at most
    // KMAX pieces, whose partial sums the combine adds in order.
    p->NCT = (p->H + 1023) / 1024;
    // KMAX - 1 >= Imax / kDownChunk, so shares of kDownChunk rows never cut a
    // group into more than KMAX pieces.  Shares are at least umax / (KMAX - 1)
    // rows, so a small KMAX idles workgroups when few wide experts hold all
    // the work: one piece per 512 rows of I keeps shares down to ~256 rows
    // there, at a partial-sum cost of a few percent of the weight bytes.
    p->KMAX = 8;
    if ((p->Imax + 511) / 512 + 1 > p->KMAX) p->KMAX = (p->Imax + 511) / 512 + 1;
    if ((p->Imax + kDownChunk - 1) / kDownChunk + 1 > p->KMAX) p->KMAX = (p->Imax + kDownChunk - 1) / kDownChunk + 1;
    // every resident workgroup takes a share (shares never go below
    // kMinShare rows, so small batches leave the rest idle); sizing GD by the
    // number of touched experts starved layers of few, wide experts (8 experts
    // x 14336 rows: 128 workgroups, 1.1 TB/s)
    p->GD = 1024;

    // MFMA path: bf16 experts with at least nm = 16 pairs.  A routed expert has
    // at most T pairs, so with T below the threshold it is off.  An expert with
    // 16 to 31 pairs costs the GEMV body 2 to 4 passes over its rows (from HBM
    // once its rows outgrow L2), more than a mostly idle 128-token MFMA tile:
    // DeepSeek-style layer, T 64: 211 -> 193 us; Mixtral-style, T 128: the
    // measurement is in the design notes.
    p->nm = INT_MAX;
    p->use_mfma = 0;
    p->NT = (p->Imax + 63) / 64;
    p->max_items = 0;
    p->max_pairs = 0;
    const int nm = kMfmaMinPairs;
    p->topk = (!calib && mode == MOE_TOPK) ? 1 : 0;
    if (!calib && !p->topk && p->dtype == MOE_BF16 && T >= nm) {
        p->nm = nm;
        p->use_mfma = 1;
        // sum over experts of ceil(n_e / 64) <= A/64 + (number of such experts)
        const int big = (p->A / p->nm < p->E ? p->A / p->nm : p->E);
        p->max_items = p->A / kMfmaTokens + big + p->S * ((T + kMfmaTokens - 1) / kMfmaTokens);
        // an expert with k tiles has ceil(k / 2) pairs
        p->max_pairs = (p->max_items + big + p->S + 1) / 2;
    }
    // pairs of the GEMV experts (fewer than nm pairs each when the MFMA path
    // is on): the rows of the down pieces after the first
    {
        const long long g = p->use_mfma ? (long long)p->EX * (p->nm - 1) : (long long)p->P;
        p->G = (int)(g < p->P ? g : p->P);
    }
    // MFMA down: a workgroup per (item, 128 columns) walks the expert's
    // neuron tiles one staged tile at a time, so with few items (a few wide
    // experts: 8 experts x 224 neuron tiles at 128-256 tokens) the grid holds
    // a few hundred long serial walks.  Splitting the tiles into segments, one
    // partial sum each (added by the combine in segment order), fills the
    // device.
    p->NKS = 1;
    if (p->use_mfma) {
        const long long units = (long long)p->max_items * (p->H / kMfmaDownCols);
        while (p->NKS < kMfmaDownMaxSegs && units * p->NKS < kMfmaDownUnits &&
               p->NT >= kMfmaDownMinTiles * (p->NKS + 1))
            ++p->NKS;
    }

    // one-launch decode path: single-token batches (every expert has one
    // pair), and small batches of layers whose experts' gate matrices hold at
    // most 16 MiB: up to 8 tokens, or up to kFusedMaxT when there are no
    // shared experts and T * K <= E (about one pair per touched expert).  That
    // path gives each (token, slot) pair its own workgroups, so an expert
    // chosen by several tokens (a shared expert by all of them) has its rows
    // read once per pair, mostly from cache while the pairs run together; with
    // small experts and few repeats that costs less than the grouping and the
    // separate down launch save.  Measured (us per call, grouped -> one
    // launch): Qwen-style T 2/4/8/12/16: 37.9/47.2/66.2/79.0/89.9 ->
    // 20.9/31.6/54.5/68.8/89.1, T 24: 114 -> 126; DeepSeek-style (2 shared
    // experts) T 2/4/8: 46.8/60.9/83.0 -> 28.8/46.3/81.8, T 12: 98 -> 113;
    // Mixtral-style (117 MiB of gate per expert) T 2: 122 -> 126.
    {
        const size_t gate_bytes = (size_t)p->Imax * p->H * (p->dtype == MOE_BF16 ? 2 : 4);
        // In DENSE mode every row of every pair is streamed, so repeated
        // experts cost three times as much: Qwen-style dense T 2/4/8
        // 48.8/68.1/105.9 -> 35.1/58.1/109.1, DeepSeek-style (whose shared
        // experts repeat for every token) 62.3/85.1/112.9 -> 49.4/90.1/174.1.
        const bool small =
            gate_bytes <= ((size_t)16 << 20) &&
            (mode == MOE_DENSE ? (T <= 2 || (p->S == 0 && T <= 4))
                               : (T <= 8 || (p->S == 0 && T <= kFusedMaxT && T * p->K <= p->E)));
        p->fused = !calib && !p->topk && T >= 1 && (T == 1 || small) ? 1 : 0;
    }

    // workspace layout
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    p->off_ids = take((size_t)p->A * 4);
    p->off_w = take((size_t)p->A * 4);
    p->off_hdr = take(64 * 4);
    p->off_counts = take((size_t)p->EX * 4);
    p->off_offsets = take((size_t)(p->EX + 1) * 4);
    p->off_touched = take((size_t)p->EX * 4);
    p->off_slotn = take((size_t)p->EX * 4);
    p->off_slotoff = take((size_t)p->EX * 4);
    p->off_pair_tok = take((size_t)p->P * 4);
    p->off_pair_slot = take((size_t)p->P * 4);
    p->off_union = take((size_t)p->EX * p->W * 4);
    p->off_ucount = take((size_t)p->EX * 4);
    p->off_npc = take(calib ? 0 : (size_t)p->P * p->NCT * 4);
    p->off_h = take(((size_t)p->A * p->I + (size_t)p->S * T * p->Is) * 4);
    // down outputs: piece 0 of every pair [P, H]; the later pieces of the
    // GEMV experts' pairs [KMAX - 1, G, H]; the later segments of the MFMA
    // experts' pairs [NKS - 1, P, H] (the one-launch path keeps its chunk
    // partial rows [P, C, H] here instead)
    p->off_partial = take(calib ? 0
                                : (p->fused ? (size_t)p->C * p->P
                                            : (size_t)p->P + (size_t)(p->KMAX - 1) * p->G +
                                                  (size_t)(p->NKS - 1) * p->P) *
                                      p->H * 4);
    p->off_cidx = take(calib ? 0 : (size_t)p->P * 4);
    p->off_taus = take((size_t)(2 + p->EX) * 4);
    const size_t blocks = (size_t)p->max_items * p->NT;
    p->off_items = take((size_t)p->max_items * 4);
    p->off_pairs = take((size_t)p->max_pairs * 4);
    p->off_blockcnt = take((size_t)((p->A + kGroupBlock - 1) / kGroupBlock) * p->E * 4);
    p->off_order = take((size_t)p->EX * 16);
    p->off_nact = take(blocks * 4);
    p->off_list = take(blocks * 64);
    p->off_hhi = take(blocks * 64 * 64 * 2);
    p->off_hlo = take(blocks * 64 * 64 * 2);
    p->off_mw = take((p->fused || p->topk) ? (size_t)p->P * p->W * 4 : 0);
    p->total = o;
    return MOE_OK;
}

static bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

template <class T>
static T *ws_at(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }

}  // namespace moe

using namespace moe;

extern "C" {

const char *moe_status_string(int32_t status)
{
    switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument (NULL pointer, bad size, bad enum, q outside [0,1] or misaligned pointer)";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape outside what the kernels implement";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than required";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP kernel launch or runtime call failed";
    }
    return "unknown moe_status";
}

moe_status moe_workspace_size(const moe_shape *shape, int32_t mode, size_t *bytes)
{
    if (!bytes) return MOE_ERR_INVALID_ARG;
    Plan pl;
    const moe_status st = make_plan(shape, mode, 0, &pl);
    if (st != MOE_OK) return st;
    *bytes = pl.total;
    return MOE_OK;
}

moe_status moe_calibrate_workspace_size(const moe_shape *shape, int32_t Tc, size_t *bytes)
{
    if (!bytes || Tc <= 0) return MOE_ERR_INVALID_ARG;
    Plan pl;
    const moe_status st = make_plan(shape, MOE_SPARSE, Tc, &pl);
    if (st != MOE_OK) return st;
    *bytes = pl.total;
    return MOE_OK;
}

moe_status moe_route_topk(const float *logits, int32_t T, int32_t E, int32_t K, int32_t renormalize,
                          int32_t *topk_ids, float *topk_w, void *hip_stream)
{
    if (T < 0 || E <= 0 || K <= 0 || K > E || (renormalize != 0 && renormalize != 1))
        return MOE_ERR_INVALID_ARG;
    if (K > kMaxK || E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return MOE_ERR_INVALID_ARG;
    return launch_route(logits, T, E, K, renormalize, topk_ids, topk_w, (hipStream_t)hip_stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

}  // extern "C"

namespace moe {

// The layer call; ev_begin / ev_end (optional) bracket the projection kernel.
static moe_status ffn_call(const moe_shape *shape, int32_t mode, const moe_ffn_args *a, hipEvent_t ev_begin,
                          hipEvent_t ev_end, void *hip_stream)
{
    if (!shape || !a) return MOE_ERR_INVALID_ARG;
    Plan pl;
    moe_status st = make_plan(shape, mode, 0, &pl);
    if (st != MOE_OK) return st;
    if (pl.T == 0) return MOE_OK;
    if (!a->x || !a->router_logits || !a->w_gate || !a->w_up || !a->w_down || !a->y || !a->workspace)
        return MOE_ERR_INVALID_ARG;
    if (pl.S > 0 && (!a->ws_gate || !a->ws_up || !a->ws_down)) return MOE_ERR_INVALID_ARG;
    if (mode == MOE_SPARSE && !a->tau) return MOE_ERR_INVALID_ARG;
    if (mode == MOE_TOPK && a->neuron_budget < 0) return MOE_ERR_INVALID_ARG;
    const void *a16[] = {a->x, a->w_gate, a->w_up, a->w_down, a->y};
    for (const void *ptr : a16)
        if (!aligned(ptr, 16)) return MOE_ERR_INVALID_ARG;
    if (pl.S > 0 && (!aligned(a->ws_gate, 16) || !aligned(a->ws_up, 16) || !aligned(a->ws_down, 16)))
        return MOE_ERR_INVALID_ARG;
    const void *a4[] = {a->router_logits, a->tau, a->mask_bits, a->union_idx, a->union_cnt, a->topk_ids, a->topk_w};
    for (const void *ptr : a4)
        if (ptr && !aligned(ptr, 4)) return MOE_ERR_INVALID_ARG;
    if (!aligned(a->workspace, 256)) return MOE_ERR_INVALID_ARG;
    if (a->workspace_bytes < pl.total) return MOE_ERR_WORKSPACE;

    hipStream_t stream = (hipStream_t)hip_stream;
    void *ws = a->workspace;
    int32_t *ids = a->topk_ids ? a->topk_ids : ws_at<int32_t>(ws, pl.off_ids);
    float *w = a->topk_w ? a->topk_w : ws_at<float>(ws, pl.off_w);
    int32_t *hdr = ws_at<int32_t>(ws, pl.off_hdr);
    int32_t *counts = ws_at<int32_t>(ws, pl.off_counts);
    int32_t *offsets = ws_at<int32_t>(ws, pl.off_offsets);
    int32_t *touched = ws_at<int32_t>(ws, pl.off_touched);
    int32_t *slot_n = ws_at<int32_t>(ws, pl.off_slotn);
    int32_t *slot_off = ws_at<int32_t>(ws, pl.off_slotoff);
    int32_t *pair_tok = ws_at<int32_t>(ws, pl.off_pair_tok);
    int32_t *pair_slot = ws_at<int32_t>(ws, pl.off_pair_slot);
    uint32_t *union_words = ws_at<uint32_t>(ws, pl.off_union);
    int32_t *ucount = ws_at<int32_t>(ws, pl.off_ucount);
    int32_t *npc = ws_at<int32_t>(ws, pl.off_npc);
    float *h = ws_at<float>(ws, pl.off_h);
    float *partial = ws_at<float>(ws, pl.off_partial);

    if (pl.fused) {
        FusedParams fp{};
        fp.logits = a->router_logits;
        fp.x = a->x; fp.wg = a->w_gate; fp.wu = a->w_up; fp.wd = a->w_down;
        fp.swg = a->ws_gate; fp.swu = a->ws_up; fp.swd = a->ws_down;
        fp.tau = a->tau;
        fp.ids = ids; fp.w = w; fp.partial = partial; fp.mw = ws_at<uint32_t>(ws, pl.off_mw);
        fp.mask_bits = a->mask_bits; fp.union_idx = a->union_idx; fp.union_cnt = a->union_cnt;
        fp.y = a->y;
        fp.T = pl.T; fp.H = pl.H; fp.E = pl.E; fp.I = pl.I; fp.Is = pl.Is; fp.S = pl.S; fp.K = pl.K;
        fp.slots = pl.slots; fp.P = pl.P; fp.C = pl.C; fp.W = pl.W; fp.Imax = pl.Imax; fp.renorm = pl.renorm;
        KernelEvents kev{ev_begin, ev_end};
        return launch_fused(pl, fp, mode, &kev, stream)
                       == hipSuccess
                   ? MOE_OK
                   : MOE_ERR_HIP;
    }

    GroupParams gp{};
    gp.ids = ids;
    gp.T = pl.T; gp.K = pl.K; gp.E = pl.E; gp.S = pl.S; gp.A = pl.A; gp.P = pl.P; gp.slots = pl.slots;
    gp.hdr = hdr; gp.counts = counts; gp.offsets = offsets; gp.touched = touched; gp.slot_n = slot_n; gp.slot_off = slot_off;
    gp.pair_tok = pair_tok; gp.pair_slot = pair_slot;
    gp.union_cnt = a->union_cnt;
    gp.union_words = union_words;
    gp.ucount = ucount;
    gp.W = pl.W;
    gp.nm = pl.nm;
    gp.items = ws_at<int32_t>(ws, pl.off_items);
    gp.pairs = ws_at<int32_t>(ws, pl.off_pairs);
    gp.cidx = ws_at<int32_t>(ws, pl.off_cidx);
    gp.blockcnt = ws_at<int32_t>(ws, pl.off_blockcnt);
    gp.order = ws_at<int32_t>(ws, pl.off_order);
    if (launch_route_group(a->router_logits, pl.renorm, ids, w, gp, stream) != hipSuccess) return MOE_ERR_HIP;

    ProjParams pp{};
    pp.x = a->x; pp.wg = a->w_gate; pp.wu = a->w_up; pp.swg = a->ws_gate; pp.swu = a->ws_up;
    pp.tau = a->tau;
    pp.hdr = hdr; pp.counts = counts; pp.offsets = offsets; pp.touched = touched; pp.order = gp.order;
    pp.pair_tok = pair_tok; pp.pair_slot = pair_slot;
    pp.h = h; pp.mask_bits = a->mask_bits; pp.union_words = union_words; pp.ucount = ucount;
    pp.H = pl.H; pp.E = pl.E; pp.I = pl.I; pp.Is = pl.Is; pp.S = pl.S; pp.K = pl.K; pp.A = pl.A;
    pp.W = pl.W; pp.slots = pl.slots; pp.C = pl.C; pp.R = pl.R;
    pp.nm = pl.nm;

    MfmaParams mp{};
    mp.x = (const uint16_t *)a->x;
    mp.wg = (const uint16_t *)a->w_gate; mp.wu = (const uint16_t *)a->w_up; mp.wd = (const uint16_t *)a->w_down;
    mp.swg = (const uint16_t *)a->ws_gate; mp.swu = (const uint16_t *)a->ws_up; mp.swd = (const uint16_t *)a->ws_down;
    mp.tau = a->tau;
    mp.hdr = hdr; mp.counts = counts; mp.offsets = offsets; mp.items = ws_at<int32_t>(ws, pl.off_items);
    mp.pairs = ws_at<int32_t>(ws, pl.off_pairs); mp.max_pairs = pl.max_pairs;
    mp.pair_tok = pair_tok; mp.pair_slot = pair_slot;
    mp.hhi = ws_at<uint16_t>(ws, pl.off_hhi); mp.hlo = ws_at<uint16_t>(ws, pl.off_hlo);
    mp.nact = ws_at<int32_t>(ws, pl.off_nact); mp.list = ws_at<uint8_t>(ws, pl.off_list);
    mp.mask_bits = a->mask_bits; mp.union_words = union_words; mp.partial = partial; mp.npc = npc; mp.NCT = pl.NCT;
    mp.union_idx = a->union_idx; mp.union_cnt = a->union_cnt;
    mp.H = pl.H; mp.E = pl.E; mp.I = pl.I; mp.Is = pl.Is; mp.S = pl.S; mp.W = pl.W; mp.Imax = pl.Imax;
    mp.slots = pl.slots; mp.NT = pl.NT; mp.max_items = pl.max_items;
    mp.NKS = pl.NKS; mp.P = pl.P; mp.mbase = (size_t)pl.P + (size_t)(pl.KMAX - 1) * pl.G;

    // the events time the expert projection (gate, score, mask, up): the
    // kernel itself, or in top-k mode its three launches
    if (pl.topk) {
        // every pair's gate scores, the per-pair selection of the budget
        // largest, then the projection under those masks (up and h; the gate
        // is not read again)
        const KernelEvents first{ev_begin, nullptr}, last{nullptr, ev_end};
        if (launch_proj(pl, pp, mp, kModeScore, stream, &first) != hipSuccess) return MOE_ERR_HIP;
        TopkParams tp{};
        tp.a = h; tp.counts = counts; tp.offsets = offsets; tp.pair_tok = pair_tok; tp.pair_slot = pair_slot;
        tp.ids = ids; tp.pmask = ws_at<uint32_t>(ws, pl.off_mw);
        tp.E = pl.E; tp.I = pl.I; tp.Is = pl.Is; tp.K = pl.K; tp.A = pl.A; tp.W = pl.W; tp.budget = a->neuron_budget;
        if (launch_topk_select(pl, tp, stream) != hipSuccess) return MOE_ERR_HIP;
        pp.pmask = tp.pmask;
        if (launch_proj(pl, pp, mp, kModeMasked, stream, &last) != hipSuccess) return MOE_ERR_HIP;
    } else {
        const KernelEvents kev{ev_begin, ev_end};
        if (launch_proj(pl, pp, mp, mode, stream, &kev) != hipSuccess) return MOE_ERR_HIP;
    }

    DownParams dp{};
    dp.wd = a->w_down; dp.swd = a->ws_down; dp.h = h;
    dp.hdr = hdr; dp.counts = counts; dp.offsets = offsets; dp.touched = touched; dp.slot_n = slot_n; dp.slot_off = slot_off;
    dp.union_words = union_words; dp.ucount = ucount; dp.partial = partial; dp.npc = npc;
    dp.cidx = gp.cidx; dp.G = pl.G;
    dp.pair_tok = pair_tok; dp.pair_slot = pair_slot; dp.slots = pl.slots;
    dp.union_idx = a->union_idx; dp.union_cnt = a->union_cnt;
    dp.H = pl.H; dp.E = pl.E; dp.I = pl.I; dp.Is = pl.Is; dp.S = pl.S; dp.A = pl.A; dp.P = pl.P;
    dp.W = pl.W; dp.Imax = pl.Imax; dp.NCT = pl.NCT; dp.KMAX = pl.KMAX;
    dp.nm = pl.nm;
    // the top-k masks and unions are consumed like the threshold's
    if (launch_down(pl, dp, mp, pl.topk ? MOE_SPARSE : mode, stream) != hipSuccess) return MOE_ERR_HIP;

    CombineParams cp{};
    cp.partial = partial; cp.cidx = gp.cidx; cp.topk_w = w; cp.npc = npc; cp.y = a->y;
    cp.T = pl.T; cp.H = pl.H; cp.K = pl.K; cp.slots = pl.slots; cp.P = pl.P; cp.NCT = pl.NCT; cp.G = pl.G;
    cp.mbase = mp.mbase;
    if (launch_combine(pl, cp, stream) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

}  // namespace moe

extern "C" {

moe_status moe_sparse_expert_ffn(const moe_shape *shape, int32_t mode, const moe_ffn_args *args, void *hip_stream)
{
    return ffn_call(shape, mode, args, nullptr, nullptr, hip_stream);
}

}  // extern "C"

namespace moe {

// Scratch of moe_sparse_expert_ffn_noalloc: a fixed device array, one per GPU
// the library runs on, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: the device address comes
// from hipGetSymbolAddress, once per device, and only that address is passed
// to the kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::atomic<void *> g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// The current device's scratch address (looked up on the first call on that
// device, with that device current), or null with *err set.
static void *scratch_address(moe_status *err)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = MOE_ERR_HIP;
        return nullptr;
    }
    void *ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            *err = MOE_ERR_HIP;
            return nullptr;
        }
        g_scratch[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

}  // namespace moe

extern "C" {

moe_status moe_sparse_expert_ffn_noalloc(const moe_shape *shape, int32_t mode, const moe_ffn_args *args,
                                         void *hip_stream)
{
    if (!shape || !args) return MOE_ERR_INVALID_ARG;
    Plan pl;
    const moe_status st = make_plan(shape, mode, 0, &pl);
    if (st != MOE_OK) return st;
    if (pl.T == 0) return MOE_OK;
    if (pl.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;  // before any HIP call
    moe_status err = MOE_OK;
    void *ptr = scratch_address(&err);
    if (!ptr) return err;
    moe_ffn_args a = *args;
    a.workspace = ptr;
    a.workspace_bytes = MOE_NOALLOC_SCRATCH_BYTES;
    return ffn_call(shape, mode, &a, nullptr, nullptr, hip_stream);
}

moe_status moe_sparse_expert_ffn_profiled(const moe_shape *shape, int32_t mode, const moe_ffn_args *args,
                                          void *ev_begin, void *ev_end, void *hip_stream)
{
    return ffn_call(shape, mode, args, (hipEvent_t)ev_begin, (hipEvent_t)ev_end, hip_stream);
}

moe_status moe_calibrate_threshold(const moe_shape *shape, const void *x_calib, const float *logits_calib,
                                   int32_t Tc, const void *w_gate, const void *ws_gate, float q,
                                   int32_t per_expert, float *tau_out, void *workspace,
                                   size_t workspace_bytes, void *hip_stream)
{
    if (!shape || Tc <= 0) return MOE_ERR_INVALID_ARG;
    if (!(q >= 0.f && q <= 1.f)) return MOE_ERR_INVALID_ARG;  // also rejects NaN
    if (per_expert != 0 && per_expert != 1) return MOE_ERR_INVALID_ARG;
    Plan pl;
    moe_status st = make_plan(shape, MOE_SPARSE, Tc, &pl);
    if (st != MOE_OK) return st;
    if (!x_calib || !logits_calib || !w_gate || !tau_out || !workspace) return MOE_ERR_INVALID_ARG;
    if (pl.S > 0 && !ws_gate) return MOE_ERR_INVALID_ARG;
    if (!aligned(x_calib, 16) || !aligned(w_gate, 16) || (pl.S > 0 && !aligned(ws_gate, 16)))
        return MOE_ERR_INVALID_ARG;
    if (!aligned(logits_calib, 4) || !aligned(tau_out, 4) || !aligned(workspace, 256))
        return MOE_ERR_INVALID_ARG;
    if (workspace_bytes < pl.total) return MOE_ERR_WORKSPACE;

    hipStream_t stream = (hipStream_t)hip_stream;
    int32_t *ids = ws_at<int32_t>(workspace, pl.off_ids);
    float *w = ws_at<float>(workspace, pl.off_w);
    int32_t *hdr = ws_at<int32_t>(workspace, pl.off_hdr);
    int32_t *counts = ws_at<int32_t>(workspace, pl.off_counts);
    int32_t *offsets = ws_at<int32_t>(workspace, pl.off_offsets);
    int32_t *touched = ws_at<int32_t>(workspace, pl.off_touched);
    int32_t *slot_n = ws_at<int32_t>(workspace, pl.off_slotn);
    int32_t *slot_off = ws_at<int32_t>(workspace, pl.off_slotoff);
    int32_t *pair_tok = ws_at<int32_t>(workspace, pl.off_pair_tok);
    int32_t *pair_slot = ws_at<int32_t>(workspace, pl.off_pair_slot);
    float *scores = ws_at<float>(workspace, pl.off_h);
    float *taus = ws_at<float>(workspace, pl.off_taus);

    GroupParams gp{};
    gp.ids = ids;
    gp.T = pl.T; gp.K = pl.K; gp.E = pl.E; gp.S = pl.S; gp.A = pl.A; gp.P = pl.P; gp.slots = pl.slots;
    gp.hdr = hdr; gp.counts = counts; gp.offsets = offsets; gp.touched = touched; gp.slot_n = slot_n; gp.slot_off = slot_off;
    gp.pair_tok = pair_tok; gp.pair_slot = pair_slot; gp.union_cnt = nullptr;
    gp.union_words = nullptr; gp.W = pl.W; gp.nm = pl.nm; gp.items = nullptr; gp.pairs = nullptr;
    gp.cidx = nullptr;
    gp.blockcnt = ws_at<int32_t>(workspace, pl.off_blockcnt);
    gp.order = ws_at<int32_t>(workspace, pl.off_order);
    if (launch_route_group(logits_calib, 1, ids, w, gp, stream) != hipSuccess) return MOE_ERR_HIP;

    ProjParams pp{};
    pp.x = x_calib; pp.wg = w_gate; pp.wu = w_gate; pp.swg = ws_gate; pp.swu = ws_gate;
    pp.tau = nullptr;
    pp.hdr = hdr; pp.counts = counts; pp.offsets = offsets; pp.touched = touched; pp.order = gp.order;
    pp.pair_tok = pair_tok; pp.pair_slot = pair_slot;
    pp.h = scores; pp.mask_bits = nullptr; pp.union_words = nullptr;
    pp.H = pl.H; pp.E = pl.E; pp.I = pl.I; pp.Is = pl.Is; pp.S = pl.S; pp.K = pl.K; pp.A = pl.A;
    pp.W = pl.W; pp.slots = pl.slots; pp.C = pl.C; pp.R = pl.R;
    pp.nm = pl.nm;  // INT_MAX: every expert is scored by the GEMV kernel
    MfmaParams none{};
    if (launch_proj(pl, pp, none, kModeScore, stream) != hipSuccess) return MOE_ERR_HIP;

    SelectParams sp{};
    sp.scores = scores; sp.counts = counts; sp.offsets = offsets; sp.taus = taus; sp.q = q;
    sp.E = pl.E; sp.I = pl.I; sp.Is = pl.Is; sp.S = pl.S; sp.A = pl.A; sp.T = pl.T; sp.EX = pl.EX;
    sp.per_expert = per_expert;
    if (launch_select(pl, sp, tau_out, stream) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_timer_create(void **event)
{
    if (!event) return MOE_ERR_INVALID_ARG;
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return MOE_ERR_HIP;
    *event = (void *)e;
    return MOE_OK;
}

moe_status moe_timer_destroy(void *event)
{
    if (!event) return MOE_ERR_INVALID_ARG;
    return hipEventDestroy((hipEvent_t)event) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_timer_elapsed_ms(void *begin, void *end, float *ms)
{
    if (!begin || !end || !ms) return MOE_ERR_INVALID_ARG;
    if (hipEventSynchronize((hipEvent_t)end) != hipSuccess) return MOE_ERR_HIP;
    return hipEventElapsedTime(ms, (hipEvent_t)begin, (hipEvent_t)end) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
