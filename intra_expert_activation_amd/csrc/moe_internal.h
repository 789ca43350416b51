// Internal definitions of libmoesparse: the launch plan, workspace carving,
// kernel parameter blocks and small device helpers.  Not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_sparse.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 512;   // E + S
constexpr int kMaxK = 32;
constexpr int kMaxRows = 16384;    // I, I_shared
constexpr int kMaxRowsPerChunk = 256;
constexpr int kMfmaTokens = 64;    // token tile of the MFMA path
constexpr int kGroupBlock = 2048;  // routed pairs per grouping workgroup when the batch has more
constexpr int kMfmaMinPairs = 16;  // pair-count threshold of the MFMA path
constexpr int kFusedMaxT = 16;     // most tokens of a batch on the one-launch decode path
constexpr int kMfmaDownCols = 128; // output columns of an MFMA down workgroup
// The MFMA down splits each expert's neuron tiles into up to kMfmaDownMaxSegs
// segments (one partial sum each) while its grid bound, items x column tiles
// x segments, stays below kMfmaDownUnits; every segment keeps at least
// kMfmaDownMinTiles neuron tiles.
constexpr int kMfmaDownUnits = 1024;
constexpr int kMfmaDownMaxSegs = 4;
constexpr int kMfmaDownMinTiles = 8;

// ---------------------------------------------------------------------------
// Launch plan: every size a kernel grid or the workspace depends on.  It is a
// pure function of the shape (never of the data), so a call can be captured in
// a graph and the workspace size is known before the call.
// ---------------------------------------------------------------------------
struct Plan {
    int T, H, E, I, K, S, Is, dtype, renorm;
    int Imax;        // max(I, I_shared)
    int W;           // mask words per (token, slot) row = Imax / 32
    int slots;       // K + S
    int A;           // routed pairs T*K
    int P;           // all pairs T*(K+S)
    int EX;          // experts E + S
    int epl;         // elements per 16-byte vector (8 bf16, 4 f32)
    int NS;          // 16-byte vectors per lane per row: H / (64 * epl)
    int max_touched; // upper bound on experts with at least one pair
    // expert projection kernel (gate, score, mask, up)
    int R;           // neuron rows per workgroup (multiple of 32, <= 256)
    int C;           // row chunks per expert: ceil(Imax / R)
    int TT;          // tokens per register tile
    // down projection kernel
    int NCT;         // down column tiles of 1024 columns: ceil(H / 1024)
    int KMAX;        // most pieces a down group (expert tile, column tile) is cut into
    int GD;          // GEMV down workgroups (each takes an equal share of the work)
    // MFMA path for experts with at least `nm` pairs (bf16 only)
    int use_mfma;    // 0 when no expert can reach nm (T < nm) or for fp32 / scores
    int nm;          // pair-count threshold (INT_MAX when the path is off)
    int NT;          // 64-neuron tiles per expert: ceil(Imax / 64)
    int max_items;   // upper bound on (expert, 64-token tile) work items
    int max_pairs;   // upper bound on pairs of them (the MFMA projection's items)
    int G;           // upper bound on the pairs of GEMV experts (rows of the down pieces after the first)
    int NKS;         // segments of an MFMA expert's neuron tiles in the down product (pieces of its pairs)
    // one-launch decode path (small batches): every (pair, 32-row chunk)
    // runs routing, gate, mask, up and down; a second launch combines
    int fused;
    int topk;        // MOE_TOPK: scores, per-pair selection, then the masked projection
    // workspace layout (byte offsets)
    size_t off_ids, off_w, off_hdr, off_counts, off_offsets, off_touched, off_slotn, off_slotoff;
    size_t off_pair_tok, off_pair_slot, off_union, off_ucount, off_npc, off_h, off_partial;
    size_t off_cidx, off_taus;
    size_t off_items, off_pairs, off_blockcnt, off_order, off_nact, off_list, off_hhi, off_hlo;
    size_t off_mw;
    size_t total;
};

// Validates a shape; fills the plan.  calib_tokens > 0 plans a calibration
// (score) pass over that many tokens instead of a forward pass.
moe_status make_plan(const moe_shape *s, int mode, int calib_tokens, Plan *p);

// ---------------------------------------------------------------------------
// Kernel parameter blocks
// ---------------------------------------------------------------------------
struct GroupParams {
    const int32_t *ids;   // [T,K]
    int T, K, E, S, A, P, slots;
    int32_t *hdr;         // [0] = number of touched experts
    int32_t *counts;      // [EX]
    int32_t *offsets;     // [EX+1]
    int32_t *touched;     // [EX], ascending expert ids with count > 0
    int32_t *slot_n;      // [EX], pair count of touched[s]
    int32_t *slot_off;    // [EX], first grouped pair of touched[s]
    int32_t *pair_tok;    // [P] token of the pair at each grouped position
    int32_t *pair_slot;   // [P] slot of the pair
    int32_t *union_cnt;   // optional output, zeroed for untouched experts
    uint32_t *union_words;// [EX,W], zeroed for the experts on the MFMA path
    int32_t *ucount;      // [EX] union sizes of the GEMV experts by touched slot, zeroed here
    int W;
    int nm;               // MFMA pair-count threshold
    int32_t *items;       // [max_items] (expert << 16 | token tile) of MFMA experts
    int32_t *pairs;       // [max_pairs] (first item << 1 | has a second) for the MFMA projection
    int32_t *cidx;        // [P] by (t * slots + slot): the pair's row in the down pieces after the
                          // first (pairs of GEMV experts, numbered in grouped order), -1 for MFMA pairs
    int32_t *blockcnt;    // [ceil(A / kGroupBlock), E] per-block expert counts (large batches), or null
    int32_t *order;       // [EX][4] (slot << 16 | expert, pairs, first pair, 0) of the touched experts,
                          // by descending pair count
};

struct ProjParams {
    const void *x;
    const void *wg, *wu, *swg, *swu;
    const float *tau;
    const int32_t *hdr, *counts, *offsets, *touched, *pair_tok, *pair_slot;
    const int32_t *order; // GroupParams::order: the order in which workgroups take the experts
    const uint32_t *pmask;// kModeMasked: mask words by grouped pair [P, W]
    float *h;             // per-expert blocks [rows][n_e] (fp32)
    uint32_t *mask_bits;  // optional output [T,slots,W]
    uint32_t *union_words;// [EX,W]
    int32_t *ucount;      // [EX] by touched slot: += popcount of each union word written
    int H, E, I, Is, S, K, A, W, slots, C, R;
    int nm;               // experts with nm or more pairs take the MFMA path
};

constexpr int kDownChunk = 1024;  // largest share of a down wavefront (union rows)

struct DownParams {
    const void *wd, *swd;
    const float *h;
    const int32_t *hdr, *counts, *offsets, *touched, *slot_n, *slot_off;
    const uint32_t *union_words;
    const int32_t *ucount;  // by touched slot
    const int32_t *pair_tok, *pair_slot;
    // down output of pair (t, slot): piece 0 of its 1024-column tile c is
    // row t * slots + slot of partial, piece k >= 1 (GEMV experts only) is
    // row P + (k - 1) * G + cidx[t * slots + slot]; npc[(t * slots + slot) *
    // NCT + c] pieces (0: no active row, the output is zero)
    float *partial;       // [P + (KMAX - 1) * G, H]
    const int32_t *cidx;  // [P]
    int32_t *npc;         // [P, NCT]
    int32_t *union_idx;   // optional output [EX, Imax]
    int32_t *union_cnt;   // optional output [EX]
    int H, E, I, Is, S, A, P, W, Imax, NCT, KMAX, GD, G, slots;
    int nm;
};

struct CombineParams {
    const float *partial; // as DownParams
    const int32_t *cidx;  // as DownParams
    const float *topk_w;
    const int32_t *npc;   // as DownParams
    float *y;
    size_t mbase;         // as MfmaParams: pieces after the first of an MFMA pair (cidx -1)
    int T, H, K, slots, P, NCT, G;
};

struct MfmaParams {
    const uint16_t *x, *wg, *wu, *wd, *swg, *swu, *swd;
    const float *tau;
    const int32_t *hdr, *counts, *offsets, *items, *pairs, *pair_tok, *pair_slot;
    uint16_t *hhi, *hlo;  // compacted h per (item, neuron tile): [64 tokens][64] bf16 hi / lo
    int32_t *nact;        // active rows per (item, neuron tile)
    uint8_t *list;        // their offsets within the tile, ascending
    uint32_t *mask_bits, *union_words;
    float *partial;       // as DownParams; piece k >= 1 of a pair at row mbase + (k - 1) P + (t * slots + slot)
    int32_t *npc;         // as DownParams
    int32_t *union_idx, *union_cnt;
    size_t mbase;         // first row of the MFMA pairs' pieces after the first
    int H, E, I, Is, S, W, Imax, slots, NT, max_items, max_pairs, NCT, NKS, P;
};

// One-launch decode path.  Pair p = t * slots + slot; chunk c = rows
// [32c, 32c + 32) of the pair's expert.
struct FusedParams {
    const float *logits;  // [T,E]
    const void *x, *wg, *wu, *wd, *swg, *swu, *swd;
    const float *tau;
    int32_t *ids;         // [T,K] routing outputs (the caller's or the workspace's)
    float *w;             // [T,K]
    float *partial;       // [P, C, H]: chunk c's down partial sum of pair p
    uint32_t *mw;         // [P, W] mask words (always written)
    uint32_t *mask_bits;  // optional output [P, W]
    int32_t *union_idx, *union_cnt;  // optional outputs
    float *y;
    int T, H, E, I, Is, S, K, slots, P, C, W, Imax, renorm;
};

// Per-pair top-k neuron selection (MOE_TOPK).
struct TopkParams {
    const float *a;       // scores as ProjParams::h after kModeScore
    const int32_t *counts, *offsets, *pair_tok, *pair_slot, *ids;
    uint32_t *pmask;      // out [P, W] by grouped pair
    int E, I, Is, K, A, W, budget;
};

struct SelectParams {
    const float *scores;  // |SiLU| per (pair, neuron), expert blocks as ProjParams::h
    const int32_t *counts, *offsets;
    float *taus;          // [2 + EX]: routed, shared, then per expert
    float q;
    int E, I, Is, S, A, T, EX, per_expert;
};

// ---------------------------------------------------------------------------
// Host-side launchers (each enqueues on `stream` and returns hipGetLastError)
// ---------------------------------------------------------------------------
// Optional timing of a launch: the kernel is dispatched by
// hipExtLaunchKernelGGL, whose start and stop events take the kernel's own
// begin and end times (events recorded around hipLaunchKernelGGL also count
// the dispatch, 2-4 us on the expert projection).  A null pointer, or null
// members, launch without events.
struct KernelEvents {
    hipEvent_t begin = nullptr, end = nullptr;
};

template <class F, class... Args>
inline void launch_timed(F kernel, dim3 grid, dim3 block, hipStream_t st, hipEvent_t begin, hipEvent_t end,
                         Args... args)
{
    if (begin || end)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, begin, end, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}
hipError_t launch_route(const float *logits, int T, int E, int K, int renorm, int32_t *ids,
                        float *w, hipStream_t stream);
// Routing then grouping of gp.T tokens (ids/w: the routing outputs, also gp.ids).
hipError_t launch_route_group(const float *logits, int renorm, int32_t *ids, float *w, const GroupParams &gp,
                              hipStream_t stream);
// mode: MOE_SPARSE, MOE_DENSE, kModeScore (gate scores a = SiLU(g) of every
// pair and neuron, written where h goes) or kModeMasked (the masks come from
// pmask and the scores from h's place; the gate is not read again)
constexpr int kModeScore = 3;
constexpr int kModeMasked = 4;
// MFMA workgroups (experts with >= nm pairs) run in the same launch for bf16
// layers with 256-thread GEMV workgroups, else in a second launch.
// ev (optional) times the launch or launches of this call.
hipError_t launch_proj(const Plan &pl, const ProjParams &pp, const MfmaParams &mp, int mode, hipStream_t stream,
                       const KernelEvents *ev = nullptr);
hipError_t launch_down(const Plan &pl, const DownParams &dp, const MfmaParams &mp, int mode, hipStream_t stream);
hipError_t launch_combine(const Plan &pl, const CombineParams &cp, hipStream_t stream);
hipError_t launch_select(const Plan &pl, const SelectParams &sp, float *tau_out, hipStream_t stream);
hipError_t launch_topk_select(const Plan &pl, const TopkParams &tp, hipStream_t stream);
hipError_t launch_proj_mfma(const Plan &pl, const MfmaParams &mp, int mode, hipStream_t stream,
                            hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr);
// The one-launch decode path and its combine; ev (optional) times the first
// launch.
hipError_t launch_fused(const Plan &pl, const FusedParams &fp, int mode, const KernelEvents *ev,
                        hipStream_t stream);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#if defined(__HIPCC__)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Loads of weight rows that a call streams once: nontemporal, so the caches do
// not keep them.  Whole 4 KiB rows read this way measured 6.8-7.0 TB/s on
// MI355X against 6.0-6.1 TB/s with ordinary loads (1 GiB, 512 to 4096
// workgroups of 256 threads).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4 *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream(const uint2 *p)
{
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 load_stream(const float4 *p)
{
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// bf16 weights/activations: 8 elements per 16-byte vector.
struct BF16 {
    using V = uint4;
    static constexpr int kEpl = 8;
    // acc + sum_i w_i * x_i over the 8 lanes of the vector (fp32 accumulate)
    static __device__ __forceinline__ float dot(V w, V x, float acc) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x),
                                              __builtin_bit_cast(bf16x2_t, x.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y),
                                              __builtin_bit_cast(bf16x2_t, x.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z),
                                              __builtin_bit_cast(bf16x2_t, x.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w),
                                              __builtin_bit_cast(bf16x2_t, x.w), acc, false);
        return acc;
    }
    static __device__ __forceinline__ void unpack(V w, float (&f)[8]) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(u[i] << 16);
            f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ V zero() { return make_uint4(0, 0, 0, 0); }
};

// fp32 weights/activations: 4 elements per 16-byte vector.
struct F32 {
    using V = float4;
    static constexpr int kEpl = 4;
    static __device__ __forceinline__ float dot(V w, V x, float acc) {
        acc = fmaf(w.x, x.x, acc);
        acc = fmaf(w.y, x.y, acc);
        acc = fmaf(w.z, x.z, acc);
        acc = fmaf(w.w, x.w, acc);
        return acc;
    }
    static __device__ __forceinline__ void unpack(V w, float (&f)[4]) {
        f[0] = w.x; f[1] = w.y; f[2] = w.z; f[3] = w.w;
    }
    static __device__ __forceinline__ V zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};

// SiLU(g) = g * sigmoid(g).  exp(-g) overflows to +inf for g < -88, giving
// g / inf = -0, the correct limit.
__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & (kWave - 1);
    return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}
#endif  // __HIPCC__

}  // namespace moe
