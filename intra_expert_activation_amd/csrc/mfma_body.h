// The gathered projections as bf16 MFMA GEMMs, for experts whose token group
// is large enough (n_e >= the plan's threshold) to make them dense
// contractions: prefill batches, and the hot experts of a skewed router.
//
// gist.science page of arXiv 2605.08575, Technical Summary, Methodology:
// Fused Up-Down Projection gathers the active neurons' weights into a dense
// tile in on-chip memory and runs a dense product over them; Dynamic Switching
// picks a codepath by batch size.  Here the switch is per expert and only picks
// the kernel: the result is the same sparse function (the GEMV kernels and
// these agree to rounding).
//
// Tiles.  A work item is (expert, tile of 64 of its tokens); the projection
// takes them in pairs (two adjacent tiles of one expert, or its last alone).
//  k_proj_mfma  (item pair, 64-neuron tile): G = X W_gate^T and U = X W_up^T
//               over K = H together with v_mfma_f32_32x32x16_bf16 (4
//               wavefronts in 2x2, each 64 tokens x 32 rows of both), operands
//               staged through LDS in 64-wide K chunks with the next chunk's
//               global loads in flight; epilogue a = SiLU(g),
//               m = NOT(|a| < tau), mask words by ballot, each 64-token tile's
//               active rows (OR over its tokens) compacted in ascending order,
//               and h = m ? a*u : 0 of those rows stored compacted
//               [64 tokens][active rows] as a bf16 pair (hi + lo = h to
//               ~2^-17) so the down product keeps fp32-level accuracy.
//  k_down_mfma  (item, segment of the neuron tiles, 128-column tile):
//               O = sum over the segment's neuron tiles of
//               H_tile[64 x active] * W_down[active rows, 128 cols]; the
//               neuron-major down rows are staged row-major in LDS and read
//               transposed (ds_read_b64_tr_b16) as the MFMA B operand.  One
//               partial output per pair and segment; the plan uses one
//               segment unless few items leave the device short of
//               workgroups (a few wide experts).
// Work indices are remapped so that each XCD (8 per MI355X, each with its own
// L2) runs a contiguous range of the work units that exist.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTM = 64;                 // tokens per tile
constexpr int kTN = 64;                 // neurons per tile
constexpr int kKC = 64;                 // K chunk staged in LDS
constexpr int kRow = kKC + 8;           // padded LDS row (bf16 elements), 144 bytes
constexpr int kTC = kMfmaDownCols;      // output columns per down tile (128)

// Logical work index of workgroup b when nvalid work units exist (known on
// the device only), or -1.  Consecutive workgroups are dispatched round-robin
// over the 8 XCDs; XCD x takes the contiguous range [x * per, (x + 1) * per)
// of the valid units, so neighbouring units share its L2 and every XCD gets
// an equal share however many of the grid's workgroups have work.
__device__ __forceinline__ int xcd_remap(int b, int nvalid)
{
    const int per = (nvalid + 7) / 8;
    const int j = b >> 3;
    if (j >= per) return -1;
    const int L = (b & 7) * per + j;
    return L < nvalid ? L : -1;
}

__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t *row_base, int k)
{
    return *reinterpret_cast<const bf16x8_t *>(row_base + k);
}


__device__ __forceinline__ void gemm2_mma(f32x16_t (&acc)[2][2], uint16_t (*sX)[kRow], uint16_t (*sW)[kRow],
                                          uint16_t (*sU)[kRow], int wm, int wn, int lane)
{
#pragma unroll
    for (int s = 0; s < kKC / 16; ++s) {
        const int k = 16 * s + 8 * (lane >> 5);
        const bf16x8_t a0 = lds_frag(sX[64 * wm + (lane & 31)], k);
        const bf16x8_t a1 = lds_frag(sX[64 * wm + 32 + (lane & 31)], k);
        const bf16x8_t g = lds_frag(sW[32 * wn + (lane & 31)], k);
        const bf16x8_t u = lds_frag(sU[32 * wn + (lane & 31)], k);
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, g, acc[0][0], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, g, acc[1][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, u, acc[0][1], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, u, acc[1][1], 0, 0, 0);
    }
}

// Gate and up products of a 128-token x 64-row tile in one pass over K:
// acc[q][0] += X * Wg^T and acc[q][1] += X * Wu^T for this wavefront's 32
// tokens 64 wm + 32 q + ... and 32 rows 32 wn + ...  Rows past nrows load row 0
// and feed unused entries; token entries below 0 load token 0.  Each chunk of
// X is loaded once for both products; the next chunk is in flight in
// registers while the MFMAs read the current one in LDS (two chunks in flight
// need 32 more registers, and measured slower at 2 workgroups per CU than one
// at 3).
__device__ __forceinline__ void gemm2_128x64(f32x16_t (&acc)[2][2], uint16_t (*sX)[kRow], uint16_t (*sW)[kRow],
                                             uint16_t (*sU)[kRow], const uint16_t *X, const int *sTok,
                                             const uint16_t *Wg, const uint16_t *Wu, int nrows, int H)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int r = tid >> 3, c8 = tid & 7;  // rows r, r + 32, ... ; 16 bytes at column 8 c8
    const int t0 = sTok[r], t1 = sTok[r + 32], t2 = sTok[r + 64], t3 = sTok[r + 96];
    const uint16_t *xp0 = X + (size_t)(t0 >= 0 ? t0 : 0) * H + c8 * 8;
    const uint16_t *xp1 = X + (size_t)(t1 >= 0 ? t1 : 0) * H + c8 * 8;
    const uint16_t *xp2 = X + (size_t)(t2 >= 0 ? t2 : 0) * H + c8 * 8;
    const uint16_t *xp3 = X + (size_t)(t3 >= 0 ? t3 : 0) * H + c8 * 8;
    const int w0 = r < nrows ? r : 0, w1 = r + 32 < nrows ? r + 32 : 0;
    const uint16_t *gp0 = Wg + (size_t)w0 * H + c8 * 8;
    const uint16_t *gp1 = Wg + (size_t)w1 * H + c8 * 8;
    const uint16_t *up0 = Wu + (size_t)w0 * H + c8 * 8;
    const uint16_t *up1 = Wu + (size_t)w1 * H + c8 * 8;
    const int NC = H / kKC;
    // a chunk, per thread: X rows r + 32 i (i < 4), Wg and Wu rows r, r + 32
#define MOE_GEMM2_LOAD(V, c)                                                   \
    do {                                                                       \
        V##0 = *reinterpret_cast<const uint4 *>(xp0 + (c) * kKC);              \
        V##1 = *reinterpret_cast<const uint4 *>(xp1 + (c) * kKC);              \
        V##2 = *reinterpret_cast<const uint4 *>(xp2 + (c) * kKC);              \
        V##3 = *reinterpret_cast<const uint4 *>(xp3 + (c) * kKC);              \
        V##4 = *reinterpret_cast<const uint4 *>(gp0 + (c) * kKC);              \
        V##5 = *reinterpret_cast<const uint4 *>(gp1 + (c) * kKC);              \
        V##6 = *reinterpret_cast<const uint4 *>(up0 + (c) * kKC);              \
        V##7 = *reinterpret_cast<const uint4 *>(up1 + (c) * kKC);              \
    } while (0)
#define MOE_GEMM2_STORE(V)                                                     \
    do {                                                                       \
        *reinterpret_cast<uint4 *>(&sX[r][c8 * 8]) = V##0;                     \
        *reinterpret_cast<uint4 *>(&sX[r + 32][c8 * 8]) = V##1;                \
        *reinterpret_cast<uint4 *>(&sX[r + 64][c8 * 8]) = V##2;                \
        *reinterpret_cast<uint4 *>(&sX[r + 96][c8 * 8]) = V##3;                \
        *reinterpret_cast<uint4 *>(&sW[r][c8 * 8]) = V##4;                     \
        *reinterpret_cast<uint4 *>(&sW[r + 32][c8 * 8]) = V##5;                \
        *reinterpret_cast<uint4 *>(&sU[r][c8 * 8]) = V##6;                     \
        *reinterpret_cast<uint4 *>(&sU[r + 32][c8 * 8]) = V##7;                \
    } while (0)
    uint4 a0, a1, a2, a3, a4, a5, a6, a7;
    MOE_GEMM2_LOAD(a, 0);
#pragma unroll 1
    for (int c = 0; c < NC; ++c) {
        MOE_GEMM2_STORE(a);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        MOE_GEMM2_LOAD(a, min(c + 1, NC - 1));  // (the last chunk again at the end: unused)
        __builtin_amdgcn_sched_barrier(0);
        gemm2_mma(acc, sX, sW, sU, wm, wn, lane);
        __syncthreads();
    }
}
#undef MOE_GEMM2_LOAD
#undef MOE_GEMM2_STORE

// LDS of a projection workgroup: a pair of 64-token tiles x 64 rows.
struct MfmaProjLds {
    uint16_t sX[2 * kTM][kRow];
    uint16_t sW[kTN][kRow];
    uint16_t sU[kTN][kRow];
    uint32_t sMask[2 * kTM][2];
    uint32_t sAct[2][2];        // [token tile][word]
    int sTok[2 * kTM];
    int sList[2][kTN];
};

constexpr int kWdRow = kTC + 32;  // padded LDS row of the down tile (bf16): 320 bytes
constexpr int kDSeg = 32;         // neuron tiles whose lists are staged at a time

struct MfmaDownLds {
    uint16_t sHhi[kTM][kRow];
    uint16_t sHlo[kTM][kRow];
    uint16_t sWd[kTN][kWdRow];       // [active row][column], row-major as in memory
    uint8_t sList[kDSeg][kTN];       // active rows of the segment's neuron tiles
    int sNact[kDSeg];
    int s_wpre[4];
    int sRow[kTM];                   // output row (t * slots + slot) of each pair of the tile
};

typedef short bf16x4_bits_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_bits_t lds_bf16x4_t;

// B operand of v_mfma_f32_32x32x16_bf16 from a row-major [k][n] LDS tile
// (k = neuron, n = column): lane l needs B[8 (l / 32) + j][l % 32], j < 8.
// ds_read_b64_tr_b16 gives lane i of each 16-lane group element i % 4 of the
// 8-byte chunk addressed by lane 4 j + i / 4 of the group (measured on gfx950),
// so lane l = 16 g + i addresses row 8 (g / 2) + i / 4 (+ 4 for j = 4..7),
// column 16 (g % 2) + 4 (i % 4).  Rows 144 dwords apart put the 32 chunks
// of a half-wavefront on distinct LDS banks.
__device__ __forceinline__ bf16x8_t lds_frag_tr(const uint16_t *tile, int ld, int k0, int n0, int lane)
{
    const int g = lane >> 4, i = lane & 15;
    const uint16_t *p0 = tile + (size_t)(k0 + 8 * (g >> 1) + (i >> 2)) * ld + n0 + 16 * (g & 1) + 4 * (i & 3);
    const bf16x4_bits_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t *)p0);
    const bf16x4_bits_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t *)(p0 + 4 * ld));
    const bf16x4_bits_t v[2] = {lo, hi};
    return *reinterpret_cast<const bf16x8_t *>(v);
}

// Projection of one (item pair, 64-neuron tile): two adjacent 64-token tiles
// of one expert (or its last tile alone), so each weight tile read serves 128
// tokens.  `b` is this workgroup's index among the MFMA workgroups.  The gate
// and up products are computed together in one pass over the tokens' hidden
// states (up for every row of the tile: at 32 or more tokens the tile's union
// covers most rows, and a second pass over X for the active rows alone read
// more bytes than it skipped); h keeps the sparse definition, with an inactive
// (token, neuron) set to exactly 0 by a select, and only each 64-token tile's
// active rows are stored, compacted, for the down projection.  Work runs pair
// major: the neuron tiles of one pair next to each other on one XCD (sharing
// its hidden states in L2), then the expert's next pair (sharing the weight
// tiles).
template <int MODE>
__device__ __forceinline__ void mfma_proj_body(const MfmaParams &p, MfmaProjLds &S, int b)
{
    auto &sX = S.sX;
    auto &sW = S.sW;
    auto &sU = S.sU;
    auto &sMask = S.sMask;
    auto &sAct = S.sAct;
    auto &sTok = S.sTok;
    auto &sList = S.sList;

    const int L = xcd_remap(b, p.hdr[2] * p.NT);
    if (L < 0) return;
    const int pi = L / p.NT, nt = L - pi * p.NT;
    const int pcode = p.pairs[pi];
    const int item0 = pcode >> 1, nblk = 1 + (pcode & 1);  // token tiles in the pair
    const int code = p.items[item0];
    const int xe = code >> 16, tile = code & 0xffff;
    const bool shared = xe >= p.E;
    const int Ie = shared ? p.Is : p.I;
    const int n0 = nt * kTN;
    if (n0 >= Ie) return;
    const int nrows = min(kTN, Ie - n0);  // 32 or 64
    const int n = p.counts[xe], off = p.offsets[xe];
    const int m0 = tile * kTM, mt = min(nblk * kTM, n - m0);  // valid tokens of the pair
    const int H = p.H;
    const size_t mat = (size_t)(shared ? xe - p.E : xe) * Ie * H;
    const uint16_t *Wg = (shared ? p.swg : p.wg) + mat + (size_t)n0 * H;
    const uint16_t *Wu = (shared ? p.swu : p.wu) + mat + (size_t)n0 * H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;  // wm: token tile of the pair
    const float tau = (MODE == MOE_SPARSE) ? p.tau[xe] : 0.f;

    if (tid < 2 * kTM) {
        sTok[tid] = tid < mt ? p.pair_tok[off + m0 + tid] : -1;
        sMask[tid][0] = sMask[tid][1] = 0u;
    }
    if (tid < 4) sAct[tid >> 1][tid & 1] = 0u;
    __syncthreads();

    // ---- gate and up ----------------------------------------------------------
    f32x16_t acc[2][2] = {};
    gemm2_128x64(acc, sX, sW, sU, p.x, sTok, Wg, Wu, nrows, H);

    // acc[q][*] entry r of this lane: token m = 64 wm + 32 q + 8 (r / 4) +
    // 4 (lane / 32) + r % 4 of the pair, row nn = 32 wn + lane % 32
    const int nn = 32 * wn + (lane & 31);
    uint32_t actw = 0, mine[2] = {0u, 0u};  // mine[q]: bit r = this lane's entry is active
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int mlo = 64 * wm + 32 * q + 8 * (r >> 2) + (r & 3);  // lanes 32..63 hold mlo + 4
            const int m = mlo + 4 * (lane >> 5);
            const float a = silu(acc[q][0][r]);
            const bool valid = m < mt && nn < nrows;
            const bool act = valid && (MODE == MOE_DENSE || !(fabsf(a) < tau));
            acc[q][0][r] = a;
            mine[q] |= (uint32_t)act << r;
            const uint64_t bb = __ballot(act);
            if (lane == 0) {
                sMask[mlo][wn] = (uint32_t)bb;
                sMask[mlo + 4][wn] = (uint32_t)(bb >> 32);
            }
            actw |= (uint32_t)bb | (uint32_t)(bb >> 32);
        }
    if (lane == 0 && actw) atomicOr(&sAct[wm][wn], actw);
    __syncthreads();

    // ---- masks, union, active rows of each token tile -------------------------
    if (p.mask_bits) {
        const int m = tid >> 1, w = tid & 1;  // tid < 256 = 2 x 128
        if (m < mt && 32 * w < nrows) {
            const int pr = off + m0 + m;
            const size_t row = (size_t)p.pair_tok[pr] * p.slots + p.pair_slot[pr];
            p.mask_bits[row * p.W + (n0 >> 5) + w] = sMask[m][w];
        }
        if (nt == 0 && tid < mt) {
            const int pr = off + m0 + tid;
            const size_t row = (size_t)p.pair_tok[pr] * p.slots + p.pair_slot[pr];
            for (int wd = Ie / 32; wd < p.W; ++wd) p.mask_bits[row * p.W + wd] = 0u;
        }
    }
    if (tid == 0) {
        const uint32_t u0 = sAct[0][0] | sAct[1][0], u1 = sAct[0][1] | sAct[1][1];
        if (u0) atomicOr(&p.union_words[(size_t)xe * p.W + (n0 >> 5)], u0);
        if (nrows > 32 && u1) atomicOr(&p.union_words[(size_t)xe * p.W + (n0 >> 5) + 1], u1);
    }
    if (wave < nblk) {  // wavefront j lists token tile j's active rows
        const uint64_t a64 = (uint64_t)sAct[wave][0] | ((uint64_t)sAct[wave][1] << 32);
        if ((a64 >> lane) & 1ull) sList[wave][__popcll(a64 & lanemask_lt())] = lane;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (j >= nblk) break;
        const int blk = (item0 + j) * p.NT + nt;
        const int na = __popc(sAct[j][0]) + __popc(sAct[j][1]);
        if (tid == 0) p.nact[blk] = na;
        if (tid < na) p.list[(size_t)blk * kTN + tid] = (uint8_t)sList[j][tid];
    }
    if (wm >= nblk) return;  // (no second token tile)

    // ---- h of token tile wm's active rows, compacted ---------------------------
    // active row nn goes to column (its rank among the tile's active rows,
    // < nact); the lane of row nn >= nact also zeroes column nn, so every
    // column of the block is written (the down product reads zeros past nact)
    const uint64_t act64 = (uint64_t)sAct[wm][0] | ((uint64_t)sAct[wm][1] << 32);
    const int nact = __popcll(act64);
    if (nact == 0) return;
    const bool row_act = (act64 >> nn) & 1ull;
    const int col = __popcll(act64 & ((1ull << nn) - 1ull));
    const int blk = (item0 + wm) * p.NT + nt;
    uint16_t *hhi = p.hhi + (size_t)blk * kTM * kTN;
    uint16_t *hlo = p.hlo + (size_t)blk * kTM * kTN;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 32 * q + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);  // token within the tile
            if (row_act) {
                const float hv = ((mine[q] >> r) & 1u) ? acc[q][0][r] * acc[q][1][r] : 0.f;  // a select
                const uint16_t hi = bf16_rne(hv);
                hhi[m * kTN + col] = hi;
                hlo[m * kTN + col] = bf16_rne(hv - bf16_to_f32(hi));
            }
            if (nn >= nact) {
                hhi[m * kTN + nn] = 0;
                hlo[m * kTN + nn] = 0;
            }
        }
}

// Down projection of one (item, 128-column tile): O = sum over the expert's
// neuron tiles of H_tile[64 tokens x active rows] * W_down[active rows, 128
// columns], hi and lo halves of H each through the MFMA.  The active rows'
// down weights are staged row-major (16-byte stores) and read transposed by
// ds_read_b64_tr_b16; the next active tile's h and weights are loaded while
// the current one is multiplied.  Loads past the tile's active rows repeat its
// last active row, and h columns past them are zero: every load is
// unconditional.
template <int MODE>
__device__ __forceinline__ void mfma_down_body(const MfmaParams &p, MfmaDownLds &S, int b)
{
    auto &sHhi = S.sHhi;
    auto &sHlo = S.sHlo;
    auto &sWd = S.sWd;
    auto &sList = S.sList;
    auto &sNact = S.sNact;
    auto &s_wpre = S.s_wpre;

    const int nct = p.H / kTC;
    const int nitems = p.hdr[1];
    const int L = xcd_remap(b, nitems * p.NKS * nct);
    if (L < 0) return;
    // item-major, then segment: the h tiles of an (item, segment) stay in L2
    // across its column tiles
    const int item = L / (p.NKS * nct);
    const int ks = (L - item * p.NKS * nct) / nct;
    const int ct = L - (item * p.NKS + ks) * nct;
    const int code = p.items[item];
    const int xe = code >> 16, tile = code & 0xffff;
    const bool shared = xe >= p.E;
    const int Ie = shared ? p.Is : p.I;
    const int n = p.counts[xe], off = p.offsets[xe];
    const int m0 = tile * kTM, mt = min(kTM, n - m0);
    const int H = p.H, c0 = ct * kTC;
    const uint16_t *Wd = (shared ? p.swd : p.wd) + (size_t)(shared ? xe - p.E : xe) * Ie * H + c0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int NTe = (Ie + kTN - 1) / kTN;
    // this workgroup's segment of the neuron tiles: [ts0, ts1)
    const int per = (NTe + p.NKS - 1) / p.NKS;
    const int ts0 = min(NTe, ks * per), ts1 = min(NTe, ts0 + per);
    // this thread's pieces: h rows tid / 8 and 32 + tid / 8 (16 bytes at
    // column 8 (tid % 8)); down rows tid / 16 + 16 i (16 bytes at column
    // 8 (tid % 16)), i < 4
    const int hr = tid >> 3, hc = (tid & 7) * 8;
    const int wr = tid >> 4, wc = (tid & 15) * 8;

    if (tid < kTM) {
        const int pr = off + m0 + min(tid, mt - 1);
        S.sRow[tid] = p.pair_tok[pr] * p.slots + p.pair_slot[pr];
    }
    f32x16_t acc[2] = {};
    for (int seg = ts0; seg < ts1; seg += kDSeg) {
        const int ns = min(kDSeg, ts1 - seg);
        __syncthreads();  // the previous segment's lists are no longer read
        for (int q = tid; q < ns * kTN; q += 256) {
            const int t = q / kTN, c = q - t * kTN;
            sList[t][c] = p.list[(size_t)(item * p.NT + seg + t) * kTN + c];
        }
        if (tid < ns) sNact[tid] = p.nact[item * p.NT + seg + tid];
        __syncthreads();
        // active tiles of the segment, in order
        auto next_active = [&](int t) {
            for (; t < ns; ++t)
                if (sNact[t] > 0) return t;
            return -1;
        };
        int cur = __builtin_amdgcn_readfirstlane(next_active(0));
        if (cur < 0) continue;
        uint4 hh0, hh1, hl0, hl1, w0, w1, w2, w3;
        auto issue = [&](int t) {
            const int blk = item * p.NT + seg + t;
            const int na = sNact[t];
            const uint16_t *hhi = p.hhi + (size_t)blk * kTM * kTN;
            const uint16_t *hlo = p.hlo + (size_t)blk * kTM * kTN;
            hh0 = *reinterpret_cast<const uint4 *>(hhi + hr * kTN + hc);
            hh1 = *reinterpret_cast<const uint4 *>(hhi + (hr + 32) * kTN + hc);
            hl0 = *reinterpret_cast<const uint4 *>(hlo + hr * kTN + hc);
            hl1 = *reinterpret_cast<const uint4 *>(hlo + (hr + 32) * kTN + hc);
            const uint16_t *wt = Wd + (size_t)((seg + t) * kTN) * H + wc;
            w0 = *reinterpret_cast<const uint4 *>(wt + (size_t)sList[t][min(wr, na - 1)] * H);
            w1 = *reinterpret_cast<const uint4 *>(wt + (size_t)sList[t][min(wr + 16, na - 1)] * H);
            w2 = *reinterpret_cast<const uint4 *>(wt + (size_t)sList[t][min(wr + 32, na - 1)] * H);
            w3 = *reinterpret_cast<const uint4 *>(wt + (size_t)sList[t][min(wr + 48, na - 1)] * H);
        };
        issue(cur);
        while (cur >= 0) {
            const int kp = (__builtin_amdgcn_readfirstlane(sNact[cur]) + 15) & ~15;
            *reinterpret_cast<uint4 *>(&sHhi[hr][hc]) = hh0;
            *reinterpret_cast<uint4 *>(&sHhi[hr + 32][hc]) = hh1;
            *reinterpret_cast<uint4 *>(&sHlo[hr][hc]) = hl0;
            *reinterpret_cast<uint4 *>(&sHlo[hr + 32][hc]) = hl1;
            *reinterpret_cast<uint4 *>(&sWd[wr][wc]) = w0;
            *reinterpret_cast<uint4 *>(&sWd[wr + 16][wc]) = w1;
            *reinterpret_cast<uint4 *>(&sWd[wr + 32][wc]) = w2;
            *reinterpret_cast<uint4 *>(&sWd[wr + 48][wc]) = w3;
            __syncthreads();
            const int nxt = __builtin_amdgcn_readfirstlane(next_active(cur + 1));
            if (nxt >= 0) issue(nxt);
            __builtin_amdgcn_sched_barrier(0);
            for (int s = 0; s < kp / 16; ++s) {
                const int k = 16 * s + 8 * (lane >> 5);
                const bf16x8_t ahi = lds_frag(sHhi[32 * wm + (lane & 31)], k);
                const bf16x8_t alo = lds_frag(sHlo[32 * wm + (lane & 31)], k);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const bf16x8_t bv = lds_frag_tr(&sWd[0][0], kWdRow, 16 * s, 64 * wn + 32 * nb, lane);
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bv, acc[nb], 0, 0, 0);
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bv, acc[nb], 0, 0, 0);
                }
            }
            __syncthreads();
            cur = nxt;
        }
    }
    // segment 0 at the pair's (token, slot) row, segment k >= 1 at row
    // mbase + (k - 1) P + (token, slot) row
    const size_t rbase = ks == 0 ? 0 : p.mbase + (size_t)(ks - 1) * p.P;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int col = c0 + 64 * wn + 32 * nb + (lane & 31);
            if (m < mt) p.partial[(rbase + S.sRow[m]) * H + col] = acc[nb][r];
        }
    // NKS pieces per pair and 1024-column tile (recorded by the first
    // segment's first 128-column tile)
    if (ks == 0 && c0 % 1024 == 0 && tid < mt) p.npc[(size_t)S.sRow[tid] * p.NCT + c0 / 1024] = p.NKS;

    // the expert's union list (complete: every projection tile has finished)
    if (tile == 0 && ct == 0 && ks == 0 && (p.union_idx || p.union_cnt)) {
        const int nw = Ie / 32;
        const uint32_t *uw = p.union_words + (size_t)xe * p.W;
        const int per = (nw + 255) / 256;
        const int wb = tid * per;
        int cnt = 0;
        for (int i = 0; i < per; ++i)
            if (wb + i < nw) cnt += __popc(uw[wb + i]);
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d, 64);
            if (lane >= d) incl += o;
        }
        if (lane == 63) s_wpre[wave] = incl;
        __syncthreads();
        int pos = incl - cnt;
        for (int i = 0; i < wave; ++i) pos += s_wpre[i];
        if (p.union_idx)
            for (int i = 0; i < per; ++i) {
                const int wd = wb + i;
                if (wd >= nw) break;
                uint32_t bits = uw[wd];
                while (bits) {
                    const int b = __ffs(bits) - 1;
                    bits &= bits - 1;
                    p.union_idx[(size_t)xe * p.Imax + pos++] = wd * 32 + b;
                }
            }
        if (p.union_cnt && tid == 0) p.union_cnt[xe] = s_wpre[0] + s_wpre[1] + s_wpre[2] + s_wpre[3];
    }
}

}  // namespace moe
