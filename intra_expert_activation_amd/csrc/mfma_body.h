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
// Tiles.  A work item is (expert, tile of 64 of its tokens).
//  k_proj_mfma  (item, 64-neuron tile): G = X W_gate^T over K = H with
//               v_mfma_f32_32x32x16_bf16 (4 wavefronts in 2x2, 32x32 each),
//               operands staged through LDS in 64-wide K chunks with the next
//               chunk's global loads in flight; epilogue a = SiLU(g),
//               m = NOT(|a| < tau), mask words by ballot, the tile's active
//               rows (OR over its tokens) compacted in ascending order; then
//               U = X W_up[active]^T over the active rows only, and
//               h = m ? a*u : 0 stored compacted [64 tokens][active rows] as a
//               bf16 pair (hi + lo, hi + lo = h to ~2^-17) so the down product
//               keeps fp32-level accuracy.
//  k_down_mfma  (item, 128-column tile): O = sum over neuron tiles of
//               H_tile[64 x active] * W_down[active rows, 128 cols]; the
//               neuron-major down rows are transposed into LDS (k-contiguous)
//               for the MFMA B operand.  One output per pair (no split).
// Work indices are remapped so that each XCD (8 per MI355X, each with its own
// L2) runs a contiguous range: the token tiles of one expert, which read the
// same weight rows, then share that L2.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTM = 64;                 // tokens per tile
constexpr int kTN = 64;                 // neurons per tile
constexpr int kKC = 64;                 // K chunk staged in LDS
constexpr int kRow = kKC + 8;           // padded LDS row (bf16 elements), 144 bytes
constexpr int kTC = 128;                // output columns per down tile

__device__ __forceinline__ int xcd_remap(int b, int nblocks)
{
    // consecutive workgroups are dispatched round-robin over the 8 XCDs; give
    // XCD x the logical range [x*per, (x+1)*per) (nblocks is a multiple of 8)
    const int per = nblocks / 8;
    return (b % 8) * per + b / 8;
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

// One 64 x 64 x H product C += X[rows sTok] * W[rows given by wrow(r)]^T with the
// 2x2 wavefront layout; `active` gates the MFMAs of this wavefront (all
// wavefronts always load, store and synchronise).
template <class WRow>
__device__ __forceinline__ void gemm_64x64(f32x16_t &acc, uint16_t (*sX)[kRow], uint16_t (*sW)[kRow],
                                           const uint16_t *X, const int *sTok, const uint16_t *W, WRow wrow,
                                           int H, bool active)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    uint4 xr[2], wr[2];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int piece = tid + 256 * i, r = piece >> 3, c8 = piece & 7;
            const int tok = sTok[r];
            xr[i] = tok >= 0 ? *reinterpret_cast<const uint4 *>(X + (size_t)tok * H + k0 + c8 * 8)
                             : make_uint4(0, 0, 0, 0);
            const int row = wrow(r);
            wr[i] = row >= 0 ? *reinterpret_cast<const uint4 *>(W + (size_t)row * H + k0 + c8 * 8)
                             : make_uint4(0, 0, 0, 0);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int piece = tid + 256 * i, r = piece >> 3, c8 = piece & 7;
            *reinterpret_cast<uint4 *>(&sX[r][c8 * 8]) = xr[i];
            *reinterpret_cast<uint4 *>(&sW[r][c8 * 8]) = wr[i];
        }
    };
    load(0);
    store();
    __syncthreads();
    for (int k0 = 0; k0 < H; k0 += kKC) {
        const bool more = k0 + kKC < H;
        if (more) load(k0 + kKC);
        if (active) {
#pragma unroll
            for (int s = 0; s < kKC / 16; ++s) {
                const int k = 16 * s + 8 * (lane >> 5);
                const bf16x8_t a = lds_frag(sX[32 * wm + (lane & 31)], k);
                const bf16x8_t b = lds_frag(sW[32 * wn + (lane & 31)], k);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
            }
        }
        __syncthreads();
        if (more) {
            store();
            __syncthreads();
        }
    }
}

struct MfmaProjLds {
    uint16_t sX[kTM][kRow];
    uint16_t sW[kTN][kRow];
    float sA[kTM][kTN + 1];
    uint32_t sMask[kTM][2];
    uint32_t sAct[2];
    int sTok[kTM];
    int sList[kTN];
    int sNact;
};

struct MfmaDownLds {
    uint16_t sHhi[kTM][kRow];
    uint16_t sHlo[kTM][kRow];
    uint16_t sWt[kTC][kRow];  // [column][active row]
    int sList[kTN];
    int s_wpre[4];
};

// Projection of one (item, 64-neuron tile); `b` and `nblocks` are this
// workgroup's index among the MFMA workgroups and their count (a multiple of 8).
template <int MODE>
__device__ __forceinline__ void mfma_proj_body(const MfmaParams &p, MfmaProjLds &S, int b, int nblocks)
{
    auto &sX = S.sX;
    auto &sW = S.sW;
    auto &sA = S.sA;
    auto &sMask = S.sMask;
    auto &sAct = S.sAct;
    auto &sTok = S.sTok;
    auto &sList = S.sList;
    auto &sNact = S.sNact;

    const int L = xcd_remap(b, nblocks);
    if (L >= p.max_items * p.NT) return;
    const int nt = L / p.max_items, item = L - nt * p.max_items;
    if (item >= p.hdr[1]) return;
    const int code = p.items[item];
    const int xe = code >> 16, tile = code & 0xffff;
    const bool shared = xe >= p.E;
    const int Ie = shared ? p.Is : p.I;
    const int n0 = nt * kTN;
    if (n0 >= Ie) return;
    const int nrows = min(kTN, Ie - n0);  // 32 or 64
    const int n = p.counts[xe], off = p.offsets[xe];
    const int m0 = tile * kTM, mt = min(kTM, n - m0);
    const int H = p.H;
    const size_t mat = (size_t)(shared ? xe - p.E : xe) * Ie * H;
    const uint16_t *Wg = (shared ? p.swg : p.wg) + mat + (size_t)n0 * H;
    const uint16_t *Wu = (shared ? p.swu : p.wu) + mat + (size_t)n0 * H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const float tau = (MODE == MOE_SPARSE) ? p.tau[xe] : 0.f;

    if (tid < kTM) sTok[tid] = tid < mt ? p.pair_tok[off + m0 + tid] : -1;
    if (tid < 2) sAct[tid] = 0u;
    if (tid < 2 * kTM) sMask[tid >> 1][tid & 1] = 0u;
    __syncthreads();

    // ---- gate ---------------------------------------------------------------
    f32x16_t acc = {};
    gemm_64x64(acc, sX, sW, p.x, sTok, Wg, [&](int r) { return r < nrows ? r : -1; }, H, true);

    uint32_t actw = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int mlo = 32 * wm + 8 * (r >> 2) + (r & 3);  // token of lanes 0..31; lanes 32..63 hold mlo + 4
        const int m = mlo + 4 * (lane >> 5);
        const int nn = 32 * wn + (lane & 31);
        const float a = silu(acc[r]);
        const bool valid = m < mt && nn < nrows;
        const bool act = valid && (MODE == MOE_DENSE || !(fabsf(a) < tau));
        sA[m][nn] = a;
        const uint64_t b = __ballot(act);
        if (lane == 0) {
            sMask[mlo][wn] = (uint32_t)b;
            sMask[mlo + 4][wn] = (uint32_t)(b >> 32);
        }
        actw |= (uint32_t)b | (uint32_t)(b >> 32);
    }
    if (lane == 0 && actw) atomicOr(&sAct[wn], actw);
    __syncthreads();

    // ---- masks, union, active rows ------------------------------------------
    const int blk = item * p.NT + nt;
    if (p.mask_bits && tid < 2 * kTM) {
        const int m = tid >> 1, w = tid & 1;
        if (m < mt && 32 * w < nrows) {
            const int pr = off + m0 + m;
            const size_t row = (size_t)p.pair_tok[pr] * p.slots + p.pair_slot[pr];
            p.mask_bits[row * p.W + (n0 >> 5) + w] = sMask[m][w];
        }
    }
    if (p.mask_bits && nt == 0 && tid < kTM && tid < mt) {
        const int pr = off + m0 + tid;
        const size_t row = (size_t)p.pair_tok[pr] * p.slots + p.pair_slot[pr];
        for (int wd = Ie / 32; wd < p.W; ++wd) p.mask_bits[row * p.W + wd] = 0u;
    }
    if (tid == 0) {
        if (sAct[0]) atomicOr(&p.union_words[(size_t)xe * p.W + (n0 >> 5)], sAct[0]);
        if (nrows > 32 && sAct[1]) atomicOr(&p.union_words[(size_t)xe * p.W + (n0 >> 5) + 1], sAct[1]);
    }
    if (wave == 0) {
        const uint64_t act64 = (uint64_t)sAct[0] | ((uint64_t)sAct[1] << 32);
        const bool bit = (act64 >> lane) & 1ull;
        const uint64_t b = __ballot(bit);
        if (bit) sList[__popcll(b & lanemask_lt())] = lane;
        if (lane == 0) sNact = __popcll(b);
    }
    __syncthreads();
    const int nact = sNact;
    if (tid == 0) p.nact[blk] = nact;
    if (tid < nact) p.list[(size_t)blk * kTN + tid] = (uint8_t)sList[tid];
    if (nact == 0) return;

    // ---- up, over the active rows only ---------------------------------------
    const int nup = nact <= 32 ? 32 : 64;
    f32x16_t accu = {};
    gemm_64x64(accu, sX, sW, p.x, sTok, Wu, [&](int r) { return r < nact ? sList[r] : -1; }, H,
               32 * wn < nup);
    if (32 * wn < nup) {
        uint16_t *hhi = p.hhi + (size_t)blk * kTM * kTN;
        uint16_t *hlo = p.hlo + (size_t)blk * kTM * kTN;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int c = 32 * wn + (lane & 31);
            float hv = 0.f;
            if (c < nact && m < mt) {
                const int j = sList[c];
                const bool mb = (sMask[m][j >> 5] >> (j & 31)) & 1u;
                hv = mb ? sA[m][j] * accu[r] : 0.f;  // a select: inactive neurons add exactly 0
            }
            const uint16_t hi = bf16_rne(hv);
            hhi[m * kTN + c] = hi;
            hlo[m * kTN + c] = bf16_rne(hv - bf16_to_f32(hi));
        }
    }
}

// Down projection of one (item, 128-column tile).
template <int MODE>
__device__ __forceinline__ void mfma_down_body(const MfmaParams &p, MfmaDownLds &S, int b, int nblocks)
{
    auto &sHhi = S.sHhi;
    auto &sHlo = S.sHlo;
    auto &sWt = S.sWt;
    auto &sList = S.sList;
    auto &s_wpre = S.s_wpre;

    const int NCT = p.H / kTC;
    const int L = xcd_remap(b, nblocks);
    if (L >= p.max_items * NCT) return;
    const int ct = L / p.max_items, item = L - ct * p.max_items;
    if (item >= p.hdr[1]) return;
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

    f32x16_t acc[2] = {};
    for (int nt = 0; nt < NTe; ++nt) {
        const int blk = item * p.NT + nt;
        const int nact = p.nact[blk];
        if (nact == 0) continue;
        const int kp = (nact + 15) & ~15;
        const uint16_t *hhi = p.hhi + (size_t)blk * kTM * kTN;
        const uint16_t *hlo = p.hlo + (size_t)blk * kTM * kTN;
        const int pieces_h = kTM * (kp / 8);
        for (int q = tid; q < pieces_h; q += 256) {
            const int r = q / (kp / 8), c8 = q - r * (kp / 8);
            *reinterpret_cast<uint4 *>(&sHhi[r][c8 * 8]) = *reinterpret_cast<const uint4 *>(hhi + r * kTN + c8 * 8);
            *reinterpret_cast<uint4 *>(&sHlo[r][c8 * 8]) = *reinterpret_cast<const uint4 *>(hlo + r * kTN + c8 * 8);
        }
        if (tid < kTN) sList[tid] = tid < nact ? (int)p.list[(size_t)blk * kTN + tid] : 0;
        __syncthreads();
        // active down rows, transposed into [column][row]
        for (int q = tid; q < kp * (kTC / 8); q += 256) {
            const int c = q / (kTC / 8), c8 = q - c * (kTC / 8);
            const uint4 v = c < nact ? *reinterpret_cast<const uint4 *>(Wd + (size_t)(nt * kTN + sList[c]) * H + c8 * 8)
                                     : make_uint4(0, 0, 0, 0);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sWt[c8 * 8 + 2 * i][c] = (uint16_t)(w4[i] & 0xffffu);
                sWt[c8 * 8 + 2 * i + 1][c] = (uint16_t)(w4[i] >> 16);
            }
        }
        __syncthreads();
        for (int s = 0; s < kp / 16; ++s) {
            const int k = 16 * s + 8 * (lane >> 5);
            const bf16x8_t ahi = lds_frag(sHhi[32 * wm + (lane & 31)], k);
            const bf16x8_t alo = lds_frag(sHlo[32 * wm + (lane & 31)], k);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const bf16x8_t b = lds_frag(sWt[64 * wn + 32 * nb + (lane & 31)], k);
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, b, acc[nb], 0, 0, 0);
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, b, acc[nb], 0, 0, 0);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int col = c0 + 64 * wn + 32 * nb + (lane & 31);
            if (m < mt) p.partial[(size_t)(off + m0 + m) * H + col] = acc[nb][r];
        }

    // the expert's union list (complete: every projection tile has finished)
    if (tile == 0 && ct == 0 && (p.union_idx || p.union_cnt)) {
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
