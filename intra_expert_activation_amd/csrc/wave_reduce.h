// Cross-lane reductions for gfx950 wavefronts (64 lanes).
//
// xreduce<M>(v) sums M per-lane values over all 64 lanes at once
// ("transposed" reduction).  Each halving stage pairs the registers two by two
// and keeps one of each pair per half-wavefront, so the register count halves
// while the lane group holding a value halves too:
//   lane bit 5  v_permlane32_swap (upper half of a <-> lower half of b)
//   lane bit 4  v_permlane16_swap (odd rows of a <-> even rows of b)
//   lane bits 3,2,1,0  DPP row_mirror, row_half_mirror, quad_perm xor 2, xor 1
// After log2(M) halving stages one register remains; the remaining lane bits
// are summed in place.  Lane L then holds the full sum of value index
//   k(L) = sum_{s < log2 M} ((L >> (5 - s)) & 1) << s,
// and every lane whose bits below (6 - log2 M) differ holds the same value.
// Cost for M = 32: 31 swaps/DPP moves and 31 adds, against 32 x 12 for a
// shuffle-based reduction per value.
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

__device__ __forceinline__ void permlane32_swap(float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

__device__ __forceinline__ void permlane16_swap(float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within 16
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppXor2 = 0x4e;            // quad_perm [2,3,0,1]
constexpr int kDppXor1 = 0xb1;            // quad_perm [1,0,3,2]

// One halving stage over lane bit B: pairs (v[2i], v[2i+1]) -> v[i].
template <int B, int M>
__device__ __forceinline__ void halve(float (&v)[M], int lane)
{
#pragma unroll
    for (int i = 0; i < M / 2; ++i) {
        float a = v[2 * i], b = v[2 * i + 1];
        if constexpr (B == 5) {
            permlane32_swap(a, b);
            v[i] = a + b;
        } else if constexpr (B == 4) {
            permlane16_swap(a, b);
            v[i] = a + b;
        } else {
            constexpr int C = B == 3 ? kDppRowMirror : B == 2 ? kDppRowHalfMirror : B == 1 ? kDppXor2 : kDppXor1;
            const bool hi = (lane >> B) & 1;
            const float keep = hi ? b : a;
            const float give = hi ? a : b;
            v[i] = keep + dpp_mov<C>(give);
        }
    }
}

// Sum of one register over lane bit B, result in every lane.
template <int B>
__device__ __forceinline__ float fold(float x)
{
    if constexpr (B == 5) {
        float a = x, b = x;
        permlane32_swap(a, b);
        return a + b;
    } else if constexpr (B == 4) {
        float a = x, b = x;
        permlane16_swap(a, b);
        return a + b;
    } else {
        constexpr int C = B == 3 ? kDppRowMirror : B == 2 ? kDppRowHalfMirror : B == 1 ? kDppXor2 : kDppXor1;
        return x + dpp_mov<C>(x);
    }
}

template <int M>
__device__ __forceinline__ float xreduce(float (&v)[M], int lane)
{
    static_assert(M >= 1 && M <= 64 && (M & (M - 1)) == 0, "M must be a power of two <= 64");
    if constexpr (M >= 2) halve<5>(v, lane);
    if constexpr (M >= 4) halve<4>(*reinterpret_cast<float(*)[M / 2]>(&v), lane);
    if constexpr (M >= 8) halve<3>(*reinterpret_cast<float(*)[M / 4]>(&v), lane);
    if constexpr (M >= 16) halve<2>(*reinterpret_cast<float(*)[M / 8]>(&v), lane);
    if constexpr (M >= 32) halve<1>(*reinterpret_cast<float(*)[M / 16]>(&v), lane);
    if constexpr (M >= 64) halve<0>(*reinterpret_cast<float(*)[M / 32]>(&v), lane);
    float r = v[0];
    if constexpr (M < 2) r = fold<5>(r);
    if constexpr (M < 4) r = fold<4>(r);
    if constexpr (M < 8) r = fold<3>(r);
    if constexpr (M < 16) r = fold<2>(r);
    if constexpr (M < 32) r = fold<1>(r);
    if constexpr (M < 64) r = fold<0>(r);
    return r;
}

// Value index held by lane L after xreduce<M>.
template <int M>
__device__ __forceinline__ int xreduce_index(int lane)
{
    int k = 0;
#pragma unroll
    for (int s = 0; (1 << s) < M; ++s) k |= ((lane >> (5 - s)) & 1) << s;
    return k;
}

// Lanes that hold a distinct value index (one writer per index).
template <int M>
__device__ __forceinline__ bool xreduce_owner(int lane)
{
    constexpr int low_bits = 6 - (M == 1 ? 0 : M == 2 ? 1 : M == 4 ? 2 : M == 8 ? 3 : M == 16 ? 4 : M == 32 ? 5 : 6);
    return (lane & ((1 << low_bits) - 1)) == 0;
}


// Wavefront-wide max / min of one value, result in every lane (same stages as
// fold: permlane swaps for lane bits 5 and 4, DPP for bits 3..0).
template <int B, class Op>
__device__ __forceinline__ uint32_t fold_bits(uint32_t x, Op op)
{
    if constexpr (B == 5) {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return op(r[0], r[1]);
    } else if constexpr (B == 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return op(r[0], r[1]);
    } else {
        constexpr int C = B == 3 ? kDppRowMirror : B == 2 ? kDppRowHalfMirror : B == 1 ? kDppXor2 : kDppXor1;
        return op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, C, 0xf, 0xf, false));
    }
}

template <class Op>
__device__ __forceinline__ uint32_t wave_fold(uint32_t x, Op op)
{
    x = fold_bits<0>(x, op);
    x = fold_bits<1>(x, op);
    x = fold_bits<2>(x, op);
    x = fold_bits<3>(x, op);
    x = fold_bits<4>(x, op);
    x = fold_bits<5>(x, op);
    return x;
}

__device__ __forceinline__ float wave_max(float v)
{
    return __uint_as_float(wave_fold(__float_as_uint(v), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
}

__device__ __forceinline__ int wave_min(int v)
{
    return (int)wave_fold((uint32_t)v, [](uint32_t a, uint32_t b) { return (int)a < (int)b ? a : b; });
}

__device__ __forceinline__ float wave_sum_all(float v)
{
    return __uint_as_float(wave_fold(__float_as_uint(v), [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}

// Inclusive prefix sum over the 64 lanes: DPP row shifts within each row of
// 16 lanes (out-of-row sources read 0), then row broadcasts of lanes 15 and
// 31 into the rows after them.
__device__ __forceinline__ int wave_incl_scan_dpp(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false); // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false); // row_bcast:31 into rows 2, 3
    return x;
}

}  // namespace moe
