// Row streaming for the GEMV bodies: loads of whole neuron rows (each lane
// its 16-byte vectors of a row) and the transposed reduction of a batch of
// row-times-token dot products across the 64 lanes.  Shared by the expert
// projection and the single-launch decode path.
#pragma once

#include "moe_internal.h"
#include "wave_reduce.h"

namespace moe {

constexpr int kChunk = 32;  // rows per workgroup = bits per mask word

// Issue the loads of UR consecutive rows starting at row r (this lane's NSW
// vectors of each).  NT: nontemporal loads, for rows that no other workgroup of
// the call reads (ordinary loads leave them in the caches for workgroups of
// other pairs of the same expert).
template <class Tr, int UR, int NSW, bool NT = false>
__device__ __forceinline__ void load_rows(typename Tr::V (&buf)[UR][NSW], const typename Tr::V *W, int r,
                                          int rowV)
{
#pragma unroll
    for (int u = 0; u < UR; ++u)
#pragma unroll
        for (int k = 0; k < NSW; ++k) {
            const typename Tr::V *q = W + (size_t)(r + u) * rowV + k * kWave;
            buf[u][k] = NT ? load_stream(q) : *q;
        }
}

// Issue the loads of the next UR rows whose bits are set in `rest` (ascending),
// clearing those bits.  Past the last active row the loads repeat row `last`
// (the highest active row): every load is unconditional, since a load under a
// branch makes the compiler wait for all loads in flight where the paths
// join.  The extra rows' dot products land in slots that are never read.  NT as
// for load_rows.
template <class Tr, int UR, int NSW, bool NT = false>
__device__ __forceinline__ void load_active_rows(typename Tr::V (&buf)[UR][NSW], const typename Tr::V *W,
                                                 uint32_t &rest, int last, int rowV)
{
#pragma unroll
    for (int u = 0; u < UR; ++u) {
        const int r = rest ? __ffs(rest) - 1 : last;
        rest &= rest - 1;
#pragma unroll
        for (int k = 0; k < NSW; ++k) {
            const typename Tr::V *q = W + (size_t)r * rowV + k * kWave;
            buf[u][k] = NT ? load_stream(q) : *q;
        }
    }
}

// Partial dot products of UR rows with the TT tokens over this wavefront's
// columns, summed across the lanes by one transposed reduction; the lane that
// owns value (u, t) stores it at s_part[wave][slot0 + u][t].
template <class Tr, int UR, int NSW, int TT, int NW>
__device__ __forceinline__ void reduce_batch(const typename Tr::V (&buf)[UR][NSW],
                                             const typename Tr::V (&xr)[TT][NSW],
                                             float (&s_part)[NW][kChunk][TT], int wave, int slot0, int lane,
                                             int kidx, bool owner)
{
    constexpr int M = UR * TT;
    float v[M];
#pragma unroll
    for (int u = 0; u < UR; ++u)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < NSW; ++k) acc = Tr::dot(buf[u][k], xr[t][k], acc);
            v[u * TT + t] = acc;
        }
    const float part = xreduce<M>(v, lane);
    if (owner) s_part[wave][slot0 + kidx / TT][kidx % TT] = part;
}

}  // namespace moe
