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
//  down body   (item, segment of the neuron tiles, 128-column tile), in the
//               merged down kernel: O = sum over the segment's neuron tiles
//               of H_tile[64 x active] * W_down[active rows, 128 cols]; the
//               neuron-major down rows are staged row-major in LDS and read
//               transposed (ds_read_b64_tr_b16) as the MFMA B operand.  One
//               partial output per pair and segment (one segment unless few
//               items leave the device short of workgroups).
// Work indices are remapped so that each XCD (8 per MI355X, each with its own
// L2) runs a contiguous range of the work units that exist.
#include "mfma_body.h"

namespace moe {

// Standalone launch of the MFMA projection, for layers whose GEMV projection
// does not fit the merged kernel (rows wider than 2048 bf16, or fewer than 4
// wavefronts); the down tiles always run in the merged down kernel.
template <int MODE>
__global__ __launch_bounds__(256, 3) void k_proj_mfma(MfmaParams p)
{
    __shared__ MfmaProjLds S;
    mfma_proj_body<MODE>(p, S, blockIdx.x);
}


static int round8(long long v) { return (int)((v + 7) / 8 * 8); }

hipError_t launch_proj_mfma(const Plan &pl, const MfmaParams &mp, int mode, hipStream_t st, hipEvent_t ev_begin,
                            hipEvent_t ev_end)
{
    if (!pl.use_mfma) return hipSuccess;
    const dim3 grid(round8((long long)pl.max_pairs * pl.NT)), block(256);
    if (mode == MOE_DENSE) launch_timed(k_proj_mfma<MOE_DENSE>, grid, block, st, ev_begin, ev_end, mp);
    else launch_timed(k_proj_mfma<MOE_SPARSE>, grid, block, st, ev_begin, ev_end, mp);
    return hipGetLastError();
}

}  // namespace moe
