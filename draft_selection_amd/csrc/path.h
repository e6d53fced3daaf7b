// select_path: the whole selector in one call.  ("DFlash 2: Keep Drafting
// Parallel", Method > Lightweight Path Selector: top-16 per position, the
// projections and gate, every adjacent pair scored in one parallel pass, then
// the walk.)
//
// The kernels are those of the separate calls, in the same order and with the
// same arithmetic, so every output has the same bits.  One fusion: the gate's
// split-K reduction, which needs neither the top-16 nor LDS, rides in the
// top-16 launch as extra workgroups after the top-16 ones.  They fill the
// workgroup slots the top-16 leaves free (at 1,024 rows it holds 4 per CU of
// the 7 its registers allow), so the reduction runs beside the HBM-bound
// top-16 instead of as a launch of its own between the gate GEMM and the
// top-16.
#pragma once

#include "project.h"
#include "topk16.h"

namespace dsel {

// Workgroups [0, topk_wgs) run the top-16, the rest run the gate reduction,
// four output elements per thread.  The branch is per workgroup, so the top-16's
// barriers are met by whole workgroups.
template <bool BF16, int U>
__global__ __launch_bounds__(64 * kTopkWaves) void topk16_gate_kernel(TopkParams tp, GateParams gp, int64_t topk_wgs) {
    const int64_t bid = blockIdx.x;
    if (bid < topk_wgs) topk16_block<BF16, U>(tp, bid);
    else gate_reduce_unit(gp, (bid - topk_wgs) * (64 * kTopkWaves) + threadIdx.x);
}

}  // namespace dsel
