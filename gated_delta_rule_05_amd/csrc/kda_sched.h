// kda_sched.h -- work-group -> (sequence, head, value tile) mapping of the
// prefill kernels.
//
// A launch has groups = N*H (sequence, head) pairs, each split into R value
// tiles, and ceil(groups/8)*8*R work-groups.  The dispatcher hands
// consecutive work-groups to the 8 XCDs round-robin (XCD = blockIdx % 8),
// so the mapping below (1) puts the R tiles of one pair on the same XCD,
// where they re-read the same q, k and gate rows from that XCD's L2,
// (2) deals pairs to XCDs round-robin for balance, and (3) keeps pair
// order within the dispatch order, so the plan's longest-first sequence
// order is the order in which work starts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kNumXcd = 8;

__host__ __device__ __forceinline__ int64_t prefill_grid_blocks(int64_t groups, int R) {
    return ((groups + kNumXcd - 1) / kNumXcd) * kNumXcd * R;
}

// Returns false for the padding work-groups (pair index >= groups).
__device__ __forceinline__ bool prefill_map_block(int64_t b, int64_t groups, int R,
                                                  int64_t& pair, int& tile) {
    const int64_t x = b % kNumXcd;
    const int64_t j = b / kNumXcd;
    tile = static_cast<int>(j % R);
    pair = (j / R) * kNumXcd + x;
    return pair < groups;
}

}  // namespace kda
