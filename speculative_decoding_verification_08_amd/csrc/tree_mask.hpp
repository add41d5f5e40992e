// Launch arguments of the tree attention mask (tree_mask.hip), shared with the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxMaskNodes = 256;  // one thread per node

struct MaskArgs {
    const int32_t *parents;     // [B][N]
    const int32_t *node_count;  // nullable [B]
    int32_t B, N;
    uint32_t *mask;             // [B][N][ceil(N / 32)]
    int32_t *depth;             // [B][N]
};

hipError_t launch_tree_mask(const MaskArgs &a, hipStream_t s);

}  // namespace sv
