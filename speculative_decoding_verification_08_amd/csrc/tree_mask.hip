// Tree attention mask on gfx950 (French lesson, section on verifying a tree
// with attention: in the tree's one verify forward each token attends only
// to its ancestors; forum post §10: tree attention needs custom masks and
// position ids).  Per sequence and node, the packed set {node} + ancestors
// and the node's depth; the verify forward turns them into its attention
// mask and position ids.
//
// One workgroup per sequence, one thread per node (N <= 256).  The parent
// entries go to LDS; each thread walks its node's chain to the root, setting
// bits in up to 8 register words (a step's word is chosen by a compare per
// word, so nothing is indexed dynamically).  A node past the count, or whose
// chain meets a parent entry outside [0, node), gets an empty row and depth
// -1.  The walk takes at most `node` steps (indices strictly fall).
#include "device.hpp"
#include "tree_mask.hpp"

namespace sv {
namespace {

__global__ __launch_bounds__(kWG) void k_tree_mask(MaskArgs a) {
    __shared__ int32_t s_par[kMaxMaskNodes];
    const int b = blockIdx.x, v = threadIdx.x, N = a.N, W = (N + 31) / 32;
    const int32_t *par = a.parents + static_cast<int64_t>(b) * N;
    if (v < N) s_par[v] = par[v];
    int n = a.node_count ? a.node_count[b] : N;
    n = min(max(n, 1), N);
    __syncthreads();
    if (v >= N) return;
    uint32_t row[kMaxMaskWords];
#pragma unroll
    for (int w = 0; w < kMaxMaskWords; ++w) row[w] = 0;
    int d = -1;
    if (v < n) {
        auto mark = [&](int j) {
#pragma unroll
            for (int w = 0; w < kMaxMaskWords; ++w)
                if (w == (j >> 5)) row[w] |= 1u << (j & 31);
        };
        int cur = v, steps = 0;
        bool attached = true;
        mark(cur);
        while (cur != 0) {
            const int p = s_par[cur];
            if (p < 0 || p >= cur) {
                attached = false;
                break;
            }
            cur = p;
            mark(cur);
            ++steps;
        }
        if (attached) {
            d = steps;
        } else {
#pragma unroll
            for (int w = 0; w < kMaxMaskWords; ++w) row[w] = 0;
        }
    }
    uint32_t *out = a.mask + (static_cast<int64_t>(b) * N + v) * W;
#pragma unroll
    for (int w = 0; w < kMaxMaskWords; ++w)
        if (w < W) out[w] = row[w];
    a.depth[static_cast<int64_t>(b) * N + v] = d;
}

}  // namespace

hipError_t launch_tree_mask(const MaskArgs &a, hipStream_t s) {
    k_tree_mask<<<dim3(static_cast<uint32_t>(a.B)), dim3(kWG), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sv
