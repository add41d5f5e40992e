// Tree attention mask on gfx950 (French lesson, section on verifying a tree
// with attention: in the tree's one verify forward each token attends only
// to its ancestors; forum post §10: tree attention needs custom masks and
// position ids).  Per sequence and node, the packed set {node} + ancestors
// and the node's depth; the verify forward turns them into its attention
// mask and position ids.
//
// One workgroup per sequence, one thread per node (N <= 256).  The parent
// entries go to LDS; each thread walks its node's chain to the root once for
// its depth (a node past the count, or whose chain meets a parent entry
// outside [0, node), gets an empty row and depth -1), then once per output
// word, accumulating that word in a register and stopping when the indices
// fall below it.  Every walk takes at most `node` steps (indices strictly
// fall), and nothing is indexed dynamically.
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
    // First walk: is the node attached, and how deep is it.
    int d = -1;
    if (v < n) {
        int cur = v, steps = 0;
        while (cur != 0) {
            const int p = s_par[cur];
            if (p < 0 || p >= cur) {
                steps = -1;
                break;
            }
            cur = p;
            ++steps;
        }
        d = steps;
    }
    a.depth[static_cast<int64_t>(b) * N + v] = d;
    // One walk per output word (in one register), stopping below the word.
    uint32_t *out = a.mask + (static_cast<int64_t>(b) * N + v) * W;
    for (int w = 0; w < W; ++w) {
        uint32_t acc = 0;
        if (d >= 0 && v >= 32 * w) {
            int cur = v;
            for (;;) {
                if ((cur >> 5) == w) acc |= 1u << (cur & 31);
                if (cur == 0 || cur < 32 * w) break;
                cur = s_par[cur];
            }
        }
        out[w] = acc;
    }
}

}  // namespace

hipError_t launch_tree_mask(const MaskArgs &a, hipStream_t s) {
    k_tree_mask<<<dim3(static_cast<uint32_t>(a.B)), dim3(kWG), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sv
