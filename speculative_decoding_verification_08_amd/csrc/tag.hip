// The tag word of calls recorded into a HIP graph.  A call records this
// one-thread kernel before its own, so every replay advances the word in the
// workspace header and the call's workgroups read their tag from it: no two
// replays share a tag, as no two host calls do.  Graph tags keep bit 31 set
// (host tags never do) and never equal 0, the value of a zeroed word.
#include "plan.hpp"

namespace sv {
namespace {

__global__ void k_advance_tag(uint32_t *word) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        uint32_t t = (*word & ~kGraphTagBit) + 1u;
        if (t >= kGraphTagBit) t = 1u;
        *word = t | kGraphTagBit;
    }
}

}  // namespace

hipError_t launch_advance_tag(uint32_t *word, hipStream_t s) {
    k_advance_tag<<<dim3(1), dim3(64), 0, s>>>(word);
    return hipGetLastError();
}

}  // namespace sv
