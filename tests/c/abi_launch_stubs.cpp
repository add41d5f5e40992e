// Stand-ins for the kernel launchers, for a host-only build of the C ABI's
// argument checks (run under the address and undefined-behaviour sanitizers
// without a GPU).  The checks exercised return before any launch, so each
// stand-in counts the call and reports a launch failure.
#include "kv.hpp"
#include "plan.hpp"
#include "topk.hpp"
#include "tree_mask.hpp"

extern "C" int abi_stub_launches = 0;

namespace sv {
namespace {
hipError_t refused() {
    ++abi_stub_launches;
    return hipErrorInvalidDeviceFunction;
}
}  // namespace

hipError_t launch_kv_commit(const KvArgs &, hipStream_t) { return refused(); }
hipError_t launch_chain_stats(const ChainArgs &, int, hipStream_t) { return refused(); }
hipError_t launch_chain_draw(const ChainArgs &, int, hipStream_t) { return refused(); }
hipError_t launch_chain_fused(const ChainArgs &, int, hipStream_t) { return refused(); }
hipError_t launch_greedy(const GreedyArgs &, int, hipStream_t) { return refused(); }
hipError_t launch_tree(const TreeArgs &, int, hipStream_t) { return refused(); }
hipError_t launch_tree_dyn(const TreeDynArgs &, int, hipStream_t) { return refused(); }
hipError_t launch_advance_tag(uint32_t *, hipStream_t) { return refused(); }
hipError_t launch_topk(const TopkArgs &, int, hipStream_t) { return refused(); }
hipError_t launch_tree_mask(const MaskArgs &, hipStream_t) { return refused(); }
}  // namespace sv
