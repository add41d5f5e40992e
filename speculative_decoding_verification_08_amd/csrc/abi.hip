// C ABI of the verify library: argument validation, launch planning and the
// workspace layout.  Everything here is host code; the kernels live in
// chain.hip, greedy_tree.hip, topk.hip, kv.hip and tree_mask.hip.
#include <math.h>
#include <string.h>

#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <random>

#include "grid_order.hpp"
#include "plan.hpp"
#include "planning.hpp"
#include "kv.hpp"
#include "tree_mask.hpp"
#include "topk.hpp"
#include "spec_verify.h"

namespace sv {
namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <class T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

spec_status launch_status(hipError_t e) { return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH; }

// Tag of one host call: a process-wide counter in [1, 2^31), so never 0 (a
// zeroed word) and never a graph tag.  It starts at a random value, so that a
// workspace whose words were left by another process or another load of the
// library holds this process's tags only by a 2^-31 chance.
uint32_t random_tag_start() {
    std::random_device rd;
    uint64_t x = (static_cast<uint64_t>(rd()) << 32) ^ rd();
    x ^= static_cast<uint64_t>(std::chrono::steady_clock::now().time_since_epoch().count());
    x ^= static_cast<uint64_t>(getpid()) << 17;
    x *= 0x9e3779b97f4a7c15ull;
    return static_cast<uint32_t>(x >> 33);
}
uint32_t next_call_tag() {
    static std::atomic<uint32_t> counter{random_tag_start()};
    return counter.fetch_add(1u, std::memory_order_relaxed) % (kGraphTagBit - 1u) + 1u;
}

// The tag of one call.  While `stream` is being captured into a graph, the
// call records a one-thread kernel that advances the tag word at the start of
// the workspace, and its workgroups read their tag from that word, so every
// replay has a tag of its own; otherwise the tag comes from the host counter.
spec_status call_tag(void *ws, hipStream_t stream, uint32_t &tag, const uint32_t *&src) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return SPEC_ERR_LAUNCH;
    if (cs == hipStreamCaptureStatusActive) {
        uint32_t *word = static_cast<uint32_t *>(ws);
        if (launch_advance_tag(word, stream) != hipSuccess) return SPEC_ERR_LAUNCH;
        tag = 0;
        src = word;
    } else {
        tag = next_call_tag();
        src = nullptr;
    }
    return SPEC_OK;
}

// Shared validation of the chain entry points.
spec_status chain_setup(const void *target, const void *draft, spec_dtype dtype, int32_t B,
                        int32_t K, int32_t V, float T, void *ws, size_t ws_bytes, Plan &plan,
                        ChainArgs &a) {
    if (!valid_dtype(dtype) || !(T > 0.f) || isinf(T)) return SPEC_ERR_INVALID_ARG;
    if (!make_plan(SPEC_MODE_CHAIN, B, K, V, dtype, plan)) return SPEC_ERR_INVALID_ARG;
    if (B == 0) return SPEC_OK;
    if (!target || !aligned(target, 16)) return SPEC_ERR_INVALID_ARG;
    if (K > 0 && (!draft || !aligned(draft, 16))) return SPEC_ERR_INVALID_ARG;
    if (!ws || ws_bytes < plan.bytes || !aligned(ws, 16)) return SPEC_ERR_WORKSPACE;
    memset(&a, 0, sizeof a);
    a.target = target;
    a.draft = draft;
    a.B = B;
    a.K = K;
    a.V = V;
    a.c = static_cast<float>(1.4426950408889634 / static_cast<double>(T));
    a.hdr = static_cast<uint32_t *>(ws);
    a.chunk = plan.chunk;
    a.nchunk = plan.nchunk;
    a.nchunk2 = plan.nchunk2;
    chain_grid_fields(plan, K, a);
    a.partial = at<uint64_t>(ws, plan.off_partial);
    a.sums = at<uint64_t>(ws, plan.off_sums);
    a.rec = at<uint64_t>(ws, plan.off_rec);
    a.pairs = at<uint64_t>(ws, plan.off_pairs);
    a.gate = at<uint64_t>(ws, plan.off_gate);
    // Skipping bonus-row chunks after a rejection costs each bonus-row item
    // one read of its record first: worth it once the bonus rows are more
    // than a few hundred chunks.
    a.gate_bonus = static_cast<int64_t>(B) * plan.nchunk >= 512;
    return SPEC_OK;
}

spec_status chain_sample_args(const int32_t *tokens, const float *ua, const float *us, int32_t B,
                              int32_t K, int32_t *out_tokens, int32_t *out_accepted,
                              float *out_diag, ChainArgs &a) {
    if (B == 0) return SPEC_OK;
    if (K > 0 && (!tokens || !ua)) return SPEC_ERR_INVALID_ARG;
    if (!us || !out_tokens || !out_accepted) return SPEC_ERR_INVALID_ARG;
    if ((tokens && !aligned(tokens, 4)) || (ua && !aligned(ua, 4)) || !aligned(us, 4) ||
        !aligned(out_tokens, 4) || !aligned(out_accepted, 4) || (out_diag && !aligned(out_diag, 16)))
        return SPEC_ERR_INVALID_ARG;
    a.tokens = tokens;
    a.u_accept = ua;
    a.u_sample = us;
    a.out_tokens = out_tokens;
    a.out_accepted = out_accepted;
    a.out_diag = out_diag;
    return SPEC_OK;
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" {

const char *spec_verify_status_string(spec_status status) {
    switch (status) {
        case SPEC_OK: return "ok";
        case SPEC_ERR_INVALID_ARG: return "invalid argument";
        case SPEC_ERR_WORKSPACE: return "workspace missing or too small";
        case SPEC_ERR_LAUNCH: return "kernel launch failed";
        case SPEC_ERR_SCRATCH_LIMIT: return "sizes need more scratch than the fixed device array holds";
    }
    return "unknown status";
}

spec_status spec_verify_workspace_bytes(spec_mode mode, int32_t B, int32_t K_or_N, int32_t V,
                                        spec_dtype dtype, size_t *bytes) {
    if (!bytes || !valid_dtype(dtype)) return SPEC_ERR_INVALID_ARG;
    if (mode != SPEC_MODE_CHAIN && mode != SPEC_MODE_GREEDY && mode != SPEC_MODE_TREE &&
        mode != SPEC_MODE_TREE_DYN && mode != SPEC_MODE_TOPK)
        return SPEC_ERR_INVALID_ARG;
    Plan p;
    if (!make_plan(mode, B, K_or_N, V, dtype, p)) return SPEC_ERR_INVALID_ARG;
    *bytes = p.bytes;
    return SPEC_OK;
}

spec_status spec_verify_chain_stats(const void *target_logits, const void *draft_logits,
                                    spec_dtype dtype, const int32_t *draft_tokens, int32_t B,
                                    int32_t K, int32_t V, float temperature, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    Plan plan;
    ChainArgs a;
    spec_status st = chain_setup(target_logits, draft_logits, dtype, B, K, V, temperature,
                                 workspace, workspace_bytes, plan, a);
    if (st != SPEC_OK || B == 0) return st;
    if (K > 0 && (!draft_tokens || !aligned(draft_tokens, 4))) return SPEC_ERR_INVALID_ARG;
    a.tokens = draft_tokens;
    st = call_tag(workspace, stream, a.tag, a.tag_src);
    if (st != SPEC_OK) return st;
    return launch_status(launch_chain_stats(a, dtype, stream));
}

spec_status spec_verify_chain_sample(const void *target_logits, const void *draft_logits,
                                     spec_dtype dtype, const int32_t *draft_tokens,
                                     const float *u_accept, const float *u_sample, int32_t B,
                                     int32_t K, int32_t V, float temperature, int32_t *out_tokens,
                                     int32_t *out_accepted, float *out_diag, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
    Plan plan;
    ChainArgs a;
    spec_status st = chain_setup(target_logits, draft_logits, dtype, B, K, V, temperature,
                                 workspace, workspace_bytes, plan, a);
    if (st != SPEC_OK || B == 0) return st;
    st = chain_sample_args(draft_tokens, u_accept, u_sample, B, K, out_tokens, out_accepted,
                           out_diag, a);
    if (st != SPEC_OK) return st;
    st = call_tag(workspace, stream, a.tag, a.tag_src);
    if (st != SPEC_OK) return st;
    a.sample_phase = true;  // the statistics carry the tag the stats phase recorded
    return launch_status(launch_chain_draw(a, dtype, stream));
}

spec_status spec_verify_chain(const void *target_logits, const void *draft_logits,
                              spec_dtype dtype, const int32_t *draft_tokens,
                              const float *u_accept, const float *u_sample, int32_t B, int32_t K,
                              int32_t V, float temperature, int32_t *out_tokens,
                              int32_t *out_accepted, float *out_diag, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    Plan plan;
    ChainArgs a;
    spec_status st = chain_setup(target_logits, draft_logits, dtype, B, K, V, temperature,
                                 workspace, workspace_bytes, plan, a);
    if (st != SPEC_OK || B == 0) return st;
    st = chain_sample_args(draft_tokens, u_accept, u_sample, B, K, out_tokens, out_accepted,
                           out_diag, a);
    if (st != SPEC_OK) return st;
    st = call_tag(workspace, stream, a.tag, a.tag_src);
    if (st != SPEC_OK) return st;
    // The position-major order when no per-position diagnostics are asked for
    // (they need every position's statistics) and one position's items fill
    // the chip (smaller batches wait on its resolvers' chain instead).  Its
    // statistics items skip their rows after a published rejection, at the
    // price of one read before their loads.  Items of position 1 skip too
    // when one position's rows take long to stream (64 MB or more), so that
    // position 0's outcomes come out early in position 1.  Measured, us per
    // step: 64 x 5 x 128256 bf16 (33 MB a position) 34.0 skipping from
    // position 2, 34.9 from position 1, 35.5 with no skips; 256 x 8 x 151936
    // fp32 (311 MB) 272.0 from position 1, 275.8 from position 2, 318.8.
    a.early_exit = out_diag == nullptr && 2ll * plan.nchunk * B >= 2048 && chain_pm_schedule(a) != 0;
    const int64_t position_bytes = 2ll * B * V * (dtype == SPEC_DTYPE_BF16 ? 2 : 4);
    a.gate_pos1 = a.early_exit && position_bytes >= (64ll << 20);
    if (a.early_exit || chain_schedule(a) != 0) return launch_status(launch_chain_fused(a, dtype, stream));
    // Too large for one grid: the two kernels of the phase entry points, the
    // draws reading the statistics under this call's own tag.
    st = launch_status(launch_chain_stats(a, dtype, stream));
    if (st != SPEC_OK) return st;
    return launch_status(launch_chain_draw(a, dtype, stream));
}

spec_status spec_verify_workspace_failures(void *workspace, size_t workspace_bytes, int32_t reset,
                                           uint32_t *failures, hipStream_t stream) {
    if (!workspace || workspace_bytes < kWorkspaceHeader || !aligned(workspace, 16) || !failures)
        return SPEC_ERR_INVALID_ARG;
    uint32_t *word = static_cast<uint32_t *>(workspace) + kHdrFailures;
    if (hipMemcpyAsync(failures, word, sizeof *failures, hipMemcpyDeviceToHost, stream) != hipSuccess)
        return SPEC_ERR_LAUNCH;
    if (reset && hipMemsetAsync(word, 0, sizeof *word, stream) != hipSuccess) return SPEC_ERR_LAUNCH;
    return hipStreamSynchronize(stream) == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}

spec_status spec_verify_greedy(const void *target_logits, spec_dtype dtype,
                               const int32_t *draft_tokens, int32_t B, int32_t K, int32_t V,
                               int32_t *out_tokens, int32_t *out_accepted, void *workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dtype(dtype)) return SPEC_ERR_INVALID_ARG;
    Plan plan;
    if (!make_plan(SPEC_MODE_GREEDY, B, K, V, dtype, plan)) return SPEC_ERR_INVALID_ARG;
    if (B == 0) return SPEC_OK;
    if (!target_logits || !aligned(target_logits, 16)) return SPEC_ERR_INVALID_ARG;
    if ((K > 0 && (!draft_tokens || !aligned(draft_tokens, 4))) || !out_tokens ||
        !out_accepted || !aligned(out_tokens, 4) || !aligned(out_accepted, 4))
        return SPEC_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < plan.bytes || !aligned(workspace, 16))
        return SPEC_ERR_WORKSPACE;
    GreedyArgs g;
    g.am.logits = target_logits;
    g.am.rows = plan.rows;
    g.am.V = V;
    g.am.chunk = plan.chunk;
    g.am.nchunk = plan.nchunk;
    g.am.fd_nch = make_fastdiv(plan.nchunk);
    const spec_status st = call_tag(workspace, stream, g.am.tag, g.am.tag_src);
    if (st != SPEC_OK) return st;
    g.am.partial = at<uint64_t>(workspace, plan.off_partial);
    g.am.hdr = static_cast<uint32_t *>(workspace);
    g.tokens = draft_tokens;
    g.B = B;
    g.K = K;
    g.fd_per = make_fastdiv(static_cast<uint32_t>(K + 1));
    g.out_tokens = out_tokens;
    g.out_accepted = out_accepted;
    return launch_status(launch_greedy(g, dtype, stream));
}

spec_status spec_verify_tree_greedy(const void *node_logits, spec_dtype dtype,
                                    const int32_t *node_tokens, const int32_t *parents,
                                    int32_t B, int32_t N, int32_t V, int32_t *out_tokens,
                                    int32_t *out_path, int32_t *out_depth, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dtype(dtype) || !parents) return SPEC_ERR_INVALID_ARG;
    Plan plan;
    if (!make_plan(SPEC_MODE_TREE, B, N, V, dtype, plan)) return SPEC_ERR_INVALID_ARG;
    TreeArgs t;
    memset(&t, 0, sizeof t);
    if (parents[0] != -1) return SPEC_ERR_INVALID_ARG;
    t.tree.N = N;
    t.tree.parent[0] = -1;
    t.tree.depth[0] = 0;
    int D = 0;
    for (int v = 1; v < N; ++v) {
        if (parents[v] < 0 || parents[v] >= v) return SPEC_ERR_INVALID_ARG;
        t.tree.parent[v] = static_cast<int16_t>(parents[v]);
        t.tree.depth[v] = static_cast<uint8_t>(t.tree.depth[parents[v]] + 1);
        if (t.tree.depth[v] > D) D = t.tree.depth[v];
    }
    t.tree.D = D;
    if (B == 0) return SPEC_OK;
    if (!node_logits || !aligned(node_logits, 16)) return SPEC_ERR_INVALID_ARG;
    if (!node_tokens || !out_tokens || !out_depth || !aligned(node_tokens, 4) ||
        !aligned(out_tokens, 4) || !aligned(out_depth, 4) || (out_path && !aligned(out_path, 4)))
        return SPEC_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < plan.bytes || !aligned(workspace, 16))
        return SPEC_ERR_WORKSPACE;
    t.am.logits = node_logits;
    t.am.rows = plan.rows;
    t.am.V = V;
    t.am.chunk = plan.chunk;
    t.am.nchunk = plan.nchunk;
    t.am.fd_nch = make_fastdiv(plan.nchunk);
    t.fd_per = make_fastdiv(static_cast<uint32_t>(N));
    const spec_status st = call_tag(workspace, stream, t.am.tag, t.am.tag_src);
    if (st != SPEC_OK) return st;
    t.am.partial = at<uint64_t>(workspace, plan.off_partial);
    t.am.hdr = static_cast<uint32_t *>(workspace);
    t.tokens = node_tokens;
    t.B = B;
    t.out_tokens = out_tokens;
    t.out_path = out_path;
    t.out_depth = out_depth;
    // Node-major order, which does not read the rows of nodes that cannot be
    // accepted, when the batch streams over many generations of workgroups
    // (so that a node's outcome is out before its children's items start)
    // and the tree reaches two levels below the root (a level-one node's
    // items start before the root's outcome is out; from the first node two
    // levels down, the items read their gate line).
    t.gate_from = N;
    for (int v = 1; v < N; ++v)
        if (t.tree.depth[v] >= 2) {
            t.gate_from = v;
            break;
        }
    t.node_major = B <= 65535 && t.gate_from < N &&
                   static_cast<int64_t>(B) * N * plan.nchunk >= kTreeNodeMajorItems;
    t.node_out = at<uint64_t>(workspace, plan.off_pairs);
    t.gate = at<uint64_t>(workspace, plan.off_gate);
    return launch_status(launch_tree(t, dtype, stream));
}

spec_status spec_verify_tree_greedy_dyn(const void *node_logits, spec_dtype dtype,
                                        const int32_t *node_tokens, const int32_t *parents,
                                        const int32_t *node_count, int32_t B, int32_t Nmax,
                                        int32_t V, int32_t *out_tokens, int32_t *out_path,
                                        int32_t *out_depth, void *workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dtype(dtype)) return SPEC_ERR_INVALID_ARG;
    Plan plan;
    if (!make_plan(SPEC_MODE_TREE_DYN, B, Nmax, V, dtype, plan)) return SPEC_ERR_INVALID_ARG;
    if (B == 0) return SPEC_OK;
    if (!node_logits || !aligned(node_logits, 16)) return SPEC_ERR_INVALID_ARG;
    if (!node_tokens || !parents || !node_count || !out_tokens || !out_depth ||
        !aligned(node_tokens, 4) || !aligned(parents, 4) || !aligned(node_count, 4) ||
        !aligned(out_tokens, 4) || !aligned(out_depth, 4) || (out_path && !aligned(out_path, 4)))
        return SPEC_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < plan.bytes || !aligned(workspace, 16))
        return SPEC_ERR_WORKSPACE;
    TreeDynArgs t;
    t.am.logits = node_logits;
    t.am.rows = plan.rows;
    t.am.V = V;
    t.am.chunk = plan.chunk;
    t.am.nchunk = plan.nchunk;
    t.am.fd_nch = make_fastdiv(plan.nchunk);
    const spec_status st = call_tag(workspace, stream, t.am.tag, t.am.tag_src);
    if (st != SPEC_OK) return st;
    t.am.partial = at<uint64_t>(workspace, plan.off_partial);
    t.am.hdr = static_cast<uint32_t *>(workspace);
    t.tokens = node_tokens;
    t.parents = parents;
    t.node_count = node_count;
    t.B = B;
    t.Nmax = Nmax;
    t.fd_nmax = make_fastdiv(static_cast<uint32_t>(Nmax));
    t.out_tokens = out_tokens;
    t.out_path = out_path;
    t.out_depth = out_depth;
    // Node-major order (rows of nodes that cannot be accepted are not read)
    // for batches that stream over many generations of workgroups, as for
    // the static tree; padding rows cost their items one read of the count.
    t.node_major = B <= 65535 && Nmax >= 3 &&
                   static_cast<int64_t>(B) * Nmax * plan.nchunk >= kTreeNodeMajorItems;
    t.node_out = at<uint64_t>(workspace, plan.off_pairs);
    t.gate = at<uint64_t>(workspace, plan.off_gate);
    return launch_status(launch_tree_dyn(t, dtype, stream));
}

spec_status spec_draft_topk(const void *logits, spec_dtype dtype, int32_t rows, int32_t V,
                            int32_t k, int32_t *out_idx, float *out_val, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dtype(dtype)) return SPEC_ERR_INVALID_ARG;
    Plan plan;
    if (!make_plan(SPEC_MODE_TOPK, rows, k, V, dtype, plan)) return SPEC_ERR_INVALID_ARG;
    if (rows == 0) return SPEC_OK;
    if (!logits || !aligned(logits, 16) || !out_idx || !aligned(out_idx, 4) ||
        (out_val && !aligned(out_val, 4)))
        return SPEC_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < plan.bytes || !aligned(workspace, 16))
        return SPEC_ERR_WORKSPACE;
    TopkArgs a;
    a.logits = logits;
    a.rows = rows;
    a.V = V;
    a.chunk = plan.chunk;
    a.nchunk = plan.nchunk;
    a.k = k;
    const spec_status st = call_tag(workspace, stream, a.tag, a.tag_src);
    if (st != SPEC_OK) return st;
    a.lag = topk_lag(rows, plan.nchunk);
    a.fd_nch = make_fastdiv(static_cast<uint32_t>(plan.nchunk));
    a.fd_blk = make_fastdiv(static_cast<uint32_t>(kTopkGroupRows * plan.nchunk + 1));
    a.partial = at<uint64_t>(workspace, plan.off_partial);
    a.hdr = static_cast<uint32_t *>(workspace);
    a.out_idx = out_idx;
    a.out_val = out_val;
    return launch_status(launch_topk(a, dtype, stream));
}

spec_status spec_kv_commit(const void *scratch, void *cache, int32_t planes, int32_t B, int32_t N,
                           int32_t S, int64_t row_bytes, const int32_t *path, int32_t P,
                           const int32_t *count, const int32_t *cache_len, int32_t *new_len,
                           hipStream_t stream) {
    if (planes < 1 || B < 0 || N < 0 || S < 0 || row_bytes < 16 || row_bytes % 16 != 0)
        return SPEC_ERR_INVALID_ARG;
    if (!path) P = N;
    if (P < 0) return SPEC_ERR_INVALID_ARG;
    const int64_t vpr = row_bytes / 16;
    // 32-bit vector indices inside a sequence's window, and a one-dimensional grid.
    if (vpr > 0x7fffffffLL || static_cast<int64_t>(P) * vpr > 0x7fffffffLL ||
        static_cast<int64_t>(planes) * B > 0x7fffffffLL)
        return SPEC_ERR_INVALID_ARG;
    if (B == 0) return SPEC_OK;
    if (!scratch || !cache || !aligned(scratch, 16) || !aligned(cache, 16) || !count ||
        !cache_len || !new_len || !aligned(count, 4) || !aligned(cache_len, 4) ||
        !aligned(new_len, 4) || (path && !aligned(path, 4)) || new_len == cache_len)
        return SPEC_ERR_INVALID_ARG;
    // The two buffers must not overlap (a copy between overlapping rows could
    // read a row it has already overwritten).
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(scratch), c0 = reinterpret_cast<uintptr_t>(cache);
    const uint64_t sbytes = static_cast<uint64_t>(planes) * B * N * row_bytes;
    const uint64_t cbytes = static_cast<uint64_t>(planes) * B * S * row_bytes;
    if (sbytes > 0 && cbytes > 0 && s0 < c0 + cbytes && c0 < s0 + sbytes) return SPEC_ERR_INVALID_ARG;
    KvArgs a;
    a.scratch = static_cast<const uint4 *>(scratch);
    a.cache = static_cast<uint4 *>(cache);
    a.planes = planes;
    a.B = B;
    a.N = N;
    a.S = S;
    a.P = P;
    a.vpr = static_cast<int32_t>(vpr);
    a.fd_planes = make_fastdiv(static_cast<uint32_t>(planes));
    a.fd_vpr = make_fastdiv(static_cast<uint32_t>(vpr));
    a.path = path;
    a.count = count;
    a.len = cache_len;
    a.new_len = new_len;
    return launch_status(launch_kv_commit(a, stream));
}

spec_status spec_tree_mask(const int32_t *parents, const int32_t *node_count, int32_t B, int32_t N,
                           uint32_t *mask, int32_t *depth, hipStream_t stream) {
    if (B < 0 || N < 1 || N > SPEC_VERIFY_MAX_TREE_NODES || N > kMaxMaskNodes)
        return SPEC_ERR_INVALID_ARG;
    if (B == 0) return SPEC_OK;
    if (!parents || !mask || !depth || !aligned(parents, 4) || !aligned(mask, 4) ||
        !aligned(depth, 4) || (node_count && !aligned(node_count, 4)))
        return SPEC_ERR_INVALID_ARG;
    MaskArgs a;
    a.parents = parents;
    a.node_count = node_count;
    a.B = B;
    a.N = N;
    a.mask = mask;
    a.depth = depth;
    return launch_status(launch_tree_mask(a, stream));
}

}  // extern "C"
