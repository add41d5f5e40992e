// Greedy verify at T = 0 on gfx950, one launch per call (French lesson, "La
// règle de l'exactitude", greedy case, for the chain; "Vérifie l'attention des
// arbres" and the EAGLE section for the tree: one target pass scores every
// candidate and the longest accepted branch wins).
//
// Argmax items: one workgroup per vocabulary chunk of one row; 16-byte loads,
// per-lane (max, lowest index) kept in index order, then a workgroup reduce.
// Values are compared as floats widened exactly from bf16, so ties and -0.0 ==
// +0.0 behave as on the raw logits.  Each publishes its chunk's (value, index)
// as two tagged words.
//
// Resolve: for the greedy chain and the static tree, the argmax item of the
// last chunk of a sequence's last row resolves the sequence once its own
// partial is out; for per-sequence trees, one resolve workgroup per tree
// placed after every argmax workgroup.  Either way a resolve waits (bounded)
// only for workgroups of lower index.  Each group of 16 lanes merges one
// row's chunk partials with a DPP tree; the comparison is exact, so the
// result does not depend on the merge order.
#include "device.hpp"
#include "handover.hpp"
#include "grid_order.hpp"
#include "plan.hpp"

namespace sv {

static_assert(kCompactTrees == kWave * kCountsPerLane, "one wavefront holds every count");
namespace {

// With VecOk (V a multiple of the vector width) every chunk starts and ends
// on a vector, so there is no unaligned head or tail to read one by one.
template <class DT, int U, bool VecOk>
__device__ __forceinline__ void argmax_item(const ArgmaxArgs &a, int64_t row, int ch) {
    constexpr int VEC = DT::kVec;
    const int64_t rbase = row * a.V;
    const int64_t g0 = rbase + static_cast<int64_t>(ch) * a.chunk;
    const int64_t g1 = min(g0 + a.chunk, rbase + a.V);
    const Span s = VecOk ? Span{g0, g0, g0 / VEC, g1 / VEC, g1, g1} : split_span<VEC>(g0, g1);

    // Each lane visits its elements in increasing index order, so a strict
    // comparison keeps the lowest index among equal values.
    float bv = -INFINITY;
    int32_t bi = INT32_MAX;
    if (!VecOk) {
        const int64_t h = s.h0 + threadIdx.x;
        if (h < s.h1) {
            const float x = load_one<DT>(a.logits, h);
            if (vi_better(x, static_cast<int32_t>(h - rbase), bv, bi)) {
                bv = x;
                bi = static_cast<int32_t>(h - rbase);
            }
        }
    }
    const uint4 *vp = static_cast<const uint4 *>(a.logits);
    int64_t v = s.va + threadIdx.x;
    for (; v + (U - 1) * kWG < s.vb; v += U * kWG) {
        uint4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = load_nt(vp + v + u * kWG);
        // Every load in flight before the first wait: left to itself the
        // scheduler starts on the first vector before issuing the last two,
        // which then leave one memory round trip later.
        __builtin_amdgcn_sched_barrier(0);
        float x[U * VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) unpack<DT>(raw[u], x + u * VEC);
        float m = x[0];
#pragma unroll
        for (int i = 1; i < U * VEC; ++i) m = fmaxf(m, x[i]);
        if (m > bv) {
            // Rare after the first batches: locate the first element equal to m.
            int at = 0;
#pragma unroll
            for (int i = U * VEC - 1; i >= 0; --i)
                if (x[i] == m) at = i;
            bv = m;
            bi = static_cast<int32_t>((v + (at / VEC) * kWG) * VEC + (at % VEC) - rbase);
        }
    }
    for (; v < s.vb; v += kWG) {
        float x[VEC];
        unpack<DT>(load_nt(vp + v), x);
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            if (x[i] > bv) {
                bv = x[i];
                bi = static_cast<int32_t>(v * VEC + i - rbase);
            }
    }
    if (!VecOk) {
        const int64_t t = s.t0 + threadIdx.x;
        if (t < s.t1) {
            const float x = load_one<DT>(a.logits, t);
            if (vi_better(x, static_cast<int32_t>(t - rbase), bv, bi)) {
                bv = x;
                bi = static_cast<int32_t>(t - rbase);
            }
        }
    }
    vi_reduce_wg(bv, bi);
    if (threadIdx.x == 0) {
        uint64_t *w = a.partial + 2 * (row * a.nchunk + ch);
        publish(w, a.tag, __float_as_uint(bv));
        publish(w + 1, a.tag, static_cast<uint32_t>(bi));
    }
}

// argmax of rows [0, nrows) of one sequence from their tagged chunk partials
// part[nrows][nch][2] into s_a (an all -inf row, outside the contract, maps to
// 0).  Group g of 16 lanes takes rows g, g + 16, ... (the loads of kPasses
// such rows issued together); lane i folds chunks i, i + 16, ...
// (Fold per load batch), then four DPP steps leave the row's (max, lowest
// index) in the group's last lane.  Words still missing are waited for
// (bounded) and everything is read again.  Ends with a barrier; returns false
// if a word did not arrive in time.
template <int Fold, int kPasses>
__device__ __forceinline__ bool merge_argmax_rows(const uint64_t *part, int nrows, int nch,
                                                  uint32_t tag, int32_t *s_a) {
    constexpr int kGroup = 16, kGroups = kWG / kGroup;
    __shared__ int s_stale[2][kWaves + 1];
    const int tid = threadIdx.x, lane = tid % kWave, grp = tid / kGroup, gl = tid % kGroup;
    const uint64_t t0 = wall_clock64();
    // The sequence's last-dispatched chunk usually lands last: waiting for it
    // first spares the rounds of reading everything again as earlier chunks
    // come in one after another.
    if (tid == 0) {
        const uint64_t *last = part + 2 * (static_cast<int64_t>(nrows - 1) * nch + nch - 1);
        wait_word(last, tag, t0);
        wait_word(last + 1, tag, t0);
    }
    __syncthreads();
    for (int it = 0;; ++it) {
        const uint64_t *miss = nullptr;
        for (int r0 = 0; r0 < nrows; r0 += kGroups * kPasses) {
            float bv[kPasses];
            int32_t bi[kPasses];
#pragma unroll
            for (int q = 0; q < kPasses; ++q) {
                bv[q] = -INFINITY;
                bi[q] = INT32_MAX;
            }
            for (int i0 = 0; i0 < nch; i0 += kGroup * Fold) {
                uint64_t pv[kPasses][Fold], pi[kPasses][Fold];
#pragma unroll
                for (int q = 0; q < kPasses; ++q) {
                    const int rr = min(r0 + grp + kGroups * q, nrows - 1);
#pragma unroll
                    for (int f = 0; f < Fold; ++f) {
                        const uint64_t *pw = part + 2 * (rr * nch + min(i0 + gl + kGroup * f, nch - 1));
                        pv[q][f] = fetch(pw);
                        pi[q][f] = fetch(pw + 1);
                    }
                }
#pragma unroll
                for (int q = 0; q < kPasses; ++q) {
                    const int r = r0 + grp + kGroups * q, rr = min(r, nrows - 1);
#pragma unroll
                    for (int f = 0; f < Fold; ++f) {
                        const int i = i0 + gl + kGroup * f;
                        const bool in = r < nrows && i < nch;
                        const bool cv = current(pv[q][f], tag), ci = current(pi[q][f], tag);
                        if (in && !(cv && ci) && !miss) miss = part + 2 * (rr * nch + i) + (cv ? 1 : 0);
                        const float v = word_f32(pv[q][f]);
                        const int32_t x = static_cast<int32_t>(static_cast<uint32_t>(pi[q][f]));
                        if (in && vi_better(v, x, bv[q], bi[q])) {
                            bv[q] = v;
                            bi[q] = x;
                        }
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < kPasses; ++q) {
                float v = bv[q];
                int32_t x = bi[q];
#define SV_AM_STEP(CTRL)                                                      \
    {                                                                         \
        const float v2 = dpp::mov_f<CTRL>(-INFINITY, v);                     \
        const int32_t i2 = dpp::mov_i<CTRL>(INT32_MAX, x);                   \
        if (vi_better(v2, i2, v, x)) {                                        \
            v = v2;                                                           \
            x = i2;                                                           \
        }                                                                     \
    }
                SV_AM_STEP(dpp::kRowShr1)
                SV_AM_STEP(dpp::kRowShr2)
                SV_AM_STEP(dpp::kRowShr4)
                SV_AM_STEP(dpp::kRowShr8)
#undef SV_AM_STEP
                const int r = r0 + grp + kGroups * q;
                if (r < nrows && gl == kGroup - 1) s_a[r] = x == INT32_MAX ? 0 : x;
            }
        }
        const uint64_t stale = __ballot(miss != nullptr);
        // Double-buffered by iteration: a wavefront may start the next
        // iteration while another still reads this one's flags.
        if (lane == 0) s_stale[it & 1][tid / kWave] = stale != 0;
        if (tid == 0) s_stale[it & 1][kWaves] = wall_clock64() - t0 > kWaitTicks;
        __syncthreads();
        int any_stale = 0;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) any_stale |= s_stale[it & 1][k];
        if (!any_stale) return true;
        if (s_stale[it & 1][kWaves]) return false;
        if (stale && lane == __ffsll(static_cast<unsigned long long>(stale)) - 1)
            wait_word(miss, tag, t0);
    }
}

__device__ __forceinline__ bool merge_argmax(const uint64_t *part, int nrows, int nch, uint32_t tag,
                                             int32_t *s_a) {
    return nch > 16     ? merge_argmax_rows<4, 1>(part, nrows, nch, tag, s_a)
           : nrows <= 16 ? merge_argmax_rows<1, 1>(part, nrows, nch, tag, s_a)
           : nrows <= 32 ? merge_argmax_rows<1, 2>(part, nrows, nch, tag, s_a)
                         : merge_argmax_rows<1, 4>(part, nrows, nch, tag, s_a);
}

// Sequence b of the greedy chain: a_k = argmax of target row k; j = the first
// k < K with x_k != a_k (else K); emits x_0..x_{j-1}, a_j.  Wavefront 0 does
// the test and the emission (lane k: position k).
__device__ __forceinline__ void greedy_resolve_item(const GreedyArgs &a, const ArgmaxArgs &am, int b) {
    __shared__ int32_t s_a[kMaxK + 1];
    const int K = a.K, nch = am.nchunk, lane = threadIdx.x % kWave;
    const int32_t tok = K > 0 ? a.tokens[static_cast<int64_t>(b) * K + min(lane, K - 1)] : 0;
    const uint64_t *part = am.partial + 2 * static_cast<int64_t>(b) * (K + 1) * nch;
    const bool ok = merge_argmax(part, K + 1, nch, am.tag, s_a);
    if (threadIdx.x >= kWave) return;
    int32_t *ot = a.out_tokens + static_cast<int64_t>(b) * (K + 1);
    if (!ok) {
        for (int k = lane; k <= K; k += kWave) ot[k] = -1;
        if (lane == 0) {
            a.out_accepted[b] = -1;
            count_failure(am.hdr);
        }
        return;
    }
    const uint64_t m = __ballot(lane < K && tok != s_a[lane]);
    const int j = m ? (__ffsll(static_cast<unsigned long long>(m)) - 1) : K;
    for (int k = lane; k <= K; k += kWave) {
        int32_t o = -1;
        if (k < j) o = tok;  // k < j <= K <= 64: k is this lane
        else if (k == j) o = s_a[k];
        ot[k] = o;
    }
    if (lane == 0) a.out_accepted[b] = j;
}

// Tree b's outputs after a bounded wait ran out: every entry -1, counted.
__device__ __forceinline__ void tree_fail(const TreeArgs &a, const ArgmaxArgs &am, int b) {
    const int v = threadIdx.x, D = a.tree.D;
    if (v <= D) {
        a.out_tokens[static_cast<int64_t>(b) * (D + 1) + v] = -1;
        if (a.out_path) a.out_path[static_cast<int64_t>(b) * (D + 1) + v] = -1;
    }
    if (v == 0) {
        a.out_depth[b] = -1;
        count_failure(am.hdr);
    }
}

// Tree b's outputs from its accepted nodes (s_ok), their argmaxes (s_a, read
// at accepted nodes only) and its shape in LDS: the deepest accepted node,
// lowest index among equals, the tokens of the nodes on its path below the
// root, then its argmax.  Thread i writes entry i.
__device__ __forceinline__ void tree_emit(const TreeArgs &a, int b, const int *s_ok, const int32_t *s_a,
                                          const int *s_par, const int *s_dep, const int32_t *s_tok) {
    __shared__ int s_best;
    __shared__ int s_path[kMaxTreeNodes];
    const int v = threadIdx.x, N = a.tree.N, D = a.tree.D;
    const int key = (v < N && s_ok[v]) ? ((s_dep[v] << 16) | (0xFFFF - v)) : -1;
    const int best_key = max_wg(key);
    if (v == 0) s_best = 0xFFFF - (best_key & 0xFFFF);
    __syncthreads();
    if (v == 0) {
        const int best = s_best;
        const int d = s_dep[best];
        int node = best;
        for (int i = d; i >= 0; --i) {
            s_path[i] = node;
            node = s_par[node];
        }
    }
    __syncthreads();
    const int best = s_best, d = s_dep[best];
    if (v <= D) {
        int32_t o = -1;
        if (v < d) o = s_tok[s_path[v + 1]];
        else if (v == d) o = s_a[best];
        a.out_tokens[static_cast<int64_t>(b) * (D + 1) + v] = o;
        if (a.out_path) a.out_path[static_cast<int64_t>(b) * (D + 1) + v] = v <= d ? s_path[v] : -1;
    }
    if (v == 0) a.out_depth[b] = d;
}

// Tree b: node v matches iff its token equals its parent's argmax; a node is
// accepted iff it and all its ancestors match; the deepest accepted node wins
// (lowest index among equals); emits the path's tokens, then that node's
// argmax.
__device__ __forceinline__ void tree_resolve_item(const TreeArgs &a, const ArgmaxArgs &am, int b) {
    __shared__ int32_t s_a[kMaxTreeNodes];
    __shared__ int s_ok[kMaxTreeNodes];
    __shared__ int s_anc[kMaxTreeNodes];
    __shared__ int s_par[kMaxTreeNodes], s_dep[kMaxTreeNodes];
    __shared__ int32_t s_tok[kMaxTreeNodes];
    static_assert(kMaxTreeNodes == kWG, "one thread per node");
    const int v = threadIdx.x;
    const int N = a.tree.N, D = a.tree.D, nch = am.nchunk;
    // The tree's shape and the drafted tokens go to LDS while the partials
    // are awaited: read from the argument block with a per-node index, each
    // would otherwise be a memory round trip after the last partial lands
    // (merge_argmax ends with a barrier).
    const int32_t tok = v < N ? a.tokens[static_cast<int64_t>(b) * N + v] : 0;
    if (v < N) {
        s_par[v] = a.tree.parent[v];
        s_dep[v] = a.tree.depth[v];
        s_tok[v] = tok;
    }
    const uint64_t *part = am.partial + 2 * static_cast<int64_t>(b) * N * nch;
    if (!merge_argmax(part, N, nch, am.tag, s_a)) {
        tree_fail(a, am, b);
        return;
    }
    // match[v], then accepted = all matches on the path to the root, folded
    // by pointer jumping: after the steps of 1, 2, 4, ... <= D every node has
    // folded all of its at most D ancestors.
    const int par = v < N ? s_par[v] : -1;
    if (v < N) {
        s_ok[v] = (v == 0) ? 1 : (tok == s_a[par]);
        s_anc[v] = par;
    }
    __syncthreads();
    for (int step = 1; step <= D; step <<= 1) {
        int ok = 0, anc = -1;
        if (v < N) {
            anc = s_anc[v];
            ok = s_ok[v];
            if (anc >= 0) {
                ok &= s_ok[anc];
                anc = s_anc[anc];
            }
        }
        __syncthreads();
        if (v < N) {
            s_ok[v] = ok;
            s_anc[v] = anc;
        }
        __syncthreads();
    }
    tree_emit(a, b, s_ok, s_a, s_par, s_dep, s_tok);
}

// ------------------------------------------------------------ node-major order
//
// A node's row matters only if the node can be accepted: its argmax decides
// its children's matches and, for the deepest accepted node, the bonus token.
// In node-major order (nodes in index order, every tree's row of a node
// together) each node's resolver publishes the node's outcome -- its argmax,
// or kNodeDead when it cannot be accepted -- and marks the gate lines of the
// children that cannot be accepted, so that their chunk items, dispatched
// later, skip their loads.  The outputs are those of the tree-major order.

constexpr uint32_t kNodeDead = 0xffffffffu, kNodeFailed = 0xfffffffeu;

__device__ __forceinline__ int64_t node_gate_line(int64_t b, int N, int v) {
    return (b * N + v) * kGateLineWords;
}

// Whether the chunk items of node v of tree b may skip: its gate line is
// marked (read through the caches: a stale line only costs the skip).
// Uniform over the workgroup.
__device__ __forceinline__ bool node_not_needed(const TreeArgs &a, uint32_t tag, int b, int v) {
    __shared__ int s_skip;
    if (threadIdx.x == 0) s_skip = current(plain_word(a.gate + node_gate_line(b, a.tree.N, v)), tag);
    __syncthreads();
    return s_skip != 0;
}

// Tree b from every node's outcome, by the resolver of its last node (whose
// own outcome is `last`): a node is accepted iff its outcome is an argmax.
__device__ __forceinline__ void tree_from_outcomes(const TreeArgs &a, const ArgmaxArgs &am, int b,
                                                   uint32_t last) {
    __shared__ int32_t s_a[kMaxTreeNodes], s_tok[kMaxTreeNodes];
    __shared__ int s_ok[kMaxTreeNodes], s_par[kMaxTreeNodes], s_dep[kMaxTreeNodes];
    __shared__ int s_fail;
    const int u = threadIdx.x, N = a.tree.N;
    if (u == 0) s_fail = 0;
    if (u < N) {
        s_par[u] = a.tree.parent[u];
        s_dep[u] = a.tree.depth[u];
        s_tok[u] = a.tokens[static_cast<int64_t>(b) * N + u];
    }
    __syncthreads();
    if (u < N) {
        uint32_t o = last;
        if (u < N - 1) {
            const uint64_t *w = a.node_out + static_cast<int64_t>(b) * N + u;
            wait_word(w, am.tag, wall_clock64());
            const uint64_t x = fetch(w);
            o = current(x, am.tag) ? static_cast<uint32_t>(x) : kNodeFailed;
        }
        if (o == kNodeFailed) s_fail = 1;
        s_ok[u] = o < kNodeFailed;
        s_a[u] = static_cast<int32_t>(o);
    }
    __syncthreads();
    if (s_fail) {
        tree_fail(a, am, b);
        return;
    }
    tree_emit(a, b, s_ok, s_a, s_par, s_dep, s_tok);
}

// Resolver of node v of tree b.  It waits (bounded) for its parent's
// outcome: v can be accepted iff the parent is and v's token is the parent's
// argmax.  Then it merges v's chunk partials into v's argmax (only if v can
// be accepted: otherwise its items may have skipped), publishes the outcome,
// and marks the gate line of each child that cannot be accepted.  A wait that
// runs out makes the outcome kNodeFailed, and the tree's outputs -1.
__device__ __forceinline__ void node_resolver_item(const TreeArgs &a, const ArgmaxArgs &am, int b, int v) {
    __shared__ int32_t s_arg[1];
    __shared__ uint32_t s_live;
    const int N = a.tree.N, u = threadIdx.x;
    const uint32_t tag = am.tag;
    uint64_t *out = a.node_out + static_cast<int64_t>(b) * N;
    const int32_t *tk = a.tokens + static_cast<int64_t>(b) * N;
    // The children and their tokens, read before anything waits.
    const bool child = u > v && u < N && a.tree.parent[u] == v;
    const int32_t tok_u = child ? tk[u] : 0;
    if (u == 0) {
        uint32_t live = 1;  // 1: can be accepted, 0: cannot, 2: a wait ran out
        if (v > 0) {
            const int32_t tok_v = tk[v];
            const uint64_t *pw = out + a.tree.parent[v];
            wait_word(pw, tag, wall_clock64());
            const uint64_t w = fetch(pw);
            const uint32_t pv = static_cast<uint32_t>(w);
            live = (!current(w, tag) || pv == kNodeFailed) ? 2u
                   : (pv == kNodeDead || static_cast<int32_t>(pv) != tok_v) ? 0u
                                                                          : 1u;
        }
        s_live = live;
    }
    __syncthreads();
    const uint32_t live = s_live;
    uint32_t res = live == 0 ? kNodeDead : kNodeFailed;
    if (live == 1) {
        const uint64_t *part = am.partial + 2 * (static_cast<int64_t>(b) * N + v) * am.nchunk;
        if (merge_argmax(part, 1, am.nchunk, tag, s_arg)) res = static_cast<uint32_t>(s_arg[0]);
    }
    if (u == 0) publish(out + v, tag, res);
    if (child && (res >= kNodeFailed || tok_u != static_cast<int32_t>(res)))
        publish(a.gate + node_gate_line(b, N, u), tag, 1u);
    if (v == N - 1) tree_from_outcomes(a, am, b, res);
}

// Tree b's outputs after a bounded wait ran out: every entry -1, counted.
__device__ __forceinline__ void tree_dyn_fail(const TreeDynArgs &a, const ArgmaxArgs &am, int b) {
    const int v = threadIdx.x;
    const int64_t row0 = static_cast<int64_t>(b) * a.Nmax;
    if (v < a.Nmax) {
        a.out_tokens[row0 + v] = -1;
        if (a.out_path) a.out_path[row0 + v] = -1;
    }
    if (v == 0) {
        a.out_depth[b] = -1;
        count_failure(am.hdr);
    }
}

// Tree b of n nodes from node v's match (s_ok), parent (s_anc, s_par; -1 if
// unattached), unit depth step (s_dep), argmax (s_a) and token (s_tok), in
// LDS: acceptance and depth folded over the ancestors by pointer jumping,
// ceil(log2 n) steps; then the deepest accepted node, lowest index among
// equals (the root always is), its path's tokens and its argmax.
__device__ __forceinline__ void tree_dyn_finish(const TreeDynArgs &a, int b, int n, int *s_ok, int *s_anc,
                                                int *s_dep, const int *s_par, const int32_t *s_a,
                                                const int32_t *s_tok) {
    __shared__ int s_best;
    __shared__ int s_path[kMaxTreeNodes];
    const int v = threadIdx.x, Nmax = a.Nmax;
    const int64_t row0 = static_cast<int64_t>(b) * Nmax;
    __syncthreads();
    for (int step = 1; step < n; step <<= 1) {
        int ok = 0, anc = -1, dep = 0;
        if (v < n) {
            anc = s_anc[v];
            ok = s_ok[v];
            dep = s_dep[v];
            if (anc >= 0) {
                ok &= s_ok[anc];
                dep += s_dep[anc];
                anc = s_anc[anc];
            }
        }
        __syncthreads();
        if (v < n) {
            s_ok[v] = ok;
            s_anc[v] = anc;
            s_dep[v] = dep;
        }
        __syncthreads();
    }
    const int key = (v < n && s_ok[v]) ? ((s_dep[v] << 16) | (0xFFFF - v)) : -1;
    const int best_key = max_wg(key);
    if (v == 0) {
        const int best = 0xFFFF - (best_key & 0xFFFF);
        s_best = best;
        int node = best;
        for (int i = s_dep[best]; i >= 0; --i) {
            s_path[i] = node;
            node = s_par[node];
        }
    }
    __syncthreads();
    const int best = s_best, d = s_dep[best];
    if (v < Nmax) {
        int32_t o = -1;
        if (v < d) o = s_tok[s_path[v + 1]];
        else if (v == d) o = s_a[best];
        a.out_tokens[row0 + v] = o;
        if (a.out_path) a.out_path[row0 + v] = v <= d ? s_path[v] : -1;
    }
    if (v == 0) a.out_depth[b] = d;
}

// Tree b of a batch of per-sequence trees: n = node_count[b] (clamped to
// [1, Nmax]) nodes with parents[b][v] < v; the static tree's rule on that
// tree.  A node whose parent entry is out of range is unattached: neither it
// nor its subtree is accepted, and nothing outside the tree is read.  Depths
// and acceptance are both folded by pointer jumping, ceil(log2 n) steps.
__device__ __forceinline__ void tree_dyn_resolve_item(const TreeDynArgs &a, const ArgmaxArgs &am, int b) {
    __shared__ int32_t s_a[kMaxTreeNodes];
    __shared__ int s_ok[kMaxTreeNodes], s_anc[kMaxTreeNodes], s_dep[kMaxTreeNodes];
    __shared__ int s_par[kMaxTreeNodes];
    __shared__ int32_t s_tok[kMaxTreeNodes];
    static_assert(kMaxTreeNodes == kWG, "one thread per node");
    const int v = threadIdx.x, Nmax = a.Nmax, nch = am.nchunk;
    const int64_t row0 = static_cast<int64_t>(b) * Nmax;
    const int n = min(max(a.node_count[b], 1), Nmax);
    const int32_t tok = v < n ? a.tokens[row0 + v] : 0;
    if (v < n) s_tok[v] = tok;  // for the path's tokens, after merge_argmax's barrier
    int par = v < n ? a.parents[row0 + v] : -1;
    const bool valid = v > 0 && v < n && par >= 0 && par < v;
    if (!valid) par = -1;
    const uint64_t *part = am.partial + 2 * row0 * nch;
    if (!merge_argmax(part, n, nch, am.tag, s_a)) {
        tree_dyn_fail(a, am, b);
        return;
    }
    if (v < n) {
        s_ok[v] = v == 0 ? 1 : (valid && tok == s_a[max(par, 0)]);
        s_anc[v] = par;
        s_dep[v] = v == 0 ? 0 : 1;
        s_par[v] = par;
    }
    tree_dyn_finish(a, b, n, s_ok, s_anc, s_dep, s_par, s_a, s_tok);
}

// Node-major order for per-sequence trees (as the static tree's, above):
// chunk items read their tree's node count and their gate line in one round
// and skip padding rows and nodes that cannot be accepted; a resolver per
// (tree, node) publishes the node's outcome and marks its children's gate
// lines; the resolver of a tree's last node resolves the tree.
__device__ __forceinline__ bool dyn_node_skips(const TreeDynArgs &a, uint32_t tag, int b, int v) {
    __shared__ int s_skip;
    if (threadIdx.x == 0) {
        const int32_t count = a.node_count[b];
        const uint64_t g = plain_word(a.gate + node_gate_line(b, a.Nmax, v));
        s_skip = v >= min(max(count, 1), a.Nmax) || current(g, tag);
    }
    __syncthreads();
    return s_skip != 0;
}

__device__ __forceinline__ void dyn_node_resolver_item(const TreeDynArgs &a, const ArgmaxArgs &am, int b,
                                                       int v) {
    __shared__ int32_t s_arg[1];
    __shared__ uint32_t s_live;
    __shared__ int32_t s_a[kMaxTreeNodes], s_tok[kMaxTreeNodes];
    __shared__ int s_ok[kMaxTreeNodes], s_anc[kMaxTreeNodes], s_dep[kMaxTreeNodes], s_par[kMaxTreeNodes];
    __shared__ int s_fail;
    const int Nmax = a.Nmax, u = threadIdx.x;
    const int n = min(max(a.node_count[b], 1), Nmax);
    if (v >= n) return;  // a padding row
    const uint32_t tag = am.tag;
    const int64_t row0 = static_cast<int64_t>(b) * Nmax;
    uint64_t *out = a.node_out + row0;
    // The children, their tokens, and (for the last node's tree resolve)
    // every node's parent and token, read before anything waits.
    const int par_u = u < n ? a.parents[row0 + u] : -1;
    const int32_t tok_u = u < n ? a.tokens[row0 + u] : 0;
    const bool child = u > v && u < n && par_u == v;
    if (u == 0) {
        uint32_t live = 1;  // 1: can be accepted, 0: cannot, 2: a wait ran out
        if (v > 0) {
            const int p = a.parents[row0 + v];
            if (p < 0 || p >= v) {
                live = 0;  // unattached
            } else {
                const int32_t tok_v = a.tokens[row0 + v];
                wait_word(out + p, tag, wall_clock64());
                const uint64_t w = fetch(out + p);
                const uint32_t pv = static_cast<uint32_t>(w);
                live = (!current(w, tag) || pv == kNodeFailed) ? 2u
                       : (pv == kNodeDead || static_cast<int32_t>(pv) != tok_v) ? 0u
                                                                              : 1u;
            }
        }
        s_live = live;
    }
    __syncthreads();
    const uint32_t live = s_live;
    uint32_t res = live == 0 ? kNodeDead : kNodeFailed;
    if (live == 1) {
        const uint64_t *part = am.partial + 2 * (row0 + v) * am.nchunk;
        if (merge_argmax(part, 1, am.nchunk, tag, s_arg)) res = static_cast<uint32_t>(s_arg[0]);
    }
    if (u == 0) publish(out + v, tag, res);
    if (child && (res >= kNodeFailed || tok_u != static_cast<int32_t>(res)))
        publish(a.gate + node_gate_line(b, Nmax, u), tag, 1u);
    if (v != n - 1) return;
    // The tree, from every node's outcome: accepted iff it is an argmax.
    if (u == 0) s_fail = 0;
    __syncthreads();
    if (u < n) {
        uint32_t o = res;
        if (u < n - 1) {
            wait_word(out + u, tag, wall_clock64());
            const uint64_t x = fetch(out + u);
            o = current(x, tag) ? static_cast<uint32_t>(x) : kNodeFailed;
        }
        if (o == kNodeFailed) s_fail = 1;
        const int par = (u > 0 && par_u >= 0 && par_u < u) ? par_u : -1;
        s_ok[u] = o < kNodeFailed;
        s_a[u] = static_cast<int32_t>(o);
        s_tok[u] = tok_u;
        s_anc[u] = par;
        s_par[u] = par;
        s_dep[u] = u == 0 ? 0 : 1;
    }
    __syncthreads();
    if (s_fail) {
        tree_dyn_fail(a, am, b);
        return;
    }
    tree_dyn_finish(a, b, n, s_ok, s_anc, s_dep, s_par, s_a, s_tok);
}

// Inclusive integer sum over lanes 0..lane of a wavefront (DPP, as the
// float scan: within rows of 16, then the rows' totals carried upward).
__device__ __forceinline__ int wave_incl_sum_i(int x) {
    x += dpp::mov_i<dpp::kRowShr1>(0, x);
    x += dpp::mov_i<dpp::kRowShr2>(0, x);
    x += dpp::mov_i<dpp::kRowShr4>(0, x);
    x += dpp::mov_i<dpp::kRowShr8>(0, x);
    x += dpp::mov_i<dpp::kRowBcast15, 0xA>(0, x);
    x += dpp::mov_i<dpp::kRowBcast31, 0xC>(0, x);
    return x;
}

// Compact order with lane l holding the row counts of trees P l .. P l + P - 1
// (0 past B): returns T, the batch's real rows, and for R < T the tree b and
// node v of real row R (the first lane whose running total passes R, then one
// of that lane's trees).
template <int P>
__device__ __forceinline__ uint32_t locate_row(const TreeDynArgs &a, uint32_t R, uint32_t &b, uint32_t &v) {
    const int lane = threadIdx.x % kWave;
    int n[P];
    // Every lane loads (a clamped, in-range address) and masks afterwards: a
    // select on t < B lets the compiler sink each load into a branch of its
    // own, and the loads then leave one after another.
    lane_tree_rows<P>(a.node_count, a.B, a.Nmax, lane, n);
    int s = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) s += n[j];
    const int incl = wave_incl_sum_i(s);
    const uint32_t T = static_cast<uint32_t>(wave_last_i(incl));
    if (R < T) {
        const uint64_t hit = __ballot(static_cast<uint32_t>(incl) > R);
        const int L = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        const uint32_t r = R - static_cast<uint32_t>(__builtin_amdgcn_readlane(incl - s, L));
        lane_row<P>(r, static_cast<uint32_t>(L) * P,
                    [&](int j) { return static_cast<uint32_t>(__builtin_amdgcn_readlane(n[j], L)); }, b, v);
    }
    return T;
}

template <class DT, bool VecOk, bool NodeMajor>
__global__ __launch_bounds__(kWG) void k_tree_dyn(TreeDynArgs a) {
    // The items' arguments in one batch ahead of everything else, so no
    // second round of argument loads stands before the first logit load.
    if constexpr (NodeMajor)
        asm volatile("" ::"s"(a.am.logits), "s"(a.am.V), "s"(a.am.chunk), "s"(a.am.partial),
                     "s"(a.am.tag), "s"(a.am.tag_src), "s"(a.am.nchunk), "s"(a.Nmax), "s"(a.node_count),
                     "s"(a.gate));
    // The argument block stays untouched (writing into it would copy it to
    // scratch); the argmax arguments with the call's tag are a local copy.
    ArgmaxArgs am = a.am;
    if (am.tag_src) am.tag = *am.tag_src;  // a graph replay's tag
    if constexpr (NodeMajor) {
        // Grid (chunks + 1) x trees x Nmax: x < nchunk a chunk item of row
        // (y, z), x = nchunk the resolver of node z of tree y.
        const int b = static_cast<int>(blockIdx.y), v = static_cast<int>(blockIdx.z);
        const int ch = static_cast<int>(blockIdx.x);
        if (ch < am.nchunk) {
            if (v > 0 && dyn_node_skips(a, am.tag, b, v)) return;
            argmax_item<DT, 4, VecOk>(am, static_cast<int64_t>(b) * a.Nmax + v, ch);
        } else {
            dyn_node_resolver_item(a, am, b, v);
        }
        return;
    }
    const uint32_t nch = a.am.nchunk, g = blockIdx.x, B = static_cast<uint32_t>(a.B);
    // This workgroup's item: an argmax item (row, ch), the resolve of tree
    // `row`, or nothing.
    TreeDynItem it;
    if (B <= static_cast<uint32_t>(kCompactTrees)) {
        const uint32_t R = fdiv(g, a.am.fd_nch);
        uint32_t b = 0, v = 0;
        const uint32_t T = B <= static_cast<uint32_t>(kWave) ? locate_row<1>(a, R, b, v)
                                                             : locate_row<kCountsPerLane>(a, R, b, v);
        it = tree_dyn_compact_item(g, R, nch, T, b, v, B, static_cast<uint32_t>(a.Nmax));
    } else {
        it = tree_dyn_full_item(g, nch, a.am.fd_nch, static_cast<uint32_t>(a.am.rows),
                                static_cast<uint32_t>(a.Nmax), a.fd_nmax, a.node_count);
    }
    if (it.argmax) argmax_item<DT, 4, VecOk>(am, it.row, static_cast<int>(it.ch));
    else if (it.resolve) tree_dyn_resolve_item(a, am, static_cast<int>(it.row));
}

template <class DT, bool VecOk>
__global__ __launch_bounds__(kWG) void k_greedy(GreedyArgs a) {
    // The argument block stays untouched (writing into it would copy it to
    // scratch); the argmax arguments with the call's tag are a local copy.
    ArgmaxArgs am = a.am;
    if (am.tag_src) am.tag = *am.tag_src;  // a graph replay's tag
    // The argmax items' arguments in one batch ahead of the decode, so no
    // second round of argument loads stands before the first logit load.
    asm volatile("" ::"s"(a.am.logits), "s"(a.am.V), "s"(a.am.chunk), "s"(a.am.partial), "s"(a.am.tag));
    const ArgmaxItem it = argmax_item_of(blockIdx.x, a.am.nchunk, a.am.fd_nch, static_cast<uint32_t>(a.am.rows));
    argmax_item<DT, 4, VecOk>(am, it.row, static_cast<int>(it.ch));
    uint32_t b;
    if (argmax_resolves(it.row, it.ch, a.am.nchunk, static_cast<uint32_t>(a.K) + 1, a.fd_per, b))
        greedy_resolve_item(a, am, static_cast<int>(b));
}

template <class DT, bool VecOk, bool NodeMajor>
__global__ __launch_bounds__(kWG) void k_tree(TreeArgs a) {
    // The items' arguments in one batch ahead of everything else, so no
    // second round of argument loads stands before the first logit load.
    if constexpr (NodeMajor)
        asm volatile("" ::"s"(a.am.logits), "s"(a.am.V), "s"(a.am.chunk), "s"(a.am.partial),
                     "s"(a.am.tag), "s"(a.am.tag_src), "s"(a.am.nchunk), "s"(a.tree.N), "s"(a.gate),
                     "s"(a.gate_from));
    // The argument block stays untouched (writing into it would copy it to
    // scratch); the argmax arguments with the call's tag are a local copy.
    ArgmaxArgs am = a.am;
    if (am.tag_src) am.tag = *am.tag_src;  // a graph replay's tag
    asm volatile("" ::"s"(a.am.logits), "s"(a.am.V), "s"(a.am.chunk), "s"(a.am.partial), "s"(a.am.tag));
    if constexpr (NodeMajor) {
        // Grid (chunks + 1) x trees x nodes: x < nchunk a chunk item of row
        // (y, z), x = nchunk the resolver of node z of tree y.
        const int b = static_cast<int>(blockIdx.y), v = static_cast<int>(blockIdx.z);
        const int ch = static_cast<int>(blockIdx.x);
        if (ch < am.nchunk) {
            if (v >= a.gate_from && node_not_needed(a, am.tag, b, v)) return;
            argmax_item<DT, 4, VecOk>(am, static_cast<int64_t>(b) * a.tree.N + v, ch);
        } else {
            node_resolver_item(a, am, b, v);
        }
        return;
    }
    const ArgmaxItem it = argmax_item_of(blockIdx.x, a.am.nchunk, a.am.fd_nch, static_cast<uint32_t>(a.am.rows));
    argmax_item<DT, 4, VecOk>(am, it.row, static_cast<int>(it.ch));
    uint32_t b;
    if (argmax_resolves(it.row, it.ch, a.am.nchunk, static_cast<uint32_t>(a.tree.N), a.fd_per, b))
        tree_resolve_item(a, am, static_cast<int>(b));
}

}  // namespace

hipError_t launch_greedy(const GreedyArgs &a, int dtype, hipStream_t s) {
    const dim3 g(argmax_only_grid(a.am.rows, a.am.nchunk)), blk(kWG);
    const bool vec = a.am.V % (dtype == 1 ? Bf16::kVec : F32::kVec) == 0;
    if (dtype == 1) {
        if (vec) k_greedy<Bf16, true><<<g, blk, 0, s>>>(a);
        else k_greedy<Bf16, false><<<g, blk, 0, s>>>(a);
    } else {
        if (vec) k_greedy<F32, true><<<g, blk, 0, s>>>(a);
        else k_greedy<F32, false><<<g, blk, 0, s>>>(a);
    }
    return hipGetLastError();
}

template <class DT, bool VecOk>
void launch_tree_order(const TreeArgs &a, hipStream_t s) {
    if (a.node_major) {
        const Grid3 g = tree_node_major_grid(a.am.nchunk, a.B, a.tree.N);
        k_tree<DT, VecOk, true><<<dim3(g.x, g.y, g.z), kWG, 0, s>>>(a);
    } else {
        k_tree<DT, VecOk, false><<<dim3(argmax_only_grid(a.am.rows, a.am.nchunk)), kWG, 0, s>>>(a);
    }
}

hipError_t launch_tree(const TreeArgs &a, int dtype, hipStream_t s) {
    const bool vec = a.am.V % (dtype == 1 ? Bf16::kVec : F32::kVec) == 0;
    if (dtype == 1) {
        if (vec) launch_tree_order<Bf16, true>(a, s);
        else launch_tree_order<Bf16, false>(a, s);
    } else {
        if (vec) launch_tree_order<F32, true>(a, s);
        else launch_tree_order<F32, false>(a, s);
    }
    return hipGetLastError();
}

template <class DT, bool VecOk>
void launch_tree_dyn_order(const TreeDynArgs &a, hipStream_t s) {
    if (a.node_major) {
        const Grid3 g = tree_node_major_grid(a.am.nchunk, a.B, a.Nmax);
        k_tree_dyn<DT, VecOk, true><<<dim3(g.x, g.y, g.z), kWG, 0, s>>>(a);
    } else {
        k_tree_dyn<DT, VecOk, false><<<dim3(argmax_grid(a.am.rows, a.am.nchunk, a.B)), kWG, 0, s>>>(a);
    }
}

hipError_t launch_tree_dyn(const TreeDynArgs &a, int dtype, hipStream_t s) {
    const bool vec = a.am.V % (dtype == 1 ? Bf16::kVec : F32::kVec) == 0;
    if (dtype == 1) {
        if (vec) launch_tree_dyn_order<Bf16, true>(a, s);
        else launch_tree_dyn_order<Bf16, false>(a, s);
    } else {
        if (vec) launch_tree_dyn_order<F32, true>(a, s);
        else launch_tree_dyn_order<F32, false>(a, s);
    }
    return hipGetLastError();
}

}  // namespace sv
