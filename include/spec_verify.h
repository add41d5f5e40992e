/*
 * spec_verify.h - the verify step of speculative sampling on MI355X (gfx950).
 *
 * Given the target model's logits at K+1 positions and the draft model's
 * logits at K positions, the chain verify accepts drafted tokens left to right
 * while u < p(x)/q(x) with p = softmax(target/T), q = softmax(draft/T); at the
 * first rejection it draws a replacement from the residual max(0, p-q)
 * normalised; if every draft is accepted it draws a bonus token from p at
 * position K+1.  At T = 0 the drafted token is compared with argmax(p), on a
 * chain or on a static candidate tree.
 *
 * Sources: the French lesson "Décodage spéculatif et Eagle" (sections "Le
 * concept", "La règle de l'exactitude", "Vérifie l'attention des arbres"), the
 * Arabic lesson "Speculative decoding: draft, verify, repeat" (steps 1 to 3 of
 * "Build it", with p and q named the other way round), and the forum post
 * "Speculative Decoding: от идеи до SOTA" (§3 acceptance and resampling rules,
 * §6 tree verification).
 *
 * Conventions shared by every entry point:
 *  - Every pointer except `parents` and `workspace_bytes`-style out-params is
 *    a DEVICE pointer owned by the caller.  The library allocates nothing
 *    (spec_verify_chain_noalloc uses a fixed array of its own instead).
 *  - Logit arrays are row-major with the vocabulary innermost and must be
 *    16-byte aligned at their base; other arrays need natural alignment.
 *  - Work is enqueued on `stream` and nothing is synchronised: outputs are
 *    valid once the stream reaches that point.  Argument errors are returned
 *    synchronously and nothing is enqueued then.  SPEC_ERR_LAUNCH reports a
 *    launch failure seen right after enqueueing.
 *  - The workspace (size from spec_verify_workspace_bytes) holds per-call
 *    scratch.  It must be zero-filled once before its first use (for
 *    example with hipMemsetAsync); after that it can serve any number of
 *    calls of any entry point and shape without clearing.  Words that
 *    workgroups hand each other carry a per-call tag (from a process-wide
 *    call counter that starts at a random value, never 0), so words left by
 *    an earlier call of this library, or zeros, are never taken for fresh
 *    ones.  Memory with other prior contents holds a word that looks fresh
 *    only by a 2^-31 chance per word, so an unzeroed workspace gives
 *    unspecified outputs.  Calls that share a workspace must be ordered on
 *    one stream.
 *  - Graph capture: every entry point can be recorded into a HIP graph.  A
 *    call made while its stream is being captured also records a one-thread
 *    kernel that advances a tag word kept in the first 256 bytes of its
 *    workspace, and its workgroups read their tag from that word, so each
 *    replay has a tag of its own (graph tags have bit 31 set; host tags never
 *    do).  Eager calls and replays may share a workspace.  The extra kernel
 *    is one more kernel boundary per recorded call (about 1-2 us on MI355X).
 *    The tree mask and the KV commit hand no words between workgroups and
 *    record one kernel.
 *  - Inputs that break a documented precondition (a drafted token outside
 *    [0, V), a uniform outside [0, 1), NaN or +inf logits, a row that is
 *    entirely -inf) give unspecified outputs but never an out-of-bounds
 *    access: token ids are clamped before they address memory.
 *  - Results are bitwise reproducible run to run (fixed reduction orders, no
 *    floating-point atomics).
 *  - The library keeps no state between calls beyond that call counter (and
 *    the device array of spec_verify_chain_noalloc) and is safe to call from
 *    several host threads.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums are 32-bit integers on both sides.  In C++ they get that fixed
 * underlying type, so every int32 value a C caller passes (a bad dtype or
 * mode included) is a valid value that the checks can reject. */
#ifdef __cplusplus
#define SPEC_ENUM_BASE : int32_t
#else
#define SPEC_ENUM_BASE
#endif

typedef enum SPEC_ENUM_BASE {
    SPEC_DTYPE_F32 = 0,  /* IEEE float32 logits                      */
    SPEC_DTYPE_BF16 = 1  /* bfloat16 logits (upper half of a float32) */
} spec_dtype;

typedef enum SPEC_ENUM_BASE {
    SPEC_MODE_CHAIN = 0,  /* spec_verify_chain (T > 0)           */
    SPEC_MODE_GREEDY = 1, /* spec_verify_greedy (T = 0, chain)   */
    SPEC_MODE_TREE = 2,   /* spec_verify_tree_greedy (T = 0)     */
    SPEC_MODE_TREE_DYN = 3, /* spec_verify_tree_greedy_dyn (T = 0) */
    SPEC_MODE_TOPK = 4      /* spec_draft_topk                     */
} spec_mode;

typedef enum SPEC_ENUM_BASE {
    SPEC_OK = 0,
    SPEC_ERR_INVALID_ARG = 1, /* a size, pointer, dtype, temperature or tree is invalid */
    SPEC_ERR_WORKSPACE = 2,   /* workspace missing or smaller than required            */
    SPEC_ERR_LAUNCH = 3,      /* the HIP runtime reported an error at enqueue          */
    SPEC_ERR_SCRATCH_LIMIT = 4 /* spec_verify_chain_noalloc: the call needs more scratch
                                  than SPEC_VERIFY_NOALLOC_SCRATCH_BYTES                 */
} spec_status;

#define SPEC_VERIFY_MAX_K 64            /* draft length limit of chain and greedy verify */
#define SPEC_VERIFY_MAX_TREE_NODES 256  /* node limit of the static tree (root included) */
#define SPEC_VERIFY_MAX_V (1 << 26)     /* vocabulary limit (greedy and tree)            */
#define SPEC_VERIFY_MAX_CHAIN_V_BF16 (1 << 19)  /* chain verify vocabulary limit, bf16 logits */
#define SPEC_VERIFY_MAX_CHAIN_V_F32 (1 << 18)   /* chain verify vocabulary limit, fp32 logits */
#define SPEC_TOPK_MAX_K 8               /* spec_draft_topk: k limit                      */
#define SPEC_TOPK_MAX_V (1 << 19)       /* spec_draft_topk: vocabulary limit             */
#define SPEC_VERIFY_NOALLOC_SCRATCH_BYTES (8u << 20) /* spec_verify_chain_noalloc's array */

/*
 * Workspace size for one call.  K_or_N is K for the chain and greedy modes,
 * N (nodes, root included) for the tree mode and Nmax for the per-sequence
 * tree mode; for SPEC_MODE_TOPK, B is the row count and K_or_N is k.  Pure
 * host arithmetic.
 * Returns SPEC_ERR_INVALID_ARG (and leaves *bytes alone) for sizes the entry
 * point would reject.
 */
spec_status spec_verify_workspace_bytes(spec_mode mode, int32_t B, int32_t K_or_N, int32_t V,
                                        spec_dtype dtype, size_t *bytes);

/*
 * Chain verify at temperature T > 0 (French lesson, "La règle de
 * l'exactitude"; forum post §3; Arabic lesson, steps 1-3).
 *
 *   target_logits [B][K+1][V]  row k < K scores drafted token k; row K is the
 *                              bonus row.
 *   draft_logits  [B][K][V]    row k is the distribution x_k was drawn from.
 *   dtype                      dtype of both logit arrays.
 *   draft_tokens  [B][K]       int32, 0 <= x < V.
 *   u_accept      [B][K]       float32 in [0,1): the accept test of position k
 *                              is u_accept[b][k] < p_k(x_k)/q_k(x_k) (strict;
 *                              q_k(x_k) = 0 accepts iff p_k(x_k) > 0).
 *   u_sample      [B]          float32 in [0,1): the one uniform of the draw
 *                              that ends the step (residual or bonus).  A draw
 *                              from weights w returns the smallest i with
 *                              w_0+...+w_i > u * sum(w).
 *   B >= 0, 0 <= K <= SPEC_VERIFY_MAX_K, T > 0, and 1 <= V <=
 *   SPEC_VERIFY_MAX_CHAIN_V_BF16 (bf16) or SPEC_VERIFY_MAX_CHAIN_V_F32 (fp32).
 *   out_tokens    [B][K+1]     int32: the first out_accepted[b]+1 entries are
 *                              the emitted tokens, the rest are -1.
 *   out_accepted  [B]          int32 j in [0, K]: accepted drafts.
 *   out_diag      nullable [B][K+1][4] float32: for k < K {p_k(x_k), q_k(x_k),
 *                              ratio, S if k == j else 0}; row K {0, 0, 0, S if
 *                              j == K else 0}.  S is the mass of the weights
 *                              the final draw used; ratio is p/q (+inf when
 *                              q = 0 < p, 0 when both are 0).
 *   workspace                  at least spec_verify_workspace_bytes(CHAIN, ...).
 *
 * One kernel launch that computes the same as spec_verify_chain_stats
 * followed by spec_verify_chain_sample, bit for bit.  Its workgroups hand
 * each other words in the workspace and wait for each other (bounded, about
 * 2 s): a sequence's accept tests wait for its statistics, its draw for its
 * accept tests, and its final draw for its chunk masses.  If a wait ever ran
 * out, the sequence gets out_accepted[b] = -1 and out_tokens[b] all -1, and
 * the workspace's failure count grows (spec_verify_workspace_failures).
 * Sizes whose one-launch grid would exceed 2^31 - 1 workgroups run as the two
 * phases instead.
 *
 * Without out_diag, and when one position's work fills the GPU, the launch
 * streams the batch position by position and publishes each position's
 * accept outcome as it goes; then the bonus row of a sequence that rejected
 * a draft, and the rows of positions after a sequence's first rejection
 * (from position 2 on, or from position 1 when one position's rows are
 * 64 MB or more), are not read once that rejection is published.  The accept rule never consults them, so the
 * outputs are the same as with every row read.  With out_diag every
 * position's p, q and ratio are computed, so every row is read.
 */
spec_status spec_verify_chain(const void *target_logits, const void *draft_logits, spec_dtype dtype,
                              const int32_t *draft_tokens, const float *u_accept,
                              const float *u_sample, int32_t B, int32_t K, int32_t V,
                              float temperature, int32_t *out_tokens, int32_t *out_accepted,
                              float *out_diag, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * First phase of the chain verify (one kernel): one streaming pass over every
 * target and draft logit that leaves each row's softmax statistics (running
 * maximum and sum of exponentials, per vocabulary chunk) in the workspace.
 * Same argument meaning as spec_verify_chain; draft_tokens is checked like
 * there, and read by the second phase.
 */
spec_status spec_verify_chain_stats(const void *target_logits, const void *draft_logits,
                                    spec_dtype dtype, const int32_t *draft_tokens, int32_t B,
                                    int32_t K, int32_t V, float temperature, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/*
 * Second phase of the chain verify (one kernel): the accept test of each
 * position, the first rejection j, the residual or bonus draw and the emitted
 * tokens, from the statistics the first phase left in the same workspace.
 * Must follow spec_verify_chain_stats with identical logits, tokens, sizes and
 * temperature on the same stream, with no other chain call on the workspace
 * in between: the statistics phase records its tag in the workspace header
 * and the sample phase reads the statistics under that tag.  Sequences whose
 * statistics were not written by that phase (no statistics phase, or another
 * call's) get out_accepted = -1 and out_tokens all -1, and each adds one to
 * the workspace's failure count; they are never drawn from other statistics.
 * The draw workgroups of one sequence wait for each other (bounded, about
 * 2 s); if a wait ran out, the sequence gets the same -1 outputs and is
 * counted.
 */
spec_status spec_verify_chain_sample(const void *target_logits, const void *draft_logits,
                                     spec_dtype dtype, const int32_t *draft_tokens,
                                     const float *u_accept, const float *u_sample, int32_t B,
                                     int32_t K, int32_t V, float temperature, int32_t *out_tokens,
                                     int32_t *out_accepted, float *out_diag, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/*
 * spec_verify_chain without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, serving loops and
 * harnesses that forbid hipMalloc).  Same arguments, outputs and kernels as
 * spec_verify_chain; the workspace is a fixed array of
 * SPEC_VERIFY_NOALLOC_SCRATCH_BYTES in the library's device memory, one copy
 * per GPU, held until the process ends.  The call allocates and frees
 * nothing.
 *
 * Returns SPEC_ERR_SCRATCH_LIMIT, before any HIP call, when
 * spec_verify_workspace_bytes(SPEC_MODE_CHAIN, B, K, V, dtype) exceeds that
 * size (B = 256, K = 8, V = 151936 fp32 needs 5.6 MiB), and
 * SPEC_ERR_INVALID_ARG for sizes spec_verify_chain rejects.  The first call on
 * a device looks up that device's copy (the current device; `stream` must
 * belong to it); SPEC_ERR_LAUNCH if that fails.
 *
 * Every call on one GPU uses the same array, which keeps the last call's
 * words.  Calls ordered on one stream (eager calls and graph replays alike)
 * need nothing cleared in between; calls that overlap on one GPU (other
 * streams, other host threads) race on the array and give unspecified
 * outputs.
 */
spec_status spec_verify_chain_noalloc(const void *target_logits, const void *draft_logits,
                                      spec_dtype dtype, const int32_t *draft_tokens,
                                      const float *u_accept, const float *u_sample, int32_t B,
                                      int32_t K, int32_t V, float temperature,
                                      int32_t *out_tokens, int32_t *out_accepted, float *out_diag,
                                      hipStream_t stream);

/*
 * Greedy chain verify, T = 0 (French lesson, "La règle de l'exactitude",
 * greedy case): a_k = argmax of target row k over raw logits (lowest index on
 * ties; -0.0 ties +0.0).  j = first k < K with x_k != a_k, else K.  Emits
 * x_0..x_{j-1}, a_j.
 *
 *   target_logits [B][K+1][V], draft_tokens [B][K] int32,
 *   out_tokens [B][K+1] (-1 padded), out_accepted [B].
 *   B >= 0, 0 <= K <= SPEC_VERIFY_MAX_K, 1 <= V <= SPEC_VERIFY_MAX_V.
 *
 * One kernel launch.  Each sequence's resolve waits (bounded, about 2 s) for
 * the argmax workgroups of its rows; if a wait ever ran out, the sequence
 * gets out_accepted[b] = -1 and out_tokens[b] all -1.
 */
spec_status spec_verify_greedy(const void *target_logits, spec_dtype dtype,
                               const int32_t *draft_tokens, int32_t B, int32_t K, int32_t V,
                               int32_t *out_tokens, int32_t *out_accepted, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * Greedy verify on a static candidate tree shared by the batch, T = 0 (French
 * lesson, "Vérifie l'attention des arbres" and the EAGLE section: one target
 * pass scores every candidate path and the longest accepted branch wins;
 * forum post §6).
 *
 *   node_logits [B][N][V]  row v is the target's distribution after the path
 *                          root..v.
 *   node_tokens [B][N]     int32 token of node v; column 0 (the root) unused.
 *   parents     [N]        HOST pointer, int32: parents[0] = -1 and
 *                          0 <= parents[v] < v (nodes in topological order).
 *   1 <= N <= SPEC_VERIFY_MAX_TREE_NODES.
 * Node v > 0 matches iff node_tokens[b][v] == argmax(row parents[v]); it is
 * accepted iff it and all its ancestors match.  The deepest accepted node
 * wins, the lowest node index among equally deep ones.  With D the tree's
 * maximum depth:
 *   out_tokens [B][D+1]    tokens of the accepted path's nodes below the root,
 *                          then the argmax of the last node's row, then -1.
 *   out_path   nullable [B][D+1]  node ids root..last, then -1.
 *   out_depth  [B]         accepted depth d (out_tokens holds d+1 tokens).
 *
 * One kernel launch.  Each tree's resolve waits (bounded, about 2 s) for the
 * argmax workgroups of its node rows; if a wait ever ran out, the tree gets
 * out_depth[b] = -1 and out_tokens[b], out_path[b] all -1.  Large batches
 * (B x N x 16 KB chunks of at least 10240) run node by node, and the row of
 * a node that can no longer be accepted (an ancestor did not match) is not
 * read; the outputs are those of reading every row.
 */
spec_status spec_verify_tree_greedy(const void *node_logits, spec_dtype dtype,
                                    const int32_t *node_tokens, const int32_t *parents,
                                    int32_t B, int32_t N, int32_t V, int32_t *out_tokens,
                                    int32_t *out_path, int32_t *out_depth, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/*
 * Greedy verify on per-sequence candidate trees, T = 0 (French lesson, EAGLE
 * section: the second version of EAGLE shapes each step's tree to the draft's
 * confidence; forum post §6).  The rule of spec_verify_tree_greedy, applied to
 * each sequence's own tree:
 *
 *   node_logits [B][Nmax][V]  row v of sequence b is the target's distribution
 *                             after the path root..v of b's tree.
 *   node_tokens [B][Nmax]     int32 token of node v; column 0 (the root) unused.
 *   parents     [B][Nmax]     DEVICE pointer, int32: parents[b][0] = -1 and
 *                             0 <= parents[b][v] < v for v < node_count[b].
 *   node_count  [B]           DEVICE pointer, int32: 1 <= node_count[b] <= Nmax.
 *   1 <= Nmax <= SPEC_VERIFY_MAX_TREE_NODES, 1 <= V <= SPEC_VERIFY_MAX_V.
 * Rows, tokens and parents at v >= node_count[b] are padding and are not read.
 * Outputs, each row padded with -1 to Nmax entries:
 *   out_tokens [B][Nmax]   tokens of the accepted path's nodes below the root,
 *                          then the argmax of the last node's row.
 *   out_path   nullable [B][Nmax]  node ids root..last.
 *   out_depth  [B]         accepted depth d (out_tokens holds d+1 tokens).
 *
 * The tree arrays live on the device, so they are not checked on the host: a
 * node count is clamped to [1, Nmax], and a node whose parent entry is out of
 * range is never accepted (nor is its subtree); no entry outside the arrays
 * is read.  One kernel launch; each tree's resolve waits (bounded, about 2 s)
 * for the argmax workgroups of its node rows; if a wait ever ran out, the tree
 * gets out_depth[b] = -1 and out_tokens[b], out_path[b] all -1.  Large
 * batches run node by node, as for spec_verify_tree_greedy, and do not read
 * the rows of nodes that can no longer be accepted.
 */
spec_status spec_verify_tree_greedy_dyn(const void *node_logits, spec_dtype dtype,
                                        const int32_t *node_tokens, const int32_t *parents,
                                        const int32_t *node_count, int32_t B, int32_t Nmax,
                                        int32_t V, int32_t *out_tokens, int32_t *out_path,
                                        int32_t *out_depth, void *workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/*
 * Per-row top-k of draft logits: the expansion step of an EAGLE-style tree
 * drafter, which grows each depth of the candidate tree from the draft's k
 * most likely tokens (French lesson, EAGLE section: 4 to 8 candidates per
 * depth; its exercises: the top three branches at each depth).  Softmax at
 * any temperature keeps the order of the logits, so the top k of the logits
 * are the top k of the draft distribution.
 *
 *   logits  [rows][V]   bf16 or fp32 (dtype), 16-byte aligned.
 *   1 <= k <= SPEC_TOPK_MAX_K, k <= V <= SPEC_TOPK_MAX_V, rows >= 0.
 *   out_idx [rows][k]   int32: the k entries of largest value, by value
 *                       descending, equal values by index ascending (values
 *                       compare as floats, so -0.0 ties +0.0).
 *   out_val nullable [rows][k]  float32: their values.
 *   workspace           at least spec_verify_workspace_bytes(TOPK, rows, k, V).
 *
 * NaN logits give unspecified outputs (never an out-of-bounds access).  One
 * kernel launch: a workgroup per (row, 16 KB of the row) leaves its k best,
 * and the row's last workgroup to finish merges them.  The merge waits
 * (bounded, about 2 s) for each list entry to carry the call's tag; if a
 * wait ever ran out the row gets out_idx = -1 (and out_val = NaN).
 */
spec_status spec_draft_topk(const void *logits, spec_dtype dtype, int32_t rows, int32_t V,
                            int32_t k, int32_t *out_idx, float *out_val, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * KV commit after verify (Arabic lesson, section on rolling the KV cache back,
 * its key-terms entry "KV rollback", and its rollback exercise; forum post
 * §10 on the cost of rolling the target's cache back).  The verifier's
 * forward writes every drafted position's keys and values to a scratch
 * buffer; this call copies the accepted ones, in order, to the end of each
 * sequence's cache and reports the new lengths.  Rejected entries are simply
 * not copied.
 *
 *   scratch  [planes][B][N][row_bytes]  DEVICE, 16-byte aligned: one row per
 *                                       scratch position (a chain's drafts, or a
 *                                       tree's nodes in the order the verify
 *                                       numbers them).
 *   cache    [planes][B][S][row_bytes]  DEVICE, 16-byte aligned; must not overlap
 *                                       scratch.
 *   planes   >= 1: e.g. 2 x layers (keys and values of each layer).
 *   row_bytes  a positive multiple of 16 (heads x head_dim x element size).
 *   path     nullable DEVICE [B][P] int32: scratch row of the i-th committed
 *            entry, e.g. out_path of spec_verify_tree_greedy(_dyn) (root
 *            included).  NULL means row i (a chain), and then P = N.
 *   count    DEVICE [B] int32: entries to commit, e.g. out_depth + 1 for a
 *            tree, or the accepted count (plus one if scratch row 0 holds the
 *            step's first input) for a chain.
 *   cache_len DEVICE [B] int32: slots in use before the commit.
 *   new_len  DEVICE [B] int32: slots in use after it; must not alias cache_len.
 *
 * Sequence b is committed iff 0 <= count[b] <= P, 0 <= cache_len[b],
 * cache_len[b] + count[b] <= S and every path[b][i], i < count[b], lies in
 * [0, N): then for every plane, slot cache_len[b] + i receives scratch row
 * path[b][i], and new_len[b] = cache_len[b] + count[b].  Otherwise nothing of
 * b is written and new_len[b] = cache_len[b] (the device arrays cannot be
 * checked on the host).  One kernel launch; no workspace.
 */
spec_status spec_kv_commit(const void *scratch, void *cache, int32_t planes, int32_t B, int32_t N,
                           int32_t S, int64_t row_bytes, const int32_t *path, int32_t P,
                           const int32_t *count, const int32_t *cache_len, int32_t *new_len,
                           hipStream_t stream);

/*
 * Tree attention mask for the verify forward (French lesson, section on
 * verifying a tree with attention: each drafted token attends only to its
 * ancestors in the tree, so the whole tree is verified in one forward; forum
 * post §10: this needs custom masks and position ids).  Per sequence and
 * node, the packed set of nodes the node attends to (itself and its
 * ancestors) and its depth (its position id is the cache length plus the
 * depth).
 *
 *   parents    DEVICE [B][N] int32, the numbering of spec_verify_tree_greedy(_dyn):
 *              node v > 0 is attached when 0 <= parents[b][v] < v and its
 *              parent is attached; node 0 is the root.
 *   node_count nullable DEVICE [B] int32: nodes v >= node_count[b] are padding
 *              (clamped to [1, N]); NULL means N for every sequence.
 *   1 <= N <= SPEC_VERIFY_MAX_TREE_NODES.
 *   mask       DEVICE [B][N][ceil(N/32)] uint32: for an attached node v, bit j % 32
 *              of word j / 32 is set iff j == v or j is an ancestor of v; the rows
 *              of padding and unattached nodes are all zero.
 *   depth      DEVICE [B][N] int32: the number of ancestors, -1 for padding and
 *              unattached nodes.
 * One kernel launch; no workspace.
 */
spec_status spec_tree_mask(const int32_t *parents, const int32_t *node_count, int32_t B, int32_t N,
                           uint32_t *mask, int32_t *depth, hipStream_t stream);

/*
 * Failures recorded in a workspace.  The verify kernels wait for each other
 * within a launch, and each wait is bounded (about 2 s).  A wait that runs
 * out leaves -1 in the outputs of its sequence (tree, or top-k row) and adds
 * one to a counter in the workspace header.  The same happens for every
 * sequence of spec_verify_chain_sample when the workspace holds no statistics
 * from spec_verify_chain_stats for its call.  So the counter is 0 as long as
 * every output written through this workspace is valid.
 *
 *   workspace, workspace_bytes  a workspace of any entry point (at least 256
 *                               bytes: the header).
 *   reset                       nonzero: set the counter back to 0 after
 *                               reading it.
 *   failures                    HOST pointer: receives the counter.
 *
 * Enqueues a 4-byte device-to-host copy (and, with reset, a 4-byte clear) on
 * `stream` and synchronises that stream, so it must not be called while the
 * stream is being captured.  Returns SPEC_ERR_INVALID_ARG for a missing or
 * too small workspace, SPEC_ERR_LAUNCH if the runtime reports an error.
 */
spec_status spec_verify_workspace_failures(void *workspace, size_t workspace_bytes, int32_t reset,
                                           uint32_t *failures, hipStream_t stream);

/* Static text for a status code. */
const char *spec_verify_status_string(spec_status status);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
