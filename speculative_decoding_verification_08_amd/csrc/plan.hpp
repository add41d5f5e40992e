// Launch plans and kernel argument blocks of the verify library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace sv {

constexpr int kMaxK = 64;
constexpr int kMaxTreeNodes = 256;
constexpr int kChunk2Bytes = 16384;  // bytes of one row per chunk of the residual / bonus pass
// The chain's statistics items take 8 KB of a row each (two 16-byte vectors
// per thread).
constexpr int kStatVecs = 2;
constexpr int kStatChunkBytes = kStatVecs * 16 * 256;
constexpr int kMaxStatChunks = 128;  // statistics chunks per row: V <= 128 x 8 KB of entries
// The draws' chunks are the statistics chunks: 8 KB of a row, two 16-byte
// vectors per thread.
constexpr int kDrawChunkBytes = kStatChunkBytes;
// Workgroups of 256 threads the chip holds at once (256 CUs, 8 each): the
// top-k merges trail their rows' chunks by about this many workgroups.
constexpr int kResidentWGs = 2048;
// Chunk items (trees x node slots x chunks) from which a tree batch takes the
// node-major order, about five generations of resident workgroups.  Measured
// on 45-node trees (branching 4, 2, 2, 1) and 64-slot per-sequence trees,
// V = 128256 bf16, us per call, tree-major against node-major: 5,760 items
// 19.9 / 24.9, 8,192 items 19.2 / 24.0, 11,520 items 33.8 / 30.0.
constexpr int64_t kTreeNodeMajorItems = 5 * kResidentWGs;
constexpr int kRecWords = 8;       // words per sequence record (five used)
// The row gate of a (sequence, position), or of a tree node, is one tagged
// word alone on its 128-byte cache line.
constexpr int kGateLineBytes = 128;
constexpr int kGateLineWords = kGateLineBytes / 8;
// Outcome of one position's accept test (the low half of its tagged word).
constexpr uint32_t kPairAccept = 0, kPairReject = 1, kPairSkip = 2, kPairFail = 3;
constexpr int kMaxDrawChunks = kMaxStatChunks;  // draw chunks per row (two per lane of a wavefront)
// LDS words of a draw workgroup: its sequence's row statistics (ref, z), the
// vector searched in the crossing chunk (4 words per row, target and draft)
// and its running mass, then the bonus row's statistics (ref, z) per
// statistics chunk.
constexpr int kDrawRawAt = (2 * (2 * kMaxK + 1) + 3) / 4 * 4;  // 16-byte aligned
constexpr int kDrawBonusAt = kDrawRawAt + 12;
constexpr int kDrawLds = kDrawBonusAt + 2 * kMaxStatChunks;

// How a launch cuts the rows it streams into vocabulary chunks, and where its
// scratch lives inside the caller's workspace.
struct Plan {
    int64_t rows = 0;      // rows streamed by the first pass
    int chunk = 0;         // elements per chunk of the first pass
    int nchunk = 0;        // chunks per row, first pass
    int chunk2 = 0;        // elements per chunk, residual / bonus pass (chain)
    int nchunk2 = 0;       // chunks per row, residual / bonus pass (chain)
    size_t off_partial = 0, off_sums = 0, off_rec = 0;
    size_t off_pairs = 0;  // chain: an outcome per position; static tree: one per node
    size_t off_gate = 0;   // gate lines of the same
    size_t bytes = 0;      // total workspace
};

// Words handed between workgroups carry the call's tag in their upper 32 bits
// and a 32-bit value below; a reader checks that a word's tag is the current
// call's, so words left by earlier calls (of any shape) are never taken for
// fresh ones.  Host tags come from a process-wide counter that starts at a
// random value; they are never 0 and never have bit 31 set.
// Tags of calls recorded into a graph have bit 31 set: each replay's tag is
// advanced on the device (launch_advance_tag), in a range host tags never use.
constexpr uint32_t kGraphTagBit = 0x80000000u;
// The first 256 bytes of every workspace: three 32-bit words.
constexpr size_t kWorkspaceHeader = 256;
constexpr int kHdrGraphTag = 0;  // the tag word of calls recorded into a graph
constexpr int kHdrPhaseTag = 1;  // the tag of the statistics the last chain_stats call left
constexpr int kHdrFailures = 2;  // count of bounded waits that ran out (and stale statistics)
static_assert(kHdrFailures == 2, "count_failure writes the third header word");

// Chain verify, all kernels.
struct ChainArgs {
    const void *target;      // [B][K+1][V]
    const void *draft;       // [B][K][V]
    const int32_t *tokens;   // [B][K]
    const float *u_accept;   // [B][K]
    const float *u_sample;   // [B]
    int32_t B, K, V;
    float c;                 // log2(e) / T
    uint32_t tag;            // this call's tag (upper half of every handed-over word)
    const uint32_t *tag_src; // nullable: read the tag from this device word instead (graph replays)
    uint32_t *hdr;           // the workspace header words
    bool sample_phase;       // the draws of the two-phase form: statistics carry the phase word's tag
    int32_t chunk, nchunk, nchunk2;  // chunk2 = kChunk2Bytes / element size
    // One-launch schedule: S statistics items per sequence that do not read
    // the bonus row, D draw items per sequence; where the blocks of
    // statistics and resolvers end, and where the bonus rows' statistics end.
    uint32_t S, D, blocks_end, bon_end;
    FastDiv fd_nch, fd_D, fd_S1;
    // Position-major one-launch order (early exit, a three-dimensional grid).
    bool early_exit;
    bool gate_pos1;          // position-major statistics of position 1 also skip rows
    bool gate_bonus;         // bonus-row statistics skip rows whose sequence rejected
    uint64_t *pairs;         // [B][K] tagged outcome of each position's accept test
    uint64_t *partial;       // [B][2K+1][nchunk][2] tagged (ref, z); rows 0..K target, K+1.. draft
    uint64_t *sums;          // [B][nchunk2][2] tagged residual and target mass per chunk
    uint64_t *rec;           // [B][kRecWords] tagged record of each resolve: j, row j's (ref, 1/z) x 2
    int32_t *out_tokens;     // [B][K+1]
    int32_t *out_accepted;   // [B]
    float *out_diag;         // nullable [B][K+1][4]
    // Last: the fields before it keep the offsets of the single batch of
    // argument loads the statistics items were measured with.
    uint64_t *gate;          // [B][K] lines: position k's rows of sequence b are not needed
};

// Row argmax over rows of [rows][V], one workgroup per (row, chunk).
struct ArgmaxArgs {
    const void *logits;
    int64_t rows;
    int32_t V, chunk, nchunk;
    FastDiv fd_nch;          // division by nchunk
    uint32_t tag;            // this call's tag (upper half of every handed-over word)
    const uint32_t *tag_src; // nullable: read the tag from this device word instead (graph replays)
    uint64_t *partial;       // [rows][nchunk][2] tagged (value bits, index)
    uint32_t *hdr;           // the workspace header words
};

// Greedy chain verify in one launch: the argmax workgroups of rows
// [B][K+1]; the one of a sequence's last chunk also resolves it.
struct GreedyArgs {
    ArgmaxArgs am;
    const int32_t *tokens;   // [B][K]
    int32_t B, K;
    FastDiv fd_per;          // division by K + 1, the rows of a sequence
    int32_t *out_tokens;     // [B][K+1]
    int32_t *out_accepted;   // [B]
};

// A static tree travels by value in the kernel arguments.
struct TreeShape {
    int16_t parent[kMaxTreeNodes];
    uint8_t depth[kMaxTreeNodes];
    int32_t N, D;
};

// Greedy static-tree verify in one launch.  Tree-major: the argmax workgroups
// of node rows [B][N]; the one of a tree's last chunk also resolves it.
// Node-major: node by node, every tree's chunk items of the node and then a
// resolver per tree; a node that cannot be accepted is not read.
struct TreeArgs {
    ArgmaxArgs am;
    const int32_t *tokens;   // [B][N]
    int32_t B;
    FastDiv fd_per;          // division by N, the rows of a tree
    int32_t *out_tokens;     // [B][D+1]
    int32_t *out_path;       // nullable [B][D+1]
    int32_t *out_depth;      // [B]
    TreeShape tree;
    // Node-major order (a 3D grid: chunk and resolver, tree, node).
    uint64_t *node_out;      // [B][N] tagged outcome of each node: its argmax, or kNodeDead
    uint64_t *gate;          // [B][N] lines: node v of tree b cannot be accepted
    int32_t gate_from;       // the first node whose chunk items read their gate line
    bool node_major;         // the launch's order (read on the host only)
};

// Greedy verify on per-sequence trees in one launch.  Tree-major: the argmax
// workgroups of node rows [B][Nmax] (rows past a tree's node count skip),
// then one resolve workgroup per tree.  Node-major: as the static tree's.
struct TreeDynArgs {
    ArgmaxArgs am;
    const int32_t *tokens;      // [B][Nmax]
    const int32_t *parents;     // [B][Nmax]
    const int32_t *node_count;  // [B]
    int32_t B, Nmax;
    FastDiv fd_nmax;            // division by Nmax
    int32_t *out_tokens;        // [B][Nmax]
    int32_t *out_path;          // nullable [B][Nmax]
    int32_t *out_depth;         // [B]
    // Node-major order (a 3D grid: chunk and resolver, tree, node slot).
    uint64_t *node_out;         // [B][Nmax] tagged outcome of each node: its argmax, or kNodeDead
    uint64_t *gate;             // [B][Nmax] lines: node v of tree b cannot be accepted
    bool node_major;            // the launch's order (read on the host only)
};

// Host launchers (defined next to their kernels).
hipError_t launch_chain_stats(const ChainArgs &a, int dtype, hipStream_t s);
hipError_t launch_chain_draw(const ChainArgs &a, int dtype, hipStream_t s);
hipError_t launch_chain_fused(const ChainArgs &a, int dtype, hipStream_t s);
hipError_t launch_greedy(const GreedyArgs &a, int dtype, hipStream_t s);
hipError_t launch_tree(const TreeArgs &a, int dtype, hipStream_t s);
hipError_t launch_tree_dyn(const TreeDynArgs &a, int dtype, hipStream_t s);
hipError_t launch_advance_tag(uint32_t *word, hipStream_t s);

}  // namespace sv
