// Launch plans and kernel argument blocks of the verify library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxK = 64;
constexpr int kMaxTreeNodes = 256;
constexpr int kChunk2Bytes = 16384;  // bytes of one row per chunk of the residual / bonus pass
// Workgroups of 256 threads the chip holds at once (256 CUs, 8 each) and the
// last-level (Infinity) cache in front of HBM.  The one-launch chain verify
// places a sequence's draw at least one resident window after its
// statistics, and close enough that the draw's second read of row j still
// finds it in that cache.
constexpr int kResidentWGs = 2048;
constexpr int64_t kLlcBytes = 256ll << 20;
constexpr int kMaxDrawChunks = 64;  // draw chunks per row: V <= 64 x 16 KB of entries
// LDS words of a draw workgroup: its sequence's row statistics (ref, z), one
// thread's raw entries of the crossing chunk (16 words per row, target and
// draft) and that thread's running mass, then the bonus row's per-chunk
// statistics (ref, z).
constexpr int kDrawRawWords = 16;
constexpr int kDrawRawAt = (2 * (2 * kMaxK + 1) + 3) / 4 * 4;  // 16-byte aligned
constexpr int kDrawBonusAt = kDrawRawAt + 2 * kDrawRawWords + 4;
constexpr int kDrawLds = kDrawBonusAt + 2 * kMaxDrawChunks;

// How a launch cuts the rows it streams into vocabulary chunks, and where its
// scratch lives inside the caller's workspace.
struct Plan {
    int64_t rows = 0;      // rows streamed by the first pass
    int chunk = 0;         // elements per chunk of the first pass
    int nchunk = 0;        // chunks per row, first pass
    int chunk2 = 0;        // elements per chunk, residual / bonus pass (chain)
    int nchunk2 = 0;       // chunks per row, residual / bonus pass (chain)
    size_t off_partial = 0, off_sums = 0;
    size_t bytes = 0;      // total workspace
};

// Words handed between workgroups carry the call's tag in their upper 32 bits
// and a 32-bit value below; a reader checks that a word's tag is the current
// call's, so words left by earlier calls (of any shape) are never taken for
// fresh ones.
constexpr uint32_t kPhasedTag = 1;  // tag of the phase entry points; whole calls use >= 2
// Tags of calls recorded into a graph have bit 31 set: each replay's tag is
// advanced on the device (launch_advance_tag), in a range host tags never use.
constexpr uint32_t kGraphTagBit = 0x80000000u;
constexpr size_t kWorkspaceHeader = 256;  // bytes at the start of every workspace: the graph tag word

// Chain verify, both kernels.
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
    int32_t chunk, nchunk, nchunk2;  // chunk2 = kChunk2Bytes / element size
    int32_t lag;             // one-launch form: sequences between a sequence's statistics and its draw
    uint64_t *partial;       // [B][2K+1][nchunk][2] tagged (ref, z); rows 0..K target, K+1.. draft
    uint64_t *sums;          // [B][nchunk2][2] tagged residual and target mass per chunk
    int32_t *out_tokens;     // [B][K+1]
    int32_t *out_accepted;   // [B]
    float *out_diag;         // nullable [B][K+1][4]
};

// Row argmax over rows of [rows][V], one workgroup per (row, chunk).
struct ArgmaxArgs {
    const void *logits;
    int64_t rows;
    int32_t V, chunk, nchunk;
    uint32_t tag;            // this call's tag (upper half of every handed-over word)
    const uint32_t *tag_src; // nullable: read the tag from this device word instead (graph replays)
    uint64_t *partial;       // [rows][nchunk][2] tagged (value bits, index)
};

// Greedy chain verify in one launch: the argmax workgroups of rows
// [B][K+1], then one resolve workgroup per sequence.
struct GreedyArgs {
    ArgmaxArgs am;
    const int32_t *tokens;   // [B][K]
    int32_t B, K;
    int32_t *out_tokens;     // [B][K+1]
    int32_t *out_accepted;   // [B]
};

// A static tree travels by value in the kernel arguments.
struct TreeShape {
    int16_t parent[kMaxTreeNodes];
    uint8_t depth[kMaxTreeNodes];
    int32_t N, D;
};

// Greedy static-tree verify in one launch: the argmax workgroups of node rows
// [B][N], then one resolve workgroup per tree.
struct TreeArgs {
    ArgmaxArgs am;
    const int32_t *tokens;   // [B][N]
    int32_t B;
    int32_t *out_tokens;     // [B][D+1]
    int32_t *out_path;       // nullable [B][D+1]
    int32_t *out_depth;      // [B]
    TreeShape tree;
};

// Greedy verify on per-sequence trees in one launch: the argmax workgroups of
// node rows [B][Nmax] (rows past a tree's node count skip), then one resolve
// workgroup per tree.
struct TreeDynArgs {
    ArgmaxArgs am;
    const int32_t *tokens;      // [B][Nmax]
    const int32_t *parents;     // [B][Nmax]
    const int32_t *node_count;  // [B]
    int32_t B, Nmax;
    int32_t *out_tokens;        // [B][Nmax]
    int32_t *out_path;          // nullable [B][Nmax]
    int32_t *out_depth;         // [B]
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
