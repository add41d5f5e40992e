// Launch plans and kernel argument blocks of the verify library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxK = 64;
constexpr int kMaxTreeNodes = 256;
constexpr int kChunk2Bytes = 16384;  // bytes of one row per chunk of the residual / bonus pass
constexpr int kMergeLds = 1024;  // row partials merged through LDS up to this many
constexpr int kSumsLds = 2048;   // chunk masses staged in LDS up to this many

// How a launch cuts the rows it streams into vocabulary chunks, and where its
// scratch lives inside the caller's workspace.
struct Plan {
    int64_t rows = 0;      // rows streamed by the first pass
    int chunk = 0;         // elements per chunk of the first pass
    int nchunk = 0;        // chunks per row, first pass
    int chunk2 = 0;        // elements per chunk, residual / bonus pass (chain)
    int nchunk2 = 0;       // chunks per row, residual / bonus pass (chain)
    size_t off_partial = 0, off_gather = 0, off_sums = 0, off_seq = 0;
    size_t bytes = 0;      // total workspace
};

// Words handed between workgroups carry the call's tag in their upper 32 bits
// and a 32-bit value below; a reader accepts a word only when its tag is the
// current call's.  Stale words from earlier calls (of any shape) are
// therefore never taken for fresh ones, and the workspace needs no clearing.
//
// What a sequence's first mass item hands its finishing item.
struct SeqInfo {
    uint64_t j;              // first rejected position, K if none
    uint64_t rt, izt;        // reference and 1/Z of target row j
    uint64_t rd, izd;        // reference and 1/Z of draft row j (j < K)
    uint64_t timeout;        // value 1: a wait of this sequence ran out
    uint64_t P[kMaxK], Q[kMaxK];  // p_k(x_k), q_k(x_k) for the diagnostics
};
constexpr uint32_t kPhasedTag = 1;  // tag of the phase entry points; fused calls use >= 2

// Chain verify, both phases.
struct ChainArgs {
    const void *target;      // [B][K+1][V]
    const void *draft;       // [B][K][V]
    const int32_t *tokens;   // [B][K]
    const float *u_accept;   // [B][K]
    const float *u_sample;   // [B]
    int32_t B, K, V;
    float c;                 // log2(e) / T
    uint32_t tag;            // this call's tag (upper half of every handed-over word)
    int32_t chunk, nchunk, nchunk2;  // chunk2 = kChunk2Bytes / element size
    uint64_t *partial;       // [B][2K+1][nchunk][2] tagged (ref, z); rows 0..K target, K+1.. draft
    uint64_t *gathered;      // [B][2K+1] tagged logit of each row at its drafted token (row K unused)
    uint64_t *sums;          // [B][nchunk2] tagged draw mass per chunk
    SeqInfo *seq;            // [B]
    int32_t *out_tokens;     // [B][K+1]
    int32_t *out_accepted;   // [B]
    float *out_diag;         // nullable [B][K+1][4]
};

constexpr int kFusedResidentWGs = 4096;  // workgroups in flight the fused order plans for
enum ChainKind { kItemStats = 0, kItemResolve = 1, kItemMass = 2, kItemFinish = 3 };

// Work order of a fused kernel.  Item kinds 0..kKinds-1 (for the chain:
// statistics, resolve, mass, finish) come in rounds: round s holds, kind by
// kind, the n[i] items of sequence s - lag[i] (when that sequence exists).
// With lag[0] = 0 <= lag[1] <= ... an item's inputs, produced by earlier
// kinds of the same sequence, always sit at lower workgroup indices, so a
// sequence's later work overlaps the streaming of later sequences.  Rounds
// of equal make-up form segments, decoded with a short scan.
constexpr int kKinds = 4;
constexpr int kMaxSegments = 2 * kKinds + 2;
struct FusedPlan {
    int32_t B;
    int32_t n[kKinds], lag[kKinds];
    int32_t nseg;
    int64_t seg_t0[kMaxSegments];   // first workgroup of the segment
    int32_t seg_s0[kMaxSegments];   // first round of the segment
    int32_t seg_size[kMaxSegments]; // workgroups per round in the segment
    int32_t seg_mask[kMaxSegments]; // kinds present in its rounds
    int64_t total;
};

// n[i] items per sequence of kind i, lags non-decreasing from lag[0] = 0.
__host__ inline FusedPlan make_fused_plan(int32_t B, const int32_t *n, const int32_t *lag) {
    FusedPlan f;
    f.B = B;
    int32_t cuts[2 * kKinds + 1];
    int nc = 0;
    for (int i = 0; i < kKinds; ++i) {
        f.n[i] = n[i];
        f.lag[i] = lag[i];
        cuts[nc++] = lag[i];
        cuts[nc++] = B + lag[i];
    }
    // sorted unique cut rounds
    for (int i = 1; i < nc; ++i)
        for (int k = i; k > 0 && cuts[k - 1] > cuts[k]; --k) {
            const int32_t t = cuts[k];
            cuts[k] = cuts[k - 1];
            cuts[k - 1] = t;
        }
    int m = 0;
    for (int i = 0; i < nc; ++i)
        if (m == 0 || cuts[m - 1] != cuts[i]) cuts[m++] = cuts[i];
    int64_t t = 0;
    f.nseg = 0;
    for (int g = 0; g + 1 < m; ++g) {
        const int32_t s0 = cuts[g], s1 = cuts[g + 1];
        int32_t size = 0, mask = 0;
        for (int i = 0; i < kKinds; ++i)
            if (n[i] > 0 && lag[i] <= s0 && s0 < B + lag[i]) {
                size += n[i];
                mask |= 1 << i;
            }
        f.seg_t0[f.nseg] = t;
        f.seg_s0[f.nseg] = s0;
        f.seg_size[f.nseg] = size;
        f.seg_mask[f.nseg] = mask;
        ++f.nseg;
        t += static_cast<int64_t>(size) * (s1 - s0);
    }
    f.total = t;
    return f;
}

// Item of workgroup t: kind, sequence and index among that kind's items.
__host__ __device__ inline void fused_item(const FusedPlan &f, int64_t t, int &kind, int &seq,
                                           int &idx) {
    int g = 0;
    while (g + 1 < f.nseg && t >= f.seg_t0[g + 1]) ++g;
    const int64_t u = t - f.seg_t0[g];
    const int32_t s = f.seg_s0[g] + static_cast<int32_t>(u / f.seg_size[g]);
    int32_t o = static_cast<int32_t>(u % f.seg_size[g]);
    kind = 0;
    seq = 0;
    idx = 0;
    for (int i = 0; i < kKinds; ++i) {
        if (!(f.seg_mask[g] >> i & 1)) continue;
        if (o < f.n[i]) {
            kind = i;
            seq = s - f.lag[i];
            idx = o;
            return;
        }
        o -= f.n[i];
    }
}

// Row argmax over rows of [rows][V].
struct ArgmaxArgs {
    const void *logits;
    int64_t rows;
    int32_t V, chunk, nchunk;
    int2 *partial;           // [rows][nchunk] (value bits, index)
};

struct GreedyArgs {
    const int2 *partial;     // [B][K+1][nchunk]
    const int32_t *tokens;   // [B][K]
    int32_t B, K, nchunk;
    int32_t *out_tokens;
    int32_t *out_accepted;
};

// A static tree travels by value in the kernel arguments.
struct TreeShape {
    int16_t parent[kMaxTreeNodes];
    uint8_t depth[kMaxTreeNodes];
    int32_t N, D;
};

struct TreeArgs {
    const int2 *partial;     // [B][N][nchunk]
    const int32_t *tokens;   // [B][N]
    int32_t B, nchunk;
    int32_t *out_tokens;     // [B][D+1]
    int32_t *out_path;       // nullable [B][D+1]
    int32_t *out_depth;      // [B]
    TreeShape tree;
};

// Host launchers (defined next to their kernels).
hipError_t launch_chain_stats(const ChainArgs &a, int dtype, hipStream_t s);
hipError_t launch_chain_sample(const ChainArgs &a, int dtype, hipStream_t s);  // mass + finish
hipError_t launch_chain_fused(const ChainArgs &a, const FusedPlan &f, int dtype, hipStream_t s);
hipError_t launch_zero_words(uint32_t *p, int64_t n, hipStream_t s);
hipError_t launch_row_argmax(const ArgmaxArgs &a, int dtype, hipStream_t s);
hipError_t launch_greedy_resolve(const GreedyArgs &a, hipStream_t s);
hipError_t launch_tree_resolve(const TreeArgs &a, hipStream_t s);

}  // namespace sv
