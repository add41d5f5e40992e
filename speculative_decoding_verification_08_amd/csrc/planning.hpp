// Host planning of every launch: chunk sizes, the workspace layout and the
// fields of the one-launch schedules.  Shared by the C ABI and the host check
// of the grid orders, so both plan a launch the same way.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "plan.hpp"
#include "spec_verify.h"
#include "topk.hpp"

namespace sv {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Elements per chunk of the streaming pass: 16 KB of logits per workgroup.
// Smaller chunks for small grids measured slower on MI355X (each workgroup's
// reduce and hand-over is a fixed cost), so the size does not depend on the
// grid.
inline int first_pass_chunk(spec_dtype dtype) { return dtype == SPEC_DTYPE_BF16 ? 8192 : 4096; }

inline bool valid_dtype(spec_dtype d) { return d == SPEC_DTYPE_F32 || d == SPEC_DTYPE_BF16; }

inline bool valid_sizes(spec_mode mode, int32_t B, int32_t KN, int32_t V) {
    if (B < 0 || V < 1 || V > SPEC_VERIFY_MAX_V) return false;
    if (mode == SPEC_MODE_TOPK) return KN >= 1 && KN <= SPEC_TOPK_MAX_K && KN <= V && V <= SPEC_TOPK_MAX_V;
    if (mode == SPEC_MODE_TREE || mode == SPEC_MODE_TREE_DYN)
        return KN >= 1 && KN <= SPEC_VERIFY_MAX_TREE_NODES;
    return KN >= 0 && KN <= SPEC_VERIFY_MAX_K;
}

inline bool make_plan(spec_mode mode, int32_t B, int32_t KN, int32_t V, spec_dtype dtype, Plan &p) {
    if (!valid_sizes(mode, B, KN, V) || !valid_dtype(dtype)) return false;
    int64_t rows;
    if (mode == SPEC_MODE_CHAIN) rows = static_cast<int64_t>(B) * (2 * KN + 1);
    else if (mode == SPEC_MODE_GREEDY) rows = static_cast<int64_t>(B) * (KN + 1);
    else if (mode == SPEC_MODE_TOPK) rows = B;
    else rows = static_cast<int64_t>(B) * KN;
    p.rows = rows;
    p.chunk = mode == SPEC_MODE_CHAIN ? kStatChunkBytes / (dtype == SPEC_DTYPE_BF16 ? 2 : 4)
                                      : first_pass_chunk(dtype);
    p.nchunk = (V + p.chunk - 1) / p.chunk;
    if (rows * p.nchunk > 0x7fffffffLL) return false;  // one-dimensional grid
    size_t off = kWorkspaceHeader;  // the graph tag word comes first
    p.off_partial = off;
    if (mode == SPEC_MODE_CHAIN) {
        off += align_up(static_cast<size_t>(rows) * p.nchunk * 16);
        p.chunk2 = kDrawChunkBytes / (dtype == SPEC_DTYPE_BF16 ? 2 : 4);
        p.nchunk2 = (V + p.chunk2 - 1) / p.chunk2;
        // The bonus draw takes a draw chunk's mass from the statistics of the
        // same chunk, and a finisher holds two chunks' masses per lane.
        if (p.chunk2 != p.chunk || p.nchunk > kMaxStatChunks || p.nchunk2 > kMaxDrawChunks)
            return false;
        if (static_cast<int64_t>(B) * p.nchunk2 > 0x7fffffffLL) return false;
        p.off_sums = off;  // two tagged masses per chunk: residual, target
        off += align_up(static_cast<size_t>(B) * p.nchunk2 * 16);
        p.off_rec = off;   // one record per sequence
        off += align_up(static_cast<size_t>(B) * kRecWords * 8);
        p.off_pairs = off;  // one tagged outcome per position
        off += align_up(static_cast<size_t>(B) * KN * 8);
        p.off_gate = off;   // one cache line per (sequence, position)
        off += align_up(static_cast<size_t>(B) * KN * kGateLineBytes);
    } else if (mode == SPEC_MODE_TOPK) {
        // One launch: a workgroup per (row, chunk) and a merge workgroup per
        // row (one wavefront holds the row's chunk maxima, two per lane).
        p.chunk = kChunk2Bytes / (dtype == SPEC_DTYPE_BF16 ? 2 : 4);
        p.nchunk = (V + p.chunk - 1) / p.chunk;
        if (p.nchunk > kTopkMaxChunks) return false;
        if (rows * p.nchunk + (rows + 3) / 4 > 0x7fffffffLL) return false;
        off += align_up(static_cast<size_t>(rows) * p.nchunk * kMaxTopK * 16);
    } else {
        // One launch: argmax workgroups (and, for per-sequence trees, one
        // resolve workgroup per tree after them).
        if (rows * p.nchunk + B > 0x7fffffffLL) return false;
        off += align_up(static_cast<size_t>(rows) * p.nchunk * 16);  // two tagged words
        if (mode == SPEC_MODE_TREE || mode == SPEC_MODE_TREE_DYN) {
            p.off_pairs = off;  // the node-major order: one tagged outcome per node
            off += align_up(static_cast<size_t>(rows) * 8);
            p.off_gate = off;   // and one gate line per node
            off += align_up(static_cast<size_t>(rows) * kGateLineBytes);
        }
    }
    p.bytes = off > 0 ? off : kAlign;
    return true;
}

// The chain's per-sequence item counts: S statistics items over the rows the
// accept tests read, D draw items (one per draw chunk).
inline void chain_grid_fields(const Plan &plan, int32_t K, ChainArgs &a) {
    a.S = static_cast<uint32_t>(2 * K) * plan.nchunk;
    a.D = plan.nchunk2;
    a.fd_nch = make_fastdiv(plan.nchunk);
    a.fd_D = make_fastdiv(a.D);
}

// The one-launch schedule (chain_fused_item): where its segments end, and
// its grid size, or 0 if it would not fit a one-dimensional grid.
inline uint32_t chain_schedule(ChainArgs &a) {
    const uint64_t B = a.B, S = a.S, D = a.D, nch = a.nchunk;
    const uint64_t total = B * (S + D + nch + 3);
    if (total > 0x7fffffffull) return 0;
    a.fd_S1 = make_fastdiv(static_cast<uint32_t>(S + 1));
    a.blocks_end = static_cast<uint32_t>(S + (B - 1) * (S + 1));
    a.bon_end = static_cast<uint32_t>(a.blocks_end + 1 + B * nch);
    return static_cast<uint32_t>(total);
}

// The position-major grid (chain_pm_grid), if the shape can take it: K >= 2,
// B within the grid's y dimension (gfx950 reports at most 65536; B <= 65535
// is taken), the tail within its two
// slabs, and every flattened index below 2^31 (the tail decode divides
// them).  Returns the number of workgroups, or 0.
inline uint32_t chain_pm_schedule(const ChainArgs &a) {
    const uint64_t B = a.B, K = a.K, nch = a.nchunk, D = a.D, X = 2 * nch + 1;
    if (K < 2 || B > 65535) return 0;
    if (nch + D + 2 > 2 * X) return 0;
    const uint64_t total = X * B * (K + 2);
    if (total > 0x7fffffffull) return 0;
    return static_cast<uint32_t>(total);
}

// Top-k: a merge trails its rows' chunks by about one resident window of
// workgroups (plus a group of rows), so its lists are usually complete on
// arrival.  Units: groups of four rows, one merge workgroup each.
inline int64_t topk_lag(int64_t rows, int32_t nchunk) {
    const int64_t groups = (rows + 3) / 4, group_wgs = 4 * static_cast<int64_t>(nchunk);
    return std::min<int64_t>(groups, (kResidentWGs + group_wgs - 1) / group_wgs + 1);
}

}  // namespace sv
