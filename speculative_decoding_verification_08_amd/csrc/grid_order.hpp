// Grid orders of the one-launch kernels: which item each workgroup runs.
//
// The kernels hand words between workgroups and wait for them (bounded), so
// each order must place every item after the items it waits for: the
// hardware dispatches workgroups in index order, and a workgroup that waits
// only for lower indices waits for workgroups already running or done.  The
// decodes are host and device code alike, so a host program can walk every
// workgroup of a launch through the same arithmetic the kernels run and check
// coverage, that order and the bounds of every index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace sv {

// ------------------------------------------------------------------ chain verify

enum ChainItemKind : int {
    kItemStats = 0,       // statistics of (row, chunk) among the rows the accept tests read
    kItemResolver = 1,    // accept tests of one sequence, j, row j's statistics
    kItemDraw = 2,        // residual (or target) mass of one chunk of row j
    kItemFinisher = 3,    // the residual draw of one sequence
    kItemBonusStats = 4,  // statistics of one chunk of the bonus row
    kItemBonus = 5,       // the bonus draw of one sequence (when j = K)
    kItemPair = 6,        // the accept test of one position of one sequence
    kItemNone = 7,        // an empty slot of a three-dimensional grid
};

struct ChainItem {
    int kind;
    uint32_t b;  // sequence
    uint32_t p;  // kItemStats: index among the sequence's S items; kItemDraw,
                 // kItemBonusStats: chunk; kItemPair: position; else 0
};

// The one-launch order (k_chain_fused).  Per sequence: S = 2K nchunk
// statistics items, a resolver, nchunk bonus-row statistics items, D draw
// items, a finisher and a bonus item, laid out as
//   block k   the statistics of sequence k, then the resolver of k - 1;
//   then      the resolver of B - 1;
//   bonus     the bonus rows' statistics, sequence by sequence;
//   tail      every draw item, every finisher, every bonus item.
__host__ __device__ __forceinline__ ChainItem chain_fused_item(uint32_t g, const ChainArgs &a) {
    const uint32_t S = a.S, D = a.D, B = a.B;
    ChainItem it{kItemStats, 0, 0};
    if (g < S) {
        it.p = g;
    } else if (g < a.blocks_end) {
        const uint32_t h = g - S, kk = fdiv(h, a.fd_S1), q = h - kk * (S + 1);
        it.kind = q < S ? kItemStats : kItemResolver;
        it.b = q < S ? kk + 1 : kk;
        it.p = q;
    } else if (g == a.blocks_end) {
        it.kind = kItemResolver;
        it.b = B - 1;
    } else if (g < a.bon_end) {
        const uint32_t h = g - a.blocks_end - 1;
        it.b = fdiv(h, a.fd_nch);
        it.p = h - it.b * a.nchunk;
        it.kind = kItemBonusStats;
    } else {
        const uint32_t h = g - a.bon_end;
        if (h < B * D) {
            it.kind = kItemDraw;
            it.b = fdiv(h, a.fd_D);
            it.p = h - it.b * D;
        } else if (h - B * D < B) {
            it.kind = kItemFinisher;
            it.b = h - B * D;
        } else {
            it.kind = kItemBonus;
            it.b = h - B * D - B;
        }
    }
    return it;
}

// Workgroups of the one-launch grid and of the draws of the two-phase form.
inline uint32_t chain_fused_grid(const ChainArgs &a) {
    return a.bon_end + static_cast<uint32_t>(a.B) * (a.D + 2);
}
inline uint32_t chain_draw_grid(const ChainArgs &a) { return static_cast<uint32_t>(a.B) * (a.D + 3); }

// The position-major one-launch order (k_chain_fused with early exit), for
// K >= 2, on a three-dimensional grid of X = 2 nchunk + 1 by B by K + 2
// workgroups, handed out x fastest, then y, then z (flattened index
// g = (z B + y) X + x).  Slab z < K is position z: its row y holds the
// statistics of target row z and draft row z of sequence y (x < 2 nchunk),
// then that sequence's pair resolver of position z (x = 2 nchunk):
//   [seq 0: L0 chunks, P0][seq 1: L0 chunks, P0] ... [slab 1] ... [slab K-1][tail]
// The two last slabs hold the tail in flattened order t = (z - K) B X + y X
// + x: the bonus rows' statistics, the draws, the finishers and the bonus
// items, then empty slots.  The item comes from the workgroup's three
// indices with no division in the slabs of positions (a division ahead of a
// workgroup's first load delays the stream).  A pair resolver waits for its
// two rows and for the pair resolvers of the earlier positions of its
// sequence, all of lower index.  Statistics items wait for nothing: with row
// skipping on, an item of position k >= 1 skips its chunk when an outcome
// already published for a position below k ended its sequence's accept
// tests.  A statistics item also gives its row and chunk; p is its index as
// chain_stats_row reads it (rows k and K + 1 + k).
__host__ __device__ __forceinline__ ChainItem chain_pm_item(uint32_t x, uint32_t y, uint32_t z,
                                                            const ChainArgs &a, int &row, int &ch) {
    const uint32_t B = a.B, K = a.K, D = a.D, nch = a.nchunk, X = 2 * nch + 1;
    if (z < K) {
        if (x == 2 * nch) return ChainItem{kItemPair, y, z};
        const uint32_t dr = x >= nch ? 1 : 0, c = x - dr * nch;
        row = static_cast<int>(dr ? K + 1 + z : z);
        ch = static_cast<int>(c);
        return ChainItem{kItemStats, y, (dr * K + z) * nch + c};
    }
    uint32_t h = ((z - K) * B + y) * X + x;
    if (h < B * nch) {
        const uint32_t b = fdiv(h, a.fd_nch);
        return ChainItem{kItemBonusStats, b, h - b * nch};
    }
    h -= B * nch;
    if (h < B * D) {
        const uint32_t b = fdiv(h, a.fd_D);
        return ChainItem{kItemDraw, b, h - b * D};
    }
    h -= B * D;
    if (h < B) return ChainItem{kItemFinisher, h, 0};
    if (h < 2 * B) return ChainItem{kItemBonus, h - B, 0};
    return ChainItem{kItemNone, 0, 0};
}

// Dimensions of the position-major grid (x, y, z).
struct Grid3 {
    uint32_t x, y, z;
};
inline Grid3 chain_pm_grid(const ChainArgs &a) {
    return Grid3{2 * static_cast<uint32_t>(a.nchunk) + 1, static_cast<uint32_t>(a.B),
                 static_cast<uint32_t>(a.K) + 2};
}

// Row and chunk of statistics item p of a sequence: rows 0..K-1 (target) and
// K+1..2K (draft), chunk-minor.
__host__ __device__ __forceinline__ void chain_stats_row(uint32_t p, const ChainArgs &a, int &row,
                                                         int &ch) {
    const uint32_t rr = fdiv(p, a.fd_nch), K = a.K;
    ch = static_cast<int>(p - rr * a.nchunk);
    row = static_cast<int>(rr < K ? rr : rr + 1);
}

// The draws of the two-phase form (k_chain_draw): B resolvers, B D draw
// items, B finishers, B bonus items.
__host__ __device__ __forceinline__ ChainItem chain_draw_item(uint32_t g, const ChainArgs &a) {
    const uint32_t B = a.B, nd = B * a.D;
    ChainItem it{kItemResolver, g, 0};
    if (g >= B && g < B + nd) {
        const uint32_t h = g - B, b = fdiv(h, a.fd_D);
        it = ChainItem{kItemDraw, b, h - b * a.D};
    } else if (g >= B + nd && g < 2 * B + nd) {
        it = ChainItem{kItemFinisher, g - B - nd, 0};
    } else if (g >= 2 * B + nd) {
        it = ChainItem{kItemBonus, g - 2 * B - nd, 0};
    }
    return it;
}

// ------------------------------------------------------------------ top-k

constexpr int kTopkGroupRows = 4;  // rows per merge workgroup (a wavefront each)

struct TopkItem {
    int64_t row, ch;  // a chunk item, when mgroup < 0
    int64_t mgroup;   // a merge item: rows mgroup * 4 .. mgroup * 4 + 3
};

// Grid order, in groups of four rows (G groups) and with L = lag groups: the
// chunks of groups 0..L-1; then for each group q >= L its chunks followed by
// one merge workgroup for group q - L; then the merges of the last L groups.
// A merge thus trails its rows' chunks by about L groups of workgroups.
// fd_nch divides by nch, fd_blk by 4 nch + 1; every numerator is an index of
// a grid of fewer than 2^31 workgroups.
__host__ __device__ __forceinline__ TopkItem topk_item(int64_t g, int64_t R, int64_t nch, int64_t L,
                                                       FastDiv fd_nch, FastDiv fd_blk) {
    const int64_t G = (R + kTopkGroupRows - 1) / kTopkGroupRows;
    auto group_chunks = [&](int64_t q) {
        const int64_t end = (q + 1) * kTopkGroupRows;
        return ((R < end ? R : end) - q * kTopkGroupRows) * nch;
    };
    // Chunk items before group q: 4 nch per full group.
    const int64_t full = kTopkGroupRows * nch, head = L < G ? L * full : R * nch;
    TopkItem it{-1, 0, -1};
    if (g < head) {
        it.row = fdiv(static_cast<uint32_t>(g), fd_nch);
        it.ch = g - it.row * nch;
    } else {
        const int64_t h = g - head, nbody = G - L;  // groups with chunks after the head
        // Body blocks: group L + b's chunks, then one merge (group b); the
        // last group may be partial.
        const int64_t blk = fdiv(static_cast<uint32_t>(h), fd_blk), off = h - blk * (full + 1);
        if (blk < nbody - 1 || (blk == nbody - 1 && off <= group_chunks(G - 1))) {
            const int64_t q = L + blk, nc = group_chunks(q);
            if (off < nc) {
                const int64_t r = fdiv(static_cast<uint32_t>(off), fd_nch);
                it.row = q * kTopkGroupRows + r;
                it.ch = off - r * nch;
            } else {
                it.mgroup = blk;
            }
        } else {
            const int64_t tail0 = (nbody - 1) * (full + 1) + group_chunks(G - 1) + 1;
            it.mgroup = nbody > 0 ? G - L + (h - tail0) : h;
        }
    }
    return it;
}

// Workgroups of the top-k launch: a chunk item per (row, chunk), a merge per
// group of four rows.
inline uint32_t topk_grid(int64_t rows, int64_t nch) {
    return static_cast<uint32_t>(rows * nch + (rows + kTopkGroupRows - 1) / kTopkGroupRows);
}

// ------------------------------------------------------------------ greedy chain and static tree

// One workgroup per (row, chunk) of the argmax, rows in order (then, for the
// per-sequence trees, one resolve per tree).
struct ArgmaxItem {
    bool argmax;
    uint32_t row;  // argmax: the row; resolve: the sequence
    uint32_t ch;
};
__host__ __device__ __forceinline__ ArgmaxItem argmax_item_of(uint32_t g, uint32_t nch, FastDiv fd_nch,
                                                              uint32_t rows) {
    const uint32_t nam = rows * nch;
    if (g < nam) {
        const uint32_t row = fdiv(g, fd_nch);
        return ArgmaxItem{true, row, g - row * nch};
    }
    return ArgmaxItem{false, g - nam, 0};
}
// Workgroups of the per-sequence-tree launch (argmax items, then a resolve
// per tree).
inline uint32_t argmax_grid(int64_t rows, int64_t nch, int64_t B) {
    return static_cast<uint32_t>(rows * nch + B);
}

// The greedy and static-tree launches have argmax items only: the item of
// the last chunk of a sequence's last row (per rows a sequence) also
// resolves the sequence.  Every other item of the sequence has a lower index,
// so its wait for their words only waits on workgroups handed out before it.
inline uint32_t argmax_only_grid(int64_t rows, int64_t nch) { return static_cast<uint32_t>(rows * nch); }
// The static tree's node-major grid: (chunks + 1) x trees x nodes; x = nchunk
// is the resolver of node z of tree y.
inline Grid3 tree_node_major_grid(int32_t nch, int32_t B, int32_t N) {
    return Grid3{static_cast<uint32_t>(nch) + 1, static_cast<uint32_t>(B), static_cast<uint32_t>(N)};
}
__host__ __device__ __forceinline__ bool argmax_resolves(uint32_t row, uint32_t ch, uint32_t nch,
                                                         uint32_t per, FastDiv fd_per, uint32_t &b) {
    b = fdiv(row, fd_per);
    return ch == nch - 1 && row == b * per + per - 1;
}

// ------------------------------------------------------------------ per-sequence trees

// Batches of at most kCompactTrees trees use the compact order: every
// workgroup reads all node counts, so the argmax items cover the real rows
// only, tree by tree, the resolve items follow them at once, and the
// workgroups left over (one per padding chunk) return at the end of the grid.
// Larger batches keep one item per (tree, row slot, chunk) and skip padding
// rows where they fall.
constexpr int kCountsPerLane = 4;
constexpr int kCompactTrees = 64 * kCountsPerLane;

// Real rows of a tree: its node count clamped to [1, Nmax].
__host__ __device__ __forceinline__ int tree_rows(int count, int Nmax) {
    const int c = count < 1 ? 1 : count;
    return c < Nmax ? c : Nmax;
}

// Lane `lane`'s share of the compact order's counts: trees lane P + j (0 past
// the batch).  The load address is clamped into the batch.
template <int P>
__host__ __device__ __forceinline__ void lane_tree_rows(const int32_t *node_count, int B, int Nmax,
                                                        int lane, int (&n)[P]) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
        const int t = lane * P + j;
        const int c = node_count[t < B ? t : B - 1];
        n[j] = tree_rows(c, Nmax) & -static_cast<int>(t < B);
    }
}

// Within lane L's trees (the first is t0), the tree b and node v at offset r
// of the lane's rows; nj(j) gives the lane's row count of its tree j.
template <int P, class NJ>
__host__ __device__ __forceinline__ void lane_row(uint32_t r, uint32_t t0, NJ nj, uint32_t &b,
                                                  uint32_t &v) {
    uint32_t t = t0;
#pragma unroll
    for (int j = 0; j < P - 1; ++j) {
        const uint32_t m = nj(j);
        if (r < m) break;
        r -= m;
        ++t;
    }
    b = t;
    v = r;
}

struct TreeDynItem {
    bool argmax, resolve;
    uint32_t row;  // argmax: row slot b Nmax + v; resolve: the tree
    uint32_t ch;
};

// The compact order, given R = g / nch, the batch's real rows T and, for
// R < T, the tree b and node v of real row R.
__host__ __device__ __forceinline__ TreeDynItem tree_dyn_compact_item(uint32_t g, uint32_t R,
                                                                      uint32_t nch, uint32_t T,
                                                                      uint32_t b, uint32_t v,
                                                                      uint32_t B, uint32_t Nmax) {
    const uint32_t nam = T * nch;
    TreeDynItem it;
    it.argmax = g < nam;
    it.resolve = !it.argmax && g < nam + B;
    it.row = it.argmax ? b * Nmax + v : g - nam;
    it.ch = g - R * nch;
    return it;
}

// The full order: item g < rows nch is (row slot, chunk), skipped when the
// slot is padding (count is the slot's tree's node count); then a resolve per
// tree.
__host__ __device__ __forceinline__ TreeDynItem tree_dyn_full_item(uint32_t g, uint32_t nch,
                                                                   FastDiv fd_nch, uint32_t rows,
                                                                   uint32_t Nmax, FastDiv fd_nmax,
                                                                   const int32_t *node_count) {
    TreeDynItem it{false, false, 0, 0};
    const uint32_t nam = rows * nch;
    if (g < nam) {
        const uint32_t slot = fdiv(g, fd_nch), b = fdiv(slot, fd_nmax), v = slot - b * Nmax;
        it.argmax = v < static_cast<uint32_t>(tree_rows(node_count[b], static_cast<int>(Nmax)));
        it.row = slot;
        it.ch = g - slot * nch;
    } else {
        it.resolve = true;
        it.row = g - nam;
    }
    return it;
}

}  // namespace sv
