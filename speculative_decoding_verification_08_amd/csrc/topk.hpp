// Launch arguments of the per-row top-k (topk.hip), shared with the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace sv {

// Top-k of rows [rows][V] in one launch: one workgroup per (row, 16 KB chunk)
// leaves its chunk's k best (value, index); a merge workgroup per group of
// four rows, `lag` groups later in the grid, takes each row's k best from
// them (a wavefront per row).
constexpr int kMaxTopK = 8;
constexpr int kTopkMaxChunks = 128;  // chunks per row: two per lane of one wavefront
struct TopkArgs {
    const void *logits;
    int64_t rows;
    int32_t V, chunk, nchunk, k;
    int64_t lag;             // groups of four rows between a group's chunks and its merge, 1 <= lag <= groups
    FastDiv fd_nch, fd_blk;  // division by nchunk and by 4 nchunk + 1 (a body block of the grid)
    uint32_t tag;
    const uint32_t *tag_src; // nullable: read the tag from this device word instead (graph replays)
    uint64_t *partial;       // [rows][nchunk][kMaxTopK][2] tagged (value bits, index)
    int32_t *out_idx;        // [rows][k]
    float *out_val;          // nullable [rows][k]
    uint32_t *hdr;           // the workspace header words
};

hipError_t launch_topk(const TopkArgs &a, int dtype, hipStream_t s);

}  // namespace sv
