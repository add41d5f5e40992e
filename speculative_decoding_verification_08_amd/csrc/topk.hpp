// Launch arguments of the per-row top-k (topk.hip), shared with the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// Top-k of rows [rows][V] in one launch: one workgroup per (row, 16 KB chunk)
// leaves its chunk's k best (value, index), then one merge workgroup per row.
constexpr int kMaxTopK = 8;
constexpr int kTopkMergeCands = 1024;  // nchunk * k at most: 16 per lane of one wavefront
struct TopkArgs {
    const void *logits;
    int64_t rows;
    int32_t V, chunk, nchunk, k;
    uint32_t tag;
    uint64_t *partial;       // [rows][nchunk][kMaxTopK][2] tagged (value bits, index)
    int32_t *out_idx;        // [rows][k]
    float *out_val;          // nullable [rows][k]
};

hipError_t launch_topk(const TopkArgs &a, int dtype, hipStream_t s);

}  // namespace sv
