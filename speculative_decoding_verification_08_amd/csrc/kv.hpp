// Launch arguments of the KV commit (kv.hip), shared with the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace sv {

struct KvArgs {
    const uint4 *scratch;    // [planes][B][N][vpr] 16-byte vectors
    uint4 *cache;            // [planes][B][S][vpr]
    int32_t planes, B, N, S, P;
    int32_t vpr;             // 16-byte vectors per row
    FastDiv fd_planes, fd_vpr;  // division by planes and by vpr
    const int32_t *path;     // nullable [B][P]
    const int32_t *count;    // [B]
    const int32_t *len;      // [B]
    int32_t *new_len;        // [B]
};

hipError_t launch_kv_commit(const KvArgs &a, hipStream_t s);

}  // namespace sv
