// KV commit after verify on gfx950: the accepted entries' keys and values go
// from the scratch buffer the verifier's forward wrote to the cache (Arabic
// lesson, section on rolling the KV cache back, and its key-terms entry: write
// the drafted positions to scratch first, commit the accepted ones, discard
// the rest).  A byte copy bound by HBM bandwidth: no arithmetic, no LDS
// traffic beyond the path.
//
// One workgroup per (plane, sequence).  It checks the sequence's count,
// length and path (a sequence with any of them out of range is left whole),
// stages the path in LDS, and copies count rows of 16-byte vectors: the
// destination window is contiguous, so flat vector f of the window goes to
// f, from row path[f / vpr] of the scratch.  Each thread keeps kUnroll loads
// in flight before its stores.
#include "device.hpp"
#include "kv.hpp"

namespace sv {
namespace {

constexpr int kPathLds = 1024;  // path entries staged in LDS; later ones are read from memory
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kWG) void k_kv_commit(KvArgs a) {
    __shared__ int32_t s_path[kPathLds];
    const int tid = threadIdx.x;
    const int b = static_cast<int>(blockIdx.x % static_cast<uint32_t>(a.B));
    const int plane = static_cast<int>(blockIdx.x / static_cast<uint32_t>(a.B));
    const int c = a.count[b], L = a.len[b];
    bool bad = !(c >= 0 && c <= a.P && L >= 0 && static_cast<int64_t>(L) + c <= a.S);
    const int32_t *pb = a.path ? a.path + static_cast<int64_t>(b) * a.P : nullptr;
    if (!bad)
        for (int i = tid; i < c; i += kWG) {
            const int r = pb ? pb[i] : i;
            bad = bad || r < 0 || r >= a.N;
            if (i < kPathLds) s_path[i] = r;
        }
    bad = __syncthreads_or(bad);
    if (plane == 0 && tid == 0) a.new_len[b] = bad ? L : L + c;
    if (bad) return;
    const int64_t pb_rows = static_cast<int64_t>(plane) * a.B + b;
    const uint4 *src = a.scratch + pb_rows * a.N * a.vpr;
    uint4 *dst = a.cache + (pb_rows * a.S + L) * a.vpr;
    const uint32_t vpr = static_cast<uint32_t>(a.vpr), total = static_cast<uint32_t>(c) * vpr;
    for (uint32_t f0 = 0; f0 < total; f0 += kWG * kUnroll) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t f = f0 + u * kWG + tid;
            if (f < total) {
                const uint32_t i = f / vpr, off = f - i * vpr;
                const int r = i < static_cast<uint32_t>(kPathLds) ? s_path[i] : (pb ? pb[i] : static_cast<int>(i));
                v[u] = src[static_cast<int64_t>(r) * vpr + off];
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t f = f0 + u * kWG + tid;
            if (f < total) dst[f] = v[u];
        }
    }
}

}  // namespace

hipError_t launch_kv_commit(const KvArgs &a, hipStream_t s) {
    const dim3 g(static_cast<uint32_t>(static_cast<int64_t>(a.planes) * a.B)), blk(kWG);
    k_kv_commit<<<g, blk, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sv
