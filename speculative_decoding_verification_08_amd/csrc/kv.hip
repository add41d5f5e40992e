// KV commit after verify on gfx950: the accepted entries' keys and values go
// from the scratch buffer the verifier's forward wrote to the cache (Arabic
// lesson, section on rolling the KV cache back, and its key-terms entry: write
// the drafted positions to scratch first, commit the accepted ones, discard
// the rest).  A byte copy bound by HBM bandwidth: no arithmetic, no LDS
// traffic beyond the path.
//
// A sequence with a count, length or path out of range is left whole.  The
// destination window of a plane is contiguous, so vector f of it comes from
// row path[f / vpr] of the scratch; no LDS is needed.
#include "device.hpp"
#include "kv.hpp"

namespace sv {
namespace {

constexpr int kUnroll = 4;  // 16-byte vectors per thread per round

// Workgroup per (sequence, plane), sequence-major: the workgroups of one
// sequence run side by side and share its count, length and path in L2.
// Round one requests the count, the length and, for each of the thread's
// vectors, the path entry of its row, all at once.  Each thread then checks
// what it read and issues its row loads (only rows in range, so every load
// is in bounds), and the workgroup's vote on the whole sequence runs while
// those loads are in flight; stores follow only if every entry passed.
// Windows longer than one round (more than kWG * kUnroll vectors) check
// their remaining path entries before the vote and copy the rest after it.
__global__ __launch_bounds__(kWG) void k_kv_commit(KvArgs a) {
    const int tid = threadIdx.x;
    const int b = static_cast<int>(fdiv(blockIdx.x, a.fd_planes));
    const int plane = static_cast<int>(blockIdx.x - static_cast<uint32_t>(b) * a.planes);
    const int32_t *pb = a.path ? a.path + static_cast<int64_t>(b) * a.P : nullptr;
    const uint32_t vpr = static_cast<uint32_t>(a.vpr);
    uint32_t fu[kUnroll], iu[kUnroll];
    int ru[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        fu[u] = static_cast<uint32_t>(u * kWG + tid);
        const uint32_t i = fdiv(fu[u], a.fd_vpr);
        iu[u] = i;
        ru[u] = static_cast<int>(i);
        if (pb && i < static_cast<uint32_t>(a.P)) ru[u] = pb[i];
    }
    const int c = a.count[b], L = a.len[b];
    // Non-short-circuit, so both loads issue together.
    const bool shape_ok = (c >= 0) & (c <= a.P) & (L >= 0) & (static_cast<int64_t>(L) + c <= a.S);
    const uint32_t total = shape_ok ? static_cast<uint32_t>(c) * vpr : 0u;
    bool bad = !shape_ok;
    const int64_t pl = static_cast<int64_t>(plane) * a.B + b;
    const uint4 *src = a.scratch + pl * a.N * vpr;
    uint4 *dst = a.cache + (pl * a.S + L) * vpr;
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int r = ru[u];
        const bool live = fu[u] < total, in = r >= 0 && r < a.N;
        bad = bad || (live && !in);
        v[u] = make_uint4(0u, 0u, 0u, 0u);
        if (live && in) v[u] = load_nt(src + static_cast<int64_t>(r) * vpr + (fu[u] - iu[u] * vpr));
    }
    // Rows past the first round: check their path entries too.
    constexpr uint32_t kRound = kWG * kUnroll;
    for (uint32_t i = fdiv(kRound, a.fd_vpr) + tid; pb && static_cast<uint64_t>(i) * vpr < total; i += kWG) {
        const int r = pb[i];
        if (r < 0 || r >= a.N) bad = true;
    }
    bad = __syncthreads_or(bad);
    if (plane == 0 && tid == 0) a.new_len[b] = bad ? L : L + c;
    if (bad) return;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
        if (fu[u] < total) dst[fu[u]] = v[u];
    for (uint32_t f0 = kRound; f0 < total; f0 += kRound) {
        uint4 w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t f = f0 + u * kWG + tid;
            w[u] = make_uint4(0u, 0u, 0u, 0u);
            if (f < total) {
                const uint32_t i = fdiv(f, a.fd_vpr);
                const int r = pb ? pb[i] : static_cast<int>(i);
                w[u] = load_nt(src + static_cast<int64_t>(r) * vpr + (f - i * vpr));
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t f = f0 + u * kWG + tid;
            if (f < total) dst[f] = w[u];
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
