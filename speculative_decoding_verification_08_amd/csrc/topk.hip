// Top-k of draft rows on gfx950, one launch per call: the expansion step of
// an EAGLE-style tree drafter (French lesson, EAGLE section: trees of 4 to 8
// candidates per depth; its exercise has the draft propose its top branches
// at each depth).  The k entries of largest value, by value descending and
// then index ascending; values compare as floats, so -0.0 ties +0.0.
//
// Chunk items: one workgroup per (row, 16 KB chunk).  The threshold theta is
// the k-th largest of the chunk's sixteen 16-lane group maxima: k groups hold
// an entry >= theta, so the chunk's k best are all >= theta, and typically
// only a few entries are.  Those are compacted into LDS and wavefront 0
// takes the k best; if ties leave more candidates than LDS holds, k exact
// rounds over all entries take over.  Each chunk leaves its k best as tagged
// words.
//
// Merge items: one workgroup per row, after every chunk workgroup; wavefront
// 0 waits (bounded) for the row's chunk lists and takes the k best of them.
//
// Every selection round takes the best entry strictly worse than the last
// one taken, under (value descending, index ascending), so no entry needs a
// taken flag.
#include "device.hpp"
#include "handover.hpp"
#include "plan.hpp"
#include "topk.hpp"

namespace sv {
namespace {

constexpr int kCandCap = 256;  // candidates compacted into LDS per chunk
constexpr int kTopkMergePerLane = kTopkMergeCands / kWave;

// (v, i) ranks before (bv, bi): larger value, then lower index.
__device__ __forceinline__ bool tk_better(float v, int32_t i, float bv, int32_t bi) {
    return v > bv || (v == bv && i < bi);
}
// (v, i) ranks after (lv, li), the last entry taken.
__device__ __forceinline__ bool tk_after(float v, int32_t i, float lv, int32_t li) {
    return tk_better(lv, li, v, i);
}

// Wavefront argmax of (v, i) under tk_better; the result in every lane.
__device__ __forceinline__ void tk_wave_best(float &v, int32_t &i) {
#define SV_TK_STEP(CTRL, MASK)                                                 \
    {                                                                          \
        const float v2 = dpp::mov_f<CTRL, MASK>(-INFINITY, v);                 \
        const int32_t i2 = dpp::mov_i<CTRL, MASK>(INT32_MAX, i);               \
        if (tk_better(v2, i2, v, i)) {                                         \
            v = v2;                                                            \
            i = i2;                                                            \
        }                                                                      \
    }
    SV_TK_STEP(dpp::kRowShr1, 0xF)
    SV_TK_STEP(dpp::kRowShr2, 0xF)
    SV_TK_STEP(dpp::kRowShr4, 0xF)
    SV_TK_STEP(dpp::kRowShr8, 0xF)
    SV_TK_STEP(dpp::kRowBcast15, 0xA)
    SV_TK_STEP(dpp::kRowBcast31, 0xC)
#undef SV_TK_STEP
    v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
    i = __builtin_amdgcn_readlane(i, kWave - 1);
}

// Workgroup argmax of (v, i); the result in every thread.  Two barriers.
__device__ __forceinline__ void tk_wg_best(float &v, int32_t &i) {
    __shared__ float s_v[kWaves];
    __shared__ int32_t s_i[kWaves];
    tk_wave_best(v, i);
    const int w = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) {
        s_v[w] = v;
        s_i[w] = i;
    }
    __syncthreads();
    v = s_v[0];
    i = s_i[0];
#pragma unroll
    for (int q = 1; q < kWaves; ++q)
        if (tk_better(s_v[q], s_i[q], v, i)) {
            v = s_v[q];
            i = s_i[q];
        }
    __syncthreads();
}

// Publishes slot q of a chunk's list.
__device__ __forceinline__ void tk_put(uint64_t *out, uint32_t tag, int q, float v, int32_t i) {
    publish(out + 2 * q, tag, __float_as_uint(v));
    publish(out + 2 * q + 1, tag, static_cast<uint32_t>(i));
}

// Chunk ch of row `row`: its k best as tagged words (slots past the chunk's
// entry count hold (-inf, INT32_MAX), which ranks after every entry).
template <class DT, bool VecOk>
__device__ __forceinline__ void topk_chunk(const TopkArgs &a, int64_t row, int ch) {
    constexpr int VEC = DT::kVec, NQ = kChunk2Bytes / 16 / kWG, E = NQ * VEC;  // entries per thread
    __shared__ float s_gmax[kWG / 16];
    __shared__ int s_count;
    __shared__ float s_cv[kCandCap];
    __shared__ int32_t s_ci[kCandCap];
    const int tid = threadIdx.x, lane = tid % kWave, k = a.k;
    const int64_t e0 = static_cast<int64_t>(ch) * a.chunk;
    const int n = static_cast<int>(min(static_cast<int64_t>(a.chunk), static_cast<int64_t>(a.V) - e0));
    uint64_t *out = a.partial + 2 * (row * a.nchunk + ch) * kMaxTopK;
    // Thread t holds vectors t, t + 256, ... of the chunk; entry e sits at pos(e).
    auto pos = [&](int e) { return (tid + (e / VEC) * kWG) * VEC + e % VEC; };
    float x[E];
    if constexpr (VecOk) {
        const uint4 *vp = static_cast<const uint4 *>(a.logits) + (row * a.V + e0) / VEC;
        uint4 raw[NQ];
        const int last = n / VEC - 1;
#pragma unroll
        for (int q = 0; q < NQ; ++q) raw[q] = vp[min(tid + q * kWG, last)];
#pragma unroll
        for (int q = 0; q < NQ; ++q) unpack<DT>(raw[q], x + q * VEC);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = load_one<DT>(a.logits, row * a.V + e0 + min(pos(e), n - 1));
    }
    if (n < a.chunk) {  // the row's last chunk: entries past its end never rank
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (pos(e) >= n) x[e] = -INFINITY;
    }
    // Maximum of each 16-thread group, then theta = the k-th largest of them.
    if (tid == 0) s_count = 0;
    float m = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) m = fmaxf(m, x[e]);
    m = fmaxf(m, dpp::mov_f<dpp::kRowShr1>(-INFINITY, m));
    m = fmaxf(m, dpp::mov_f<dpp::kRowShr2>(-INFINITY, m));
    m = fmaxf(m, dpp::mov_f<dpp::kRowShr4>(-INFINITY, m));
    m = fmaxf(m, dpp::mov_f<dpp::kRowShr8>(-INFINITY, m));
    if (lane % 16 == 15) s_gmax[tid / 16] = m;
    __syncthreads();
    float theta;
    {
        const float g = s_gmax[lane % 16];
        int ge = 0;
#pragma unroll
        for (int i = 0; i < kWG / 16; ++i) ge += s_gmax[i] >= g;
        float t = ge >= k ? g : -INFINITY;
        t = fmaxf(t, dpp::mov_f<dpp::kRowShr1>(-INFINITY, t));
        t = fmaxf(t, dpp::mov_f<dpp::kRowShr2>(-INFINITY, t));
        t = fmaxf(t, dpp::mov_f<dpp::kRowShr4>(-INFINITY, t));
        t = fmaxf(t, dpp::mov_f<dpp::kRowShr8>(-INFINITY, t));
        theta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 15));
    }
    // Candidates (entries >= theta) go to LDS, a wavefront's worth at a time.
    if (theta > -INFINITY) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool hit = x[e] >= theta;
            const uint64_t b = __ballot(hit);
            if (b) {
                const int first = __ffsll(static_cast<unsigned long long>(b)) - 1;
                int base = 0;
                if (lane == first) base = atomicAdd(&s_count, __popcll(b));
                base = __builtin_amdgcn_readlane(base, first);
                const int o = base + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0));
                if (hit && o < kCandCap) {
                    s_cv[o] = x[e];
                    s_ci[o] = static_cast<int32_t>(e0 + pos(e));
                }
            }
        }
    }
    __syncthreads();
    const int C = s_count;
    if (theta > -INFINITY && C <= kCandCap) {
        // Candidate t's rank is the number of candidates ahead of it; ranks
        // below k are the chunk's list.  Slots past C get the filler.
        if (tid >= max(C, k)) return;
        if (tid < C) {
            const float v = s_cv[tid];
            const int32_t i = s_ci[tid];
            int r = 0;
            for (int j = 0; j < C; ++j) r += tk_better(s_cv[j], s_ci[j], v, i);
            if (r < k) tk_put(out, a.tag, r, v, i);
        } else {
            tk_put(out, a.tag, tid, -INFINITY, INT32_MAX);
        }
        return;
    }
    // Ties beyond LDS, or fewer than k entries above -inf: k exact rounds.
    float lv = INFINITY;
    int32_t li = -1;
    for (int q = 0; q < k; ++q) {
        float bv = -INFINITY;
        int32_t bi = INT32_MAX;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int32_t i = static_cast<int32_t>(e0 + pos(e));
            if (pos(e) < n && tk_after(x[e], i, lv, li) && tk_better(x[e], i, bv, bi)) {
                bv = x[e];
                bi = i;
            }
        }
        tk_wg_best(bv, bi);
        if (tid == 0) tk_put(out, a.tag, q, bv, bi);
        lv = bv;
        li = bi;
    }
}

// Row `row`: the k best of its chunks' lists (nchunk * k <= 64 * 16 entries,
// kept in wavefront 0's registers).
__device__ __forceinline__ void topk_merge(const TopkArgs &a, int64_t row) {
    if (threadIdx.x >= kWave) return;
    const int lane = threadIdx.x, k = a.k, n = a.nchunk * k;
    const uint64_t *part = a.partial + 2 * row * a.nchunk * kMaxTopK;
    auto word = [&](int j) { return part + 2 * ((j / k) * kMaxTopK + j % k); };  // candidate j
    const uint64_t t0 = wall_clock64();
    float cv[kTopkMergePerLane];
    int32_t ci[kTopkMergePerLane];
    bool ok = true;
    for (;;) {
        bool fresh = true;
        const uint64_t *miss = nullptr;
#pragma unroll
        for (int s = 0; s < kTopkMergePerLane; ++s) {
            const int j = min(lane + s * kWave, n - 1);
            const uint64_t wv = fetch(word(j)), wi = fetch(word(j) + 1);
            const bool in = lane + s * kWave < n, cur = current(wv, a.tag) && current(wi, a.tag);
            if (in && !cur && !miss) miss = current(wv, a.tag) ? word(j) + 1 : word(j);
            fresh = fresh && (!in || cur);
            cv[s] = in ? word_f32(wv) : -INFINITY;
            ci[s] = in ? static_cast<int32_t>(static_cast<uint32_t>(wi)) : INT32_MAX;
        }
        const uint64_t stale = __ballot(!fresh);
        if (!stale) break;
        if (wall_clock64() - t0 > kWaitTicks) {
            ok = false;
            break;
        }
        if (lane == __ffsll(static_cast<unsigned long long>(stale)) - 1) wait_word(miss, a.tag, t0);
    }
    float lv = INFINITY;
    int32_t li = -1;
    for (int q = 0; q < k; ++q) {
        float bv = -INFINITY;
        int32_t bi = INT32_MAX;
#pragma unroll
        for (int s = 0; s < kTopkMergePerLane; ++s)
            if (tk_after(cv[s], ci[s], lv, li) && tk_better(cv[s], ci[s], bv, bi)) {
                bv = cv[s];
                bi = ci[s];
            }
        tk_wave_best(bv, bi);
        if (lane == 0) {
            a.out_idx[row * k + q] = ok ? bi : -1;
            if (a.out_val) a.out_val[row * k + q] = ok ? bv : NAN;
        }
        lv = bv;
        li = bi;
    }
}

template <class DT, bool VecOk>
__global__ __launch_bounds__(kWG) void k_topk(TopkArgs a) {
    const uint32_t nc = static_cast<uint32_t>(a.rows) * a.nchunk, g = blockIdx.x;
    if (g < nc) {
        const uint32_t row = g / a.nchunk;
        topk_chunk<DT, VecOk>(a, row, static_cast<int>(g - row * a.nchunk));
    } else {
        topk_merge(a, g - nc);
    }
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, int dtype, hipStream_t s) {
    const dim3 g(static_cast<uint32_t>(a.rows * a.nchunk + a.rows)), blk(kWG);
    if (dtype == 1) {
        if (a.V % Bf16::kVec == 0) k_topk<Bf16, true><<<g, blk, 0, s>>>(a);
        else k_topk<Bf16, false><<<g, blk, 0, s>>>(a);
    } else {
        if (a.V % F32::kVec == 0) k_topk<F32, true><<<g, blk, 0, s>>>(a);
        else k_topk<F32, false><<<g, blk, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace sv
