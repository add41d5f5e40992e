// Top-k of draft rows on gfx950, one launch per call: the expansion step of
// an EAGLE-style tree drafter (French lesson, EAGLE section: trees of 4 to 8
// candidates per depth; its exercise has the draft propose its top branches
// at each depth).  The k entries of largest value, by value descending and
// then index ascending; values compare as floats, so -0.0 ties +0.0.
//
// One workgroup per (row, 16 KB chunk).  The threshold theta is the k-th
// largest of the chunk's sixteen 16-lane group maxima: k groups hold an
// entry >= theta, so the chunk's k best are all >= theta, and typically only
// a few entries are.  Those are compacted into LDS by ballot, and one
// wavefront ranks them, one per lane; if ties leave more than 64 candidates
// (or fewer than k entries exceed -inf), k exact selection rounds over all
// entries take over, each taking the best entry strictly after the last one
// taken.  Each chunk leaves its k best as tagged words.  A merge workgroup
// per four rows, placed in the grid well after their chunks, takes each
// row's k best from the row's lists on one wavefront.
#include "device.hpp"
#include "handover.hpp"
#include "grid_order.hpp"
#include "plan.hpp"
#include "topk.hpp"

namespace sv {

static_assert(kTopkGroupRows == kWaves, "a merge workgroup holds one wavefront per row");
namespace {

constexpr int kCandPerWave = 64;  // candidates compacted into LDS per wavefront of a chunk

// Ranking key of (v, i): larger means ranks first.  The high word maps the
// value to an unsigned integer of the same order (-0.0 taken as +0.0); the
// low word holds INT32_MAX - i above a bit that records a -0.0, which never
// decides an order (indices differ) but restores the value's bits.
__device__ __forceinline__ uint64_t tk_key(float v, int32_t i) {
    uint32_t u = __float_as_uint(v);
    const uint32_t negz = u == 0x80000000u;
    u = negz ? 0u : u;
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(u) << 32) |
           (static_cast<uint32_t>(INT32_MAX - i) << 1) | negz;
}
__device__ __forceinline__ int32_t tk_key_index(uint64_t key) {
    return INT32_MAX - static_cast<int32_t>(static_cast<uint32_t>(key) >> 1);
}
__device__ __forceinline__ float tk_key_value(uint64_t key) {
    if (key & 1u) return -0.0f;
    const uint32_t u = static_cast<uint32_t>(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Key of the filler (-inf, INT32_MAX): below every entry's key.
constexpr uint64_t kFillKey = static_cast<uint64_t>(0x007fffffu) << 32;

// Wavefront maximum of a key; the result in every lane.
__device__ __forceinline__ uint64_t tk_wave_max_key(uint64_t x) {
#define SV_TK_STEP(CTRL, MASK)                                                               \
    {                                                                                        \
        const uint32_t lo = dpp::mov_i<CTRL, MASK>(0, static_cast<int>(x));                  \
        const uint32_t hi = dpp::mov_i<CTRL, MASK>(0, static_cast<int>(x >> 32));            \
        const uint64_t y = (static_cast<uint64_t>(hi) << 32) | lo;                           \
        x = y > x ? y : x;                                                                   \
    }
    SV_TK_STEP(dpp::kRowShr1, 0xF)
    SV_TK_STEP(dpp::kRowShr2, 0xF)
    SV_TK_STEP(dpp::kRowShr4, 0xF)
    SV_TK_STEP(dpp::kRowShr8, 0xF)
    SV_TK_STEP(dpp::kRowBcast15, 0xA)
    SV_TK_STEP(dpp::kRowBcast31, 0xC)
#undef SV_TK_STEP
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(x), kWave - 1);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(x >> 32), kWave - 1);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Workgroup maximum of a key; the result in every thread.  Two barriers.
__device__ __forceinline__ uint64_t tk_wg_max_key(uint64_t x) {
    __shared__ uint64_t s_k[kWaves];
    x = tk_wave_max_key(x);
    if (threadIdx.x % kWave == 0) s_k[threadIdx.x / kWave] = x;
    __syncthreads();
    x = s_k[0];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) x = s_k[q] > x ? s_k[q] : x;
    __syncthreads();
    return x;
}

__device__ __forceinline__ uint64_t tk_readlane(uint64_t x, int src) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(x), src);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(x >> 32), src);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Keys of up to H chunk-list slots (value word, index word each): every word
// is read at once, then any that lacks the call's tag is read again (bounded
// wait) until it has it.  False if a wait ran out.
template <int H>
__device__ __forceinline__ bool tk_take_keys(const uint64_t *const (&p)[H], const bool (&in)[H],
                                             uint32_t tag, uint64_t t0, uint64_t (&key)[H]) {
    uint64_t wv[H], wi[H];
#pragma unroll
    for (int h = 0; h < H; ++h)
        if (in[h]) {
            wv[h] = fetch(p[h]);
            wi[h] = fetch(p[h] + 1);
        }
#pragma unroll
    for (int h = 0; h < H; ++h)
        if (in[h]) {
            while (!current(wv[h], tag) || !current(wi[h], tag)) {
                if (wall_clock64() - t0 > kWaitTicks) return false;
                __builtin_amdgcn_s_sleep(2);
                wv[h] = fetch(p[h]);
                wi[h] = fetch(p[h] + 1);
            }
            key[h] = tk_key(word_f32(wv[h]), static_cast<int32_t>(static_cast<uint32_t>(wi[h])));
        }
    return true;
}

// Row `row` when its lists hold at most 128 entries: slot j of the row (entry
// j % k of chunk j / k) sits in lane j % 64, register j / 64, all read in
// one round.  M is found from the chunk maxima as in topk_merge, and every
// entry at or above M (every entry, with fewer than k chunks) is ranked
// against the others.
__device__ void topk_merge_small(const TopkArgs &a, int64_t row) {
    const int lane = threadIdx.x % kWave, k = a.k, nch = a.nchunk, n = nch * k;
    const uint64_t *part = a.partial + 2 * row * nch * kMaxTopK;
    const uint64_t t0 = wall_clock64();
    uint64_t key[2] = {0, 0};
    const uint64_t *p[2];
    bool in[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int j = lane + h * kWave;
        in[h] = j < n;
        p[h] = part + 2 * ((j / k) * kMaxTopK + j % k);
    }
    const bool ok = tk_take_keys<2>(p, in, a.tag, t0, key);
    if (__ballot(!ok)) {
        if (lane < k) {
            a.out_idx[row * k + lane] = -1;
            if (a.out_val) a.out_val[row * k + lane] = NAN;
        }
        if (lane == 0) count_failure(a.hdr);
        return;
    }
    // M: the maximum (slot 0 of a list) that kt - 1 other maxima outrank.
    const int kt = min(k, nch);
    int rk[2] = {0, 0};
    for (int d = 0; d < nch; ++d) {
        const int j = d * k;
        const uint64_t kd = tk_readlane(j < kWave ? key[0] : key[1], j % kWave);
        rk[0] += kd > key[0];
        rk[1] += kd > key[1];
    }
    const uint64_t m0 = __ballot(lane < n && lane % k == 0 && rk[0] == kt - 1);
    const uint64_t m1 = __ballot(lane + kWave < n && (lane + kWave) % k == 0 && rk[1] == kt - 1);
    const uint64_t M = tk_readlane(m0 ? key[0] : key[1],
                                   __ffsll(static_cast<unsigned long long>(m0 ? m0 : m1)) - 1);
    bool keep[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) keep[h] = lane + h * kWave < n && (nch < k || key[h] >= M);
    int r[2] = {0, 0};
#pragma unroll
    for (int g = 0; g < 2; ++g)
        for (uint64_t b = __ballot(keep[g]); b; b &= b - 1) {
            const uint64_t kb = tk_readlane(key[g], __ffsll(static_cast<unsigned long long>(b)) - 1);
            r[0] += kb > key[0];
            r[1] += kb > key[1];
        }
#pragma unroll
    for (int h = 0; h < 2; ++h)
        if (keep[h] && r[h] < k) {
            a.out_idx[row * k + r[h]] = tk_key_index(key[h]);
            if (a.out_val) a.out_val[row * k + r[h]] = tk_key_value(key[h]);
        }
}

// Row `row`: the k best of its chunks' lists, on one wavefront.  Every entry
// of the row's top k lies in the list of one of the k chunks with the
// largest maxima (were its chunk's maximum ranked lower, k better entries
// would exist), and, when the row has at least k chunks, ranks at or above
// the k-th largest maximum M (the k best maxima are k entries at or above
// M).  So lane l takes entry l % k of the (l / k)-th best chunk, keeps it if
// it ranks at or above M, and counts the kept entries ahead of it; ranks
// below k are the row's list.  Every read waits (bounded) for the word to
// carry this call's tag; if a wait runs out the row gets -1 and NaN.
__device__ void topk_merge(const TopkArgs &a, int64_t row) {
    const int lane = threadIdx.x % kWave, k = a.k, nch = a.nchunk;
    const uint64_t *part = a.partial + 2 * row * nch * kMaxTopK;
    const uint64_t t0 = wall_clock64();
    bool ok = true;
    // Keys of the chunk maxima (slot 0 of each list): chunks lane and lane + 64.
    uint64_t mk[2] = {0, 0};
    {
        const uint64_t *p[2] = {part + 2 * lane * kMaxTopK, part + 2 * (lane + kWave) * kMaxTopK};
        const bool in[2] = {lane < nch, lane + kWave < nch};
        ok = tk_take_keys<2>(p, in, a.tag, t0, mk);
    }
    // Rank of each maximum among the maxima.
    int rk[2] = {0, 0};
    for (int d = 0; d < nch; ++d) {
        const uint64_t kd = tk_readlane(d < kWave ? mk[0] : mk[1], d % kWave);
        rk[0] += kd > mk[0];
        rk[1] += kd > mk[1];
    }
    // Lane l's chunk: the one whose maximum ranks l / k; M ranks kt - 1.
    const int kt = min(k, nch), m = k * kt;
    int mych = 0;
    uint64_t M = 0;
    for (int r = 0; r < kt; ++r) {
        const uint64_t b0 = __ballot(lane < nch && rk[0] == r);
        const uint64_t b1 = __ballot(lane + kWave < nch && rk[1] == r);
        const int src = __ffsll(static_cast<unsigned long long>(b0 ? b0 : b1)) - 1;
        if (lane / k == r) mych = b0 ? src : src + kWave;
        if (r == kt - 1) M = tk_readlane(b0 ? mk[0] : mk[1], src);
    }
    uint64_t key[1] = {0};
    {
        const uint64_t *p[1] = {part + 2 * (mych * kMaxTopK + lane % k)};
        const bool in[1] = {lane < m};
        ok = ok && tk_take_keys<1>(p, in, a.tag, t0, key);
    }
    const bool keep = ok && lane < m && (nch < k || key[0] >= M);
    if (__ballot(!ok)) {
        if (lane < k) {
            a.out_idx[row * k + lane] = -1;
            if (a.out_val) a.out_val[row * k + lane] = NAN;
        }
        if (lane == 0) count_failure(a.hdr);
        return;
    }
    int r = 0;
    for (uint64_t b = __ballot(keep); b; b &= b - 1)
        r += tk_readlane(key[0], __ffsll(static_cast<unsigned long long>(b)) - 1) > key[0];
    if (keep && r < k) {
        a.out_idx[row * k + r] = tk_key_index(key[0]);
        if (a.out_val) a.out_val[row * k + r] = tk_key_value(key[0]);
    }
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
    __shared__ int s_count[kWaves];
    __shared__ uint64_t s_c[kWaves][kCandPerWave];  // ranking keys
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave, k = a.k;
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
        for (int q = 0; q < NQ; ++q) raw[q] = load_nt(vp + min(tid + q * kWG, last));
        // Every load in flight before the first wait: one memory round trip.
        __builtin_amdgcn_sched_barrier(0);
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
    // Candidates (entries >= theta) go to the wavefront's LDS segment in
    // ballot order; the running count stays in a scalar register.
    int cnt = 0;
    if (theta > -INFINITY) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool hit = x[e] >= theta;
            const uint64_t b = __ballot(hit);
            if (b) {
                const int o = cnt + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                                              __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0));
                if (hit && o < kCandPerWave)
                    s_c[w][o] = tk_key(x[e], static_cast<int32_t>(e0 + pos(e)));
                cnt += __popcll(b);
            }
        }
    }
    if (lane == 0) s_count[w] = cnt;
    __syncthreads();
    int C = 0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) C += s_count[q];
    if (theta > -INFINITY && C <= kWave) {
        // Wavefront 0 takes candidate `lane` (segments in wave order) and
        // ranks it by the number of candidates ahead of it; ranks below k
        // are the chunk's list.  (There are at least k candidates: the k
        // groups whose maxima are >= theta each hold one.)
        if (w != 0) return;
        uint64_t key = 0;
        int base = 0;
#pragma unroll
        for (int q = 0; q < kWaves; ++q) {
            const int nq = s_count[q];
            if (lane >= base && lane < base + nq) key = s_c[q][lane - base];
            base += nq;
        }
        int r = 0;
        for (int j = 0; j < C; ++j) r += tk_readlane(key, j) > key;
        if (lane < C && r < k) tk_put(out, a.tag, r, tk_key_value(key), tk_key_index(key));
    } else {
        // Ties beyond 64 candidates, or fewer than k entries above -inf: k
        // exact rounds, each taking the best key below the last one taken.
        // They re-read the chunk (a rare path, so the registers holding it
        // are not kept alive for it).
        uint64_t last = ~0ull;
        for (int q = 0; q < k; ++q) {
            uint64_t best = kFillKey;
            for (int e = 0; e < E; ++e) {
                const int at = pos(e);
                if (at < n) {
                    const uint64_t key = tk_key(load_one<DT>(a.logits, row * a.V + e0 + at),
                                                static_cast<int32_t>(e0 + at));
                    if (key < last && key > best) best = key;
                }
            }
            best = tk_wg_max_key(best);
            if (tid == 0) tk_put(out, a.tag, q, tk_key_value(best), tk_key_index(best));
            last = best;
        }
    }
}

// The order of topk_item: a merge trails its rows' chunks by about `lag`
// groups of workgroups, by when they have usually finished, so merge
// workgroups rarely wait and the streaming runs on.
template <class DT, bool VecOk>
__global__ __launch_bounds__(kWG) void k_topk(TopkArgs a) {
    if (a.tag_src) a.tag = *a.tag_src;  // a graph replay's tag
    const int64_t R = a.rows;
    const TopkItem it = topk_item(blockIdx.x, R, a.nchunk, a.lag, a.fd_nch, a.fd_blk);
    const int64_t row = it.row, ch = it.ch, mgroup = it.mgroup;
    if (mgroup < 0) {
        topk_chunk<DT, VecOk>(a, row, static_cast<int>(ch));
        return;
    }
    const int64_t mrow = mgroup * kTopkGroupRows + threadIdx.x / kWave;
    if (mrow >= R) return;
    if (static_cast<int64_t>(a.nchunk) * a.k <= 2 * kWave) topk_merge_small(a, mrow);
    else topk_merge(a, mrow);
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, int dtype, hipStream_t s) {
    const dim3 g(topk_grid(a.rows, a.nchunk)), blk(kWG);
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
