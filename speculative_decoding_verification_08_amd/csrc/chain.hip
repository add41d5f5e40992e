// Chain verify at T > 0 on gfx950.
//
// Three kinds of work, written once as workgroup-level item functions:
//
//  stats item  (sequence b, row r, vocabulary chunk): streams one 16 KB chunk
//      of a target row (rows 0..K) or draft row (0..K-1) once, folds it into
//      softmax statistics (ref, z) and publishes them; the chunk holding the
//      row's drafted token also publishes that logit.  These items carry all
//      the logit bytes: the HBM-bound part.
//  resolve item (sequence b): merges the sequence's row statistics,
//      evaluates the accept test of every drafted token (u < p(x)/q(x),
//      French lesson "La règle de l'exactitude"; forum post §3), finds the
//      first rejection j and publishes j with row j's statistics.
//  mass item   (sequence b, 16 KB chunk of row j): publishes the draw mass of
//      its chunk: max(0, p_j - q_j) after a rejection (the residual of the
//      same passages) or p_K when every draft was accepted (the bonus draw).
//  finish item (sequence b): finds the chunk whose running mass first exceeds
//      u * S, scans that chunk in index order and writes the emitted tokens.
//
// spec_verify_chain runs them as one fused kernel: workgroup t executes the
// t-th item of an order in which every item depends only on items with lower
// indices (fused_item), so a sequence's resolve, mass and finish work overlap
// the streaming of later sequences.  Items hand over 64-bit words holding the call's tag
// and a value, written and read with device-scope relaxed atomics (coherent
// across the XCDs' L2 caches without fences); a reader waits, for a bounded
// time, until every word it needs carries the current tag.  The phase entry
// points run the same items as four ordinary kernels, where the kernel
// boundary has already made every word current.  Device-scope fences, an L2
// write-back and invalidate per workgroup on this chip, are not used.
#include "device.hpp"
#include "plan.hpp"

namespace sv {
namespace {

// ------------------------------------------------------------ hand-over

__device__ __forceinline__ void publish(uint64_t *p, uint32_t tag, uint32_t bits) {
    __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | bits, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_f32(uint64_t *p, uint32_t tag, float v) {
    publish(p, tag, __float_as_uint(v));
}
__device__ __forceinline__ uint64_t fetch(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool current(uint64_t w, uint32_t tag) {
    return static_cast<uint32_t>(w >> 32) == tag;
}
__device__ __forceinline__ float word_f32(uint64_t w) {
    return __uint_as_float(static_cast<uint32_t>(w));
}
__device__ __forceinline__ uint32_t word_u32(uint64_t w) { return static_cast<uint32_t>(w); }

// Bounded wait of a workgroup: `stale` is this thread's count of words still
// carrying an old tag.  Returns 1 when no thread has one, 0 to poll again,
// -1 once 0.2 s of the 100 MHz wall clock have passed (or at once when the
// workgroup may not wait).
constexpr uint64_t kWaitLimitTicks = 20000000ull;
__device__ __forceinline__ int poll_done(int stale, bool may_wait, uint64_t t0) {
    if (!__syncthreads_or(stale)) return 1;
    const int expired =
        threadIdx.x == 0 && (!may_wait || wall_clock64() - t0 > kWaitLimitTicks);
    if (__syncthreads_or(expired)) return -1;
    __builtin_amdgcn_s_sleep(2);
    return 0;
}

// ------------------------------------------------------------ stats item

template <class DT, int U>
__device__ __forceinline__ void stats_item(const ChainArgs &a, int64_t row, int ch) {
    constexpr int VEC = DT::kVec;
    const int K = a.K, V = a.V, R = 2 * K + 1;
    const int64_t b = row / R;
    const int r = static_cast<int>(row % R);
    const void *base;
    int64_t trow;
    int k;  // drafted position this row scores, -1 for the bonus row
    if (r <= K) {
        base = a.target;
        trow = b * (K + 1) + r;
        k = r < K ? r : -1;
    } else {
        base = a.draft;
        trow = b * K + (r - K - 1);
        k = r - K - 1;
    }
    const int64_t e0 = static_cast<int64_t>(ch) * a.chunk;
    const int64_t e1 = min(e0 + a.chunk, static_cast<int64_t>(V));
    const Span s = split_span<VEC>(trow * V + e0, trow * V + e1);

    float ref = -INFINITY, z = 0.f;
    {
        const int64_t h = s.h0 + threadIdx.x;
        if (h < s.h1) {
            const float x = load_one<DT>(base, h);
            mz_batch<1>(&x, a.c, ref, z);
        }
    }
    const uint4 *vp = static_cast<const uint4 *>(base);
    int64_t v = s.va + threadIdx.x;
    for (; v + (U - 1) * kWG < s.vb; v += U * kWG) {
        uint4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = vp[v + u * kWG];
        float x[U * VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) unpack<DT>(raw[u], x + u * VEC);
        mz_batch<U * VEC>(x, a.c, ref, z);
    }
    for (; v < s.vb; v += kWG) {
        float x[VEC];
        unpack<DT>(vp[v], x);
        mz_batch<VEC>(x, a.c, ref, z);
    }
    {
        const int64_t t = s.t0 + threadIdx.x;
        if (t < s.t1) {
            const float x = load_one<DT>(base, t);
            mz_batch<1>(&x, a.c, ref, z);
        }
    }
    if (threadIdx.x == 0 && k >= 0) {
        const int x = min(max(a.tokens[b * K + k], 0), V - 1);
        if (x >= e0 && x < e1)
            publish_f32(&a.gathered[row], a.tag, load_one<DT>(base, trow * V + x));
    }
    mz_reduce_wg(ref, z);
    if (threadIdx.x == 0) {
        uint64_t *w = a.partial + 2 * (row * a.nchunk + ch);
        publish_f32(w, a.tag, ref);
        publish_f32(w + 1, a.tag, z);
    }
}

// ------------------------------------------------------------ draw weights

// Entries per chunk of the residual / bonus pass: 16 KB of one row.
template <class DT>
struct Chunk2 {
    static constexpr int kElems = kChunk2Bytes / (16 / DT::kVec);
};

// Draw weight of one vocabulary entry of row j.
__device__ __forceinline__ float draw_weight(float t, float d, float c, float rt, float izt,
                                             float rd, float izd, bool resid) {
    const float p = __fmul_rn(exp2_hw(fmaf(t, c, -rt)), izt);
    if (!resid) return p;
    const float q = __fmul_rn(exp2_hw(fmaf(d, c, -rd)), izd);
    return fmaxf(p - q, 0.f);
}

// Row j's draw weights: statistics of its target (and draft) row.
struct DrawRow {
    int64_t trow, drow;  // element offsets of target row j and draft row j
    float rt, izt, rd, izd;
    bool resid;
};

// Per-lane sum of the draw weights of chunk [e0, e1) of row j.  With V a
// multiple of the vector width every lane issues all its 16-byte loads (4
// per row) before using any.
template <class DT>
__device__ __forceinline__ float lane_mass(const ChainArgs &a, const DrawRow &w, int64_t e0,
                                           int64_t e1) {
    constexpr int VEC = DT::kVec;
    constexpr int NV = Chunk2<DT>::kElems / (VEC * kWG);
    float acc = 0.f;
    if (a.V % VEC == 0) {
        const uint4 *tp = static_cast<const uint4 *>(a.target);
        const uint4 *dp = static_cast<const uint4 *>(a.draft);
        const int64_t v0 = (w.trow + e0) / VEC, nv = (e1 - e0) / VEC;
        const int64_t d0 = (w.drow + e0) / VEC;
        uint4 rt[NV], rd[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int64_t o = threadIdx.x + i * kWG;
            if (o < nv) {
                rt[i] = tp[v0 + o];
                if (w.resid) rd[i] = dp[d0 + o];
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int64_t o = threadIdx.x + i * kWG;
            if (o < nv) {
                float t[VEC], d[VEC];
                unpack<DT>(rt[i], t);
                if (w.resid) unpack<DT>(rd[i], d);
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    acc += draw_weight(t[q], w.resid ? d[q] : 0.f, a.c, w.rt, w.izt, w.rd, w.izd,
                                       w.resid);
            }
        }
    } else {
        for (int64_t e = e0 + threadIdx.x; e < e1; e += kWG) {
            const float t = load_one<DT>(a.target, w.trow + e);
            const float d = w.resid ? load_one<DT>(a.draft, w.drow + e) : 0.f;
            acc += draw_weight(t, d, a.c, w.rt, w.izt, w.rd, w.izd, w.resid);
        }
    }
    return acc;
}

// Waits for sequence b's row statistics and drafted-token logits, merges the
// statistics over chunks (in chunk order) and evaluates the accept test of
// every drafted token.  Returns j, the first rejected position (K if none),
// with row j's statistics in `w` and p_k(x_k), q_k(x_k) in s_P, s_Q; sets
// `ok` to false if the wait ran out.
template <class DT>
__device__ int accept_prefix(const ChainArgs &a, int b, bool may_wait, float *s_P, float *s_Q,
                             DrawRow &w, bool &ok) {
    __shared__ float s_ref[2 * kMaxK + 1], s_z[2 * kMaxK + 1];
    __shared__ float s_pr[kMergeLds], s_pz[kMergeLds];
    __shared__ int s_j;
    const int K = a.K, V = a.V, R = 2 * K + 1, tid = threadIdx.x;
    const int np = R * a.nchunk;
    const uint64_t *part = a.partial + 2 * static_cast<int64_t>(b) * np;
    const uint64_t *gat = a.gathered + static_cast<int64_t>(b) * R;
    const bool staged = np <= kMergeLds;
    float lt = 0.f, ld = 0.f;
    const float u = tid < K ? a.u_accept[b * K + tid] : 0.f;
    const uint64_t t0 = wall_clock64();
    ok = true;
    for (;;) {
        int stale = 0;
        for (int i = tid; i < np; i += kWG) {
            const uint64_t wr = fetch(part + 2 * i), wz = fetch(part + 2 * i + 1);
            if (!current(wr, a.tag) || !current(wz, a.tag)) {
                stale = 1;
            } else if (staged) {
                s_pr[i] = word_f32(wr);
                s_pz[i] = word_f32(wz);
            }
        }
        if (tid < K) {
            const uint64_t wt = fetch(gat + tid), wd = fetch(gat + K + 1 + tid);
            if (!current(wt, a.tag) || !current(wd, a.tag)) stale = 1;
            lt = word_f32(wt);
            ld = word_f32(wd);
        }
        const int st = poll_done(stale, may_wait, t0);
        if (st == 1) break;
        if (st < 0) {
            ok = false;
            break;
        }
    }
    for (int r = tid; r < R; r += kWG) {
        float ref = -INFINITY, z = 0.f;
        for (int i = 0; i < a.nchunk; ++i) {
            const int q = r * a.nchunk + i;
            const float pr = staged ? s_pr[q] : word_f32(fetch(part + 2 * q));
            const float pz = staged ? s_pz[q] : word_f32(fetch(part + 2 * q + 1));
            mz_merge(ref, z, pr, pz);
        }
        s_ref[r] = ref;
        s_z[r] = z;
    }
    __syncthreads();
    // Accept test u < P/Q (strict; Q = 0 accepts iff P > 0), wave 0, K <= 64.
    if (tid < kWave) {
        bool reject = false;
        if (tid < K) {
            const float P = exp2_hw(fmaf(lt, a.c, -s_ref[tid])) / s_z[tid];
            const float Q = exp2_hw(fmaf(ld, a.c, -s_ref[K + 1 + tid])) / s_z[K + 1 + tid];
            reject = !(Q > 0.f ? (u < P / Q) : (P > 0.f));
            s_P[tid] = P;
            s_Q[tid] = Q;
        }
        const uint64_t m = __ballot(reject);
        if (tid == 0) s_j = m ? (__ffsll(static_cast<unsigned long long>(m)) - 1) : K;
    }
    __syncthreads();
    const int j = s_j;
    w.resid = j < K;
    w.rt = s_ref[j];
    w.izt = 1.f / s_z[j];
    w.rd = w.resid ? s_ref[K + 1 + j] : 0.f;
    w.izd = w.resid ? 1.f / s_z[K + 1 + j] : 0.f;
    w.trow = (static_cast<int64_t>(b) * (K + 1) + j) * V;
    w.drow = w.resid ? (static_cast<int64_t>(b) * K + j) * V : 0;
    return j;
}

// Row j's record as the resolve item published it: waits (bounded) until the
// five words are current; returns false on a timeout.
__device__ __forceinline__ bool wait_record(const ChainArgs &a, int b, bool may_wait,
                                            uint64_t *s_info) {
    SeqInfo &si = a.seq[b];
    const uint64_t t0 = wall_clock64();
    for (;;) {
        int stale = 0;
        if (threadIdx.x < 5) {
            const uint64_t *f = threadIdx.x == 0   ? &si.j
                                : threadIdx.x == 1 ? &si.rt
                                : threadIdx.x == 2 ? &si.izt
                                : threadIdx.x == 3 ? &si.rd
                                                   : &si.izd;
            const uint64_t v = fetch(f);
            if (!current(v, a.tag)) stale = 1;
            s_info[threadIdx.x] = v;
        }
        const int st = poll_done(stale, may_wait, t0);
        if (st != 0) return st == 1;
    }
}

__device__ __forceinline__ DrawRow draw_row(const ChainArgs &a, int b, const uint64_t *info,
                                            int &j) {
    const uint32_t jw = word_u32(info[0]);
    j = jw > static_cast<uint32_t>(a.K) ? a.K : static_cast<int>(jw);
    DrawRow w;
    w.resid = j < a.K;
    w.rt = word_f32(info[1]);
    w.izt = word_f32(info[2]);
    w.rd = word_f32(info[3]);
    w.izd = word_f32(info[4]);
    w.trow = (static_cast<int64_t>(b) * (a.K + 1) + j) * a.V;
    w.drow = w.resid ? (static_cast<int64_t>(b) * a.K + j) * a.V : 0;
    return w;
}

// Marks sequence b as timed out; the flag lands before the caller's next word.
__device__ __forceinline__ void flag_timeout(const ChainArgs &a, int b) {
    publish(&a.seq[b].timeout, a.tag, 1u);
    __builtin_amdgcn_s_waitcnt(0);
}

template <class DT>
__device__ __forceinline__ void resolve_item(const ChainArgs &a, int b, bool may_wait) {
    __shared__ float s_P[kMaxK], s_Q[kMaxK];
    const int K = a.K;
    DrawRow w;
    bool ok;
    const int j = accept_prefix<DT>(a, b, may_wait, s_P, s_Q, w, ok);
    SeqInfo &si = a.seq[b];
    for (int k = threadIdx.x; k < K; k += kWG) {
        publish_f32(&si.P[k], a.tag, s_P[k]);
        publish_f32(&si.Q[k], a.tag, s_Q[k]);
    }
    if (threadIdx.x == 0) {
        if (!ok) flag_timeout(a, b);
        publish(&si.j, a.tag, static_cast<uint32_t>(j));
        publish_f32(&si.rt, a.tag, w.rt);
        publish_f32(&si.izt, a.tag, w.izt);
        publish_f32(&si.rd, a.tag, w.rd);
        publish_f32(&si.izd, a.tag, w.izd);
    }
}

template <class DT>
__device__ __forceinline__ void mass_item(const ChainArgs &a, int b, int ch, bool may_wait) {
    __shared__ uint64_t s_info[5];
    constexpr int C2 = Chunk2<DT>::kElems;
    const bool ok = wait_record(a, b, may_wait, s_info);
    int j;
    const DrawRow w = draw_row(a, b, s_info, j);
    const int64_t e0 = static_cast<int64_t>(ch) * C2;
    const int64_t e1 = min(static_cast<int64_t>(a.V), e0 + C2);
    const float mass = sum_wg(lane_mass<DT>(a, w, e0, e1));
    if (threadIdx.x == 0) {
        if (!ok) flag_timeout(a, b);
        publish_f32(&a.sums[static_cast<int64_t>(b) * a.nchunk2 + ch], a.tag, mass);
    }
}

// ------------------------------------------------------------ finish item

template <class DT>
__device__ __forceinline__ void finish_item(const ChainArgs &a, int b, bool may_wait) {
    constexpr int VEC = DT::kVec;
    constexpr int C2 = Chunk2<DT>::kElems;
    constexpr int kSeg = C2 / kWG;  // contiguous entries per thread in the final scan
    const int K = a.K, V = a.V, tid = threadIdx.x;
    __shared__ float s_m[kSumsLds];
    __shared__ float s_S, s_tau, s_base;
    __shared__ int s_cstar;
    __shared__ uint64_t s_info[5];
    SeqInfo &si = a.seq[b];
    uint64_t *sums = a.sums + static_cast<int64_t>(b) * a.nchunk2;
    const int nc = a.nchunk2;
    const bool staged = nc <= kSumsLds;
    const float us = a.u_sample[b];

    // Wait until the sequence record and every chunk mass are current.
    const uint64_t t0 = wall_clock64();
    bool timed_out = false;
    for (;;) {
        int stale = 0;
        if (tid < 5) {
            const uint64_t *f = tid == 0 ? &si.j
                                : tid == 1 ? &si.rt
                                : tid == 2 ? &si.izt
                                : tid == 3 ? &si.rd
                                           : &si.izd;
            const uint64_t v = fetch(f);
            if (!current(v, a.tag)) stale = 1;
            s_info[tid] = v;
        }
        for (int i = tid; i < nc; i += kWG) {
            const uint64_t v = fetch(&sums[i]);
            if (!current(v, a.tag)) stale = 1;
            else if (staged) s_m[i] = word_f32(v);
        }
        if (a.out_diag && tid < K &&
            (!current(fetch(&si.P[tid]), a.tag) || !current(fetch(&si.Q[tid]), a.tag)))
            stale = 1;
        const int st = poll_done(stale, may_wait, t0);
        if (st == 1) break;
        if (st < 0) {
            timed_out = true;
            break;
        }
    }
    if (current(fetch(&si.timeout), a.tag)) timed_out = true;
    int j;
    DrawRow w = draw_row(a, b, s_info, j);

    // Total mass, chunk masses added in chunk order.
    if (tid == 0) {
        float S = 0.f;
        for (int i = 0; i < nc; ++i) S += staged ? s_m[i] : word_f32(fetch(&sums[i]));
        s_S = S;
    }
    __syncthreads();
    if (w.resid && s_S == 0.f) {
        // All-zero residual (reachable only through rounding): draw from p_j.
        w.resid = false;
        for (int i = 0; i < nc; ++i) {
            const int64_t e0 = static_cast<int64_t>(i) * C2;
            const int64_t e1 = min(static_cast<int64_t>(V), e0 + C2);
            const float mass = sum_wg(lane_mass<DT>(a, w, e0, e1));
            if (tid == 0) {
                if (staged) s_m[i] = mass;
                else publish_f32(&sums[i], a.tag, mass);
            }
        }
        if (tid == 0) {
            float S = 0.f;
            for (int i = 0; i < nc; ++i) S += staged ? s_m[i] : word_f32(fetch(&sums[i]));
            s_S = S;
        }
        __syncthreads();
    }

    // Crossing chunk: the first whose inclusive running mass exceeds u * S.
    if (tid == 0) {
        const float S = s_S;
        const float tau = us * S;
        float cum = 0.f, base = 0.f, base_last = 0.f;
        int cstar = -1, last_pos = 0;
        for (int i = 0; i < nc; ++i) {
            const float m = staged ? s_m[i] : word_f32(fetch(&sums[i]));
            if (m > 0.f) {
                last_pos = i;
                base_last = cum;
            }
            if (cstar < 0 && cum + m > tau) {
                cstar = i;
                base = cum;
            }
            cum += m;
        }
        if (cstar < 0) {  // u * S rounded up to S: the last chunk with mass
            cstar = last_pos;
            base = base_last;
        }
        s_cstar = cstar;
        s_base = base;
        s_tau = tau;
    }
    __syncthreads();

    // Weights of the crossing chunk: kSeg contiguous entries per thread, in
    // registers; a workgroup exclusive scan gives each thread its start.
    const int64_t c0 = static_cast<int64_t>(s_cstar) * C2;
    const int n = static_cast<int>(min(static_cast<int64_t>(C2), static_cast<int64_t>(V) - c0));
    const int s0 = tid * kSeg;
    float wt[kSeg];
    if (V % VEC == 0) {
        constexpr int NQ = kSeg / VEC;
        const uint4 *tp = static_cast<const uint4 *>(a.target);
        const uint4 *dp = static_cast<const uint4 *>(a.draft);
        uint4 rt[NQ], rd[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int e = s0 + q * VEC;
            if (e < n) {
                rt[q] = tp[(w.trow + c0 + e) / VEC];
                if (w.resid) rd[q] = dp[(w.drow + c0 + e) / VEC];
            }
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int e = s0 + q * VEC;
            float t[VEC], d[VEC];
            if (e < n) {
                unpack<DT>(rt[q], t);
                if (w.resid) unpack<DT>(rd[q], d);
            }
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                wt[q * VEC + i] = e < n ? draw_weight(t[i], w.resid ? d[i] : 0.f, a.c, w.rt, w.izt,
                                                      w.rd, w.izd, w.resid)
                                        : 0.f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kSeg; ++i) {
            const int e = s0 + i;
            float x = 0.f;
            if (e < n) {
                const float t = load_one<DT>(a.target, w.trow + c0 + e);
                const float d = w.resid ? load_one<DT>(a.draft, w.drow + c0 + e) : 0.f;
                x = draw_weight(t, d, a.c, w.rt, w.izt, w.rd, w.izd, w.resid);
            }
            wt[i] = x;
        }
    }
    float local = 0.f;
#pragma unroll
    for (int i = 0; i < kSeg; ++i) local += wt[i];
    float run = s_base + exclusive_scan_wg(local);
    const float tau = s_tau;
    int found = INT32_MAX, last_nz = -1;
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
        run += wt[i];
        if (found == INT32_MAX && run > tau && s0 + i < n) found = s0 + i;
        if (wt[i] > 0.f) last_nz = s0 + i;
    }
    found = min_wg(found);
    last_nz = max_wg(last_nz);
    const int pick = (found != INT32_MAX) ? found : max(last_nz, 0);
    const int32_t token = static_cast<int32_t>(c0 + pick);

    // Emit x_0..x_{j-1}, then the drawn token, then -1 (all -1 after a timeout).
    for (int k = tid; k <= K; k += kWG) {
        int32_t o = -1;
        if (!timed_out) {
            if (k < j) o = a.tokens[b * K + k];
            else if (k == j) o = token;
        }
        a.out_tokens[static_cast<int64_t>(b) * (K + 1) + k] = o;
        if (a.out_diag) {
            float4 dg = make_float4(0.f, 0.f, 0.f, 0.f);
            if (k < K) {
                const float P = word_f32(fetch(&si.P[k])), Q = word_f32(fetch(&si.Q[k]));
                dg.x = P;
                dg.y = Q;
                dg.z = Q > 0.f ? P / Q : (P > 0.f ? INFINITY : 0.f);
            }
            if (k == j) dg.w = s_S;
            reinterpret_cast<float4 *>(a.out_diag)[static_cast<int64_t>(b) * (K + 1) + k] = dg;
        }
    }
    if (tid == 0) a.out_accepted[b] = timed_out ? -1 : j;
}

// ------------------------------------------------------------ kernels

template <class DT, int U>
__global__ __launch_bounds__(kWG) void k_chain_stats(ChainArgs a) {
    stats_item<DT, U>(a, blockIdx.x / a.nchunk, blockIdx.x % a.nchunk);
}

template <class DT>
__global__ __launch_bounds__(kWG) void k_chain_resolve(ChainArgs a) {
    resolve_item<DT>(a, blockIdx.x, false);
}

template <class DT>
__global__ __launch_bounds__(kWG) void k_chain_mass(ChainArgs a) {
    mass_item<DT>(a, blockIdx.x / a.nchunk2, blockIdx.x % a.nchunk2, false);
}

template <class DT>
__global__ __launch_bounds__(kWG) void k_chain_finish(ChainArgs a) {
    finish_item<DT>(a, blockIdx.x, false);
}

template <class DT, int U>
__global__ __launch_bounds__(kWG) void k_chain_fused(ChainArgs a, FusedPlan f) {
    int kind, seq, idx;
    fused_item(f, blockIdx.x, kind, seq, idx);
    if (kind == kItemStats) {
        const int64_t row = static_cast<int64_t>(seq) * (2 * a.K + 1) + idx / a.nchunk;
        stats_item<DT, U>(a, row, idx % a.nchunk);
    } else if (kind == kItemResolve) {
        resolve_item<DT>(a, seq, true);
    } else if (kind == kItemMass) {
        mass_item<DT>(a, seq, idx, true);
    } else {
        finish_item<DT>(a, seq, true);
    }
}

__global__ void k_zero_words(uint32_t *p, int64_t n) {
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

}  // namespace

hipError_t launch_chain_stats(const ChainArgs &a, int dtype, hipStream_t s) {
    const int64_t grid = static_cast<int64_t>(a.B) * (2 * a.K + 1) * a.nchunk;
    if (dtype == 1)
        k_chain_stats<Bf16, 4><<<dim3(static_cast<uint32_t>(grid)), dim3(kWG), 0, s>>>(a);
    else
        k_chain_stats<F32, 4><<<dim3(static_cast<uint32_t>(grid)), dim3(kWG), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_chain_sample(const ChainArgs &a, int dtype, hipStream_t s) {
    const int64_t grid = static_cast<int64_t>(a.B) * a.nchunk2;
    const dim3 seqs(static_cast<uint32_t>(a.B));
    if (dtype == 1) {
        k_chain_resolve<Bf16><<<seqs, dim3(kWG), 0, s>>>(a);
        k_chain_mass<Bf16><<<dim3(static_cast<uint32_t>(grid)), dim3(kWG), 0, s>>>(a);
        k_chain_finish<Bf16><<<seqs, dim3(kWG), 0, s>>>(a);
    } else {
        k_chain_resolve<F32><<<seqs, dim3(kWG), 0, s>>>(a);
        k_chain_mass<F32><<<dim3(static_cast<uint32_t>(grid)), dim3(kWG), 0, s>>>(a);
        k_chain_finish<F32><<<seqs, dim3(kWG), 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_chain_fused(const ChainArgs &a, const FusedPlan &f, int dtype, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(f.total));
    if (dtype == 1)
        k_chain_fused<Bf16, 4><<<grid, dim3(kWG), 0, s>>>(a, f);
    else
        k_chain_fused<F32, 4><<<grid, dim3(kWG), 0, s>>>(a, f);
    return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t *p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t want = (n + kWG - 1) / kWG;
    const int64_t blocks = want < 1024 ? want : 1024;
    k_zero_words<<<dim3(static_cast<uint32_t>(blocks)), dim3(kWG), 0, s>>>(p, n);
    return hipGetLastError();
}

}  // namespace sv
