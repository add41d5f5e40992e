// Chain verify at T > 0 on gfx950: two kernels in stream order.
//
// k_chain_stats streams every logit of the step once.  One workgroup takes one
// 16 KB vocabulary chunk of one row (target rows 0..K and draft rows 0..K-1 of
// a sequence), folds it into softmax statistics (ref, z) and publishes them;
// the workgroup whose chunk holds the row's drafted token also publishes that
// logit.  This is the HBM-bound pass that carries the bytes.
//
// k_chain_tail runs one workgroup per (sequence b, 16 KB chunk of a row).
// Each merges the sequence's row statistics, evaluates the accept test of
// every drafted token (u < p(x)/q(x), French lesson "La règle de
// l'exactitude"; forum post §3) and finds the first rejection j.  It then
// sums the draw weights of its chunk of row j: max(0, p_j - q_j) after a
// rejection (the residual of the same passages) or p_K when every draft was
// accepted (the bonus draw), publishes that mass and counts itself done.  The
// last workgroup of the sequence to finish finds the chunk whose running mass
// first exceeds u * S, scans that chunk in index order and writes the emitted
// tokens.
//
// Hand-over words are 64 bits: the call's tag above a 32-bit value.  Between
// the kernels the boundary orders everything; inside the tail kernel a chunk
// mass is published with a device-scope atomic exchange that has returned
// before the counter increment, and read with device-scope atomic loads, so
// no fence (an L2 write-back and invalidate per workgroup on this chip) is
// needed.  The tags let the tail kernel check that every word it reads was
// written for this call.  The per-sequence counters are zeroed by the
// statistics kernel, so the workspace needs no initialisation.
#include "device.hpp"
#include "plan.hpp"

namespace sv {
namespace {

// ------------------------------------------------------------ hand-over

// Words the statistics kernel leaves for the tail kernel: plain stores and
// loads (the kernel boundary orders them, and the tail kernel's workgroups of
// one sequence share them through L2).
__device__ __forceinline__ void put_f32(uint64_t *p, uint32_t tag, float v) {
    *p = (static_cast<uint64_t>(tag) << 32) | __float_as_uint(v);
}
// Keeps an atomic's returned value alive, so the atomic is issued with return
// and a later s_waitcnt covers its completion.
__device__ __forceinline__ void keep(uint64_t v) {
    asm volatile("" ::"v"(static_cast<uint32_t>(v)), "v"(static_cast<uint32_t>(v >> 32)));
}
// Publish and wait until the exchange has been performed device-wide.
__device__ __forceinline__ void publish_f32_sync(uint64_t *p, uint32_t tag, float v) {
    keep(__hip_atomic_exchange(p, (static_cast<uint64_t>(tag) << 32) | __float_as_uint(v),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    __builtin_amdgcn_s_waitcnt(0);
}
// Publish without waiting (a device-scope store; readers check the tag).
__device__ __forceinline__ void publish_f32(uint64_t *p, uint32_t tag, float v) {
    __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | __float_as_uint(v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr uint64_t kWaitTicks = 200000000ull;  // 2 s of the 100 MHz wall clock

// Words exchanged inside the tail kernel: device-scope atomics.
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
            put_f32(&a.gathered[row], a.tag, load_one<DT>(base, trow * V + x));
    }
    mz_reduce_wg(ref, z);
    if (threadIdx.x == 0) {
        uint64_t *w = a.partial + 2 * (row * a.nchunk + ch);
        put_f32(w, a.tag, ref);
        put_f32(w + 1, a.tag, z);
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
        // Every lane issues all its loads before using any: indices past the
        // chunk are clamped to its last vector and their weights dropped (a
        // branch around each load would make each one wait for the last).
        // The bonus draw has no draft row and re-reads the target row instead.
        const uint4 *tp = static_cast<const uint4 *>(a.target);
        const uint4 *dp = w.resid ? static_cast<const uint4 *>(a.draft) : tp;
        const int64_t v0 = (w.trow + e0) / VEC, nv = (e1 - e0) / VEC;
        const int64_t d0 = ((w.resid ? w.drow : w.trow) + e0) / VEC;
        uint4 rt[NV], rd[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int64_t o = min(static_cast<int64_t>(threadIdx.x + i * kWG), nv - 1);
            rt[i] = tp[v0 + o];
            rd[i] = dp[d0 + o];
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const bool in = threadIdx.x + i * kWG < nv;
            float t[VEC], d[VEC];
            unpack<DT>(rt[i], t);
            unpack<DT>(rd[i], d);
            float part = 0.f;
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                part += draw_weight(t[q], d[q], a.c, w.rt, w.izt, w.rd, w.izd, w.resid);
            acc += in ? part : 0.f;
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

// Inclusive scan across a wavefront (lane order).
__device__ __forceinline__ float wave_incl_scan(float x) {
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Running masses of a sequence's draw chunks, scanned 64 chunks at a time
// by one wavefront in a fixed order (chunk masses from LDS when staged, else
// from the published words).  Returns S, the total, in every lane.  With
// `cstar`, also finds the crossing chunk: the first whose inclusive running
// mass exceeds tau (the inverse CDF, strict), else the last chunk with mass
// (tau rounded up to S), and `base`, the running mass before it.
__device__ float scan_masses(const float *s_m, const uint64_t *sums, int nc, bool staged,
                             float tau, int *cstar, float *base) {
    const int lane = threadIdx.x % kWave;
    float carry = 0.f, last_base = 0.f;
    int found = -1, last_pos = 0;
    float found_base = 0.f;
    for (int i0 = 0; i0 < nc; i0 += kWave) {
        const int i = i0 + lane;
        float m = 0.f;
        if (i < nc) m = staged ? s_m[i] : word_f32(fetch(&sums[i]));
        const float incl = carry + wave_incl_scan(m);
        float excl = __shfl_up(incl, 1);
        if (lane == 0) excl = carry;
        if (cstar) {
            const uint64_t cross = __ballot(i < nc && incl > tau);
            if (found < 0 && cross) {
                const int l = __ffsll(static_cast<unsigned long long>(cross)) - 1;
                found = i0 + l;
                found_base = __shfl(excl, l);
            }
            const uint64_t pos = __ballot(i < nc && m > 0.f);
            if (pos) {
                const int l = 63 - __clzll(static_cast<long long>(pos));
                last_pos = i0 + l;
                last_base = __shfl(excl, l);
            }
        }
        carry = __shfl(incl, kWave - 1);
    }
    if (cstar) {
        *cstar = found >= 0 ? found : last_pos;
        *base = found >= 0 ? found_base : last_base;
    }
    return carry;
}

// Merges sequence b's row statistics over chunks (in a fixed order) and
// evaluates the accept test of every drafted token.  Returns j, the first
// rejected position (K if none), with row j's statistics in `w` and
// p_k(x_k), q_k(x_k) in s_P, s_Q; `ok` is false if a word was not written for
// this call (the statistics phase did not run with these arguments).
template <class DT>
__device__ int accept_prefix(const ChainArgs &a, int b, float *s_P, float *s_Q, DrawRow &w,
                             bool &ok) {
    __shared__ float s_ref[2 * kMaxK + 1], s_z[2 * kMaxK + 1];
    __shared__ float s_pr[kMergeLds], s_pz[kMergeLds];
    __shared__ int s_j;
    const int K = a.K, V = a.V, R = 2 * K + 1, tid = threadIdx.x;
    const int np = R * a.nchunk;
    const uint64_t *part = a.partial + 2 * static_cast<int64_t>(b) * np;
    const uint64_t *gat = a.gathered + static_cast<int64_t>(b) * R;
    const bool staged = np <= kMergeLds;
    // One round trip: partials, drafted-token logits and uniforms are all
    // loaded (from clamped indices, without branches) before any is used.
    int stale = 0;
    float lt = 0.f, ld = 0.f;
    const float *ua = K > 0 ? a.u_accept + static_cast<int64_t>(b) * K : a.u_sample + b;
    const int kk = min(tid, max(K - 1, 0));
    float u = ua[kk];
    const uint64_t wt = gat[min(tid, R - 1)], wd = gat[min(K + 1 + tid, R - 1)];
    const int i0 = min(tid, np - 1);
    const uint64_t wr0 = part[2 * i0], wz0 = part[2 * i0 + 1];
    if (tid < K) {
        stale |= !current(wt, a.tag) || !current(wd, a.tag);
        lt = word_f32(wt);
        ld = word_f32(wd);
    } else {
        u = 0.f;
    }
    if (staged) {
        if (tid < np) {
            stale |= !current(wr0, a.tag) || !current(wz0, a.tag);
            s_pr[tid] = word_f32(wr0);
            s_pz[tid] = word_f32(wz0);
        }
        for (int i = tid + kWG; i < np; i += kWG) {
            const uint64_t wr = part[2 * i], wz = part[2 * i + 1];
            stale |= !current(wr, a.tag) || !current(wz, a.tag);
            s_pr[i] = word_f32(wr);
            s_pz[i] = word_f32(wz);
        }
    }
    ok = !__syncthreads_or(stale);
    // Row r's chunk statistics are merged by wave r % kWaves: lane i folds
    // chunks i, i + 64, ... in order, then a fixed butterfly merges the lanes
    // and lane 0's result is the row's.
    const int lane = tid % kWave;
    bool fresh = true;
    for (int r = tid / kWave; r < R; r += kWaves) {
        float ref = -INFINITY, z = 0.f;
        for (int i = lane; i < a.nchunk; i += kWave) {
            const int q = r * a.nchunk + i;
            float pr, pz;
            if (staged) {
                pr = s_pr[q];
                pz = s_pz[q];
            } else {
                const uint64_t wr = part[2 * q], wz = part[2 * q + 1];
                fresh = fresh && current(wr, a.tag) && current(wz, a.tag);
                pr = word_f32(wr);
                pz = word_f32(wz);
            }
            mz_merge(ref, z, pr, pz);
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1)
            mz_merge(ref, z, __shfl_xor(ref, off), __shfl_xor(z, off));
        if (lane == 0) {
            s_ref[r] = ref;
            s_z[r] = z;
        }
    }
    if (!staged) ok = ok && !__syncthreads_or(!fresh);
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

// ------------------------------------------------------------ tail kernel

template <class DT>
__global__ __launch_bounds__(kWG) void k_chain_tail(ChainArgs a) {
    constexpr int VEC = DT::kVec;
    constexpr int C2 = Chunk2<DT>::kElems;
    constexpr int kSeg = C2 / kWG;  // contiguous entries per thread in the final scan
    const int K = a.K, V = a.V, tid = threadIdx.x;
    const int b = blockIdx.x / a.nchunk2, ch = blockIdx.x % a.nchunk2;
    const int nc = a.nchunk2;
    __shared__ float s_P[kMaxK], s_Q[kMaxK];
    __shared__ float s_m[kSumsLds];
    __shared__ float s_S, s_tau, s_base;
    __shared__ int s_cstar, s_last;

    static_assert(kMaxK + 1 <= kWG, "one thread per emitted token");
    // Drafted tokens for the emission, loaded now (thread k emits token k).
    const int32_t *tk = K > 0 ? a.tokens + static_cast<int64_t>(b) * K
                              : reinterpret_cast<const int32_t *>(a.u_sample + b);
    const int32_t my_tok = tk[min(tid, max(K - 1, 0))];

    DrawRow w;
    bool ok;
    const int j = accept_prefix<DT>(a, b, s_P, s_Q, w, ok);

    // This workgroup's share: the draw mass of chunk ch of row j.
    uint64_t *sums = a.sums + static_cast<int64_t>(b) * nc;
    {
        const int64_t e0 = static_cast<int64_t>(ch) * C2;
        const int64_t e1 = min(static_cast<int64_t>(V), e0 + C2);
        const float mass = sum_wg(lane_mass<DT>(a, w, e0, e1));
        if (tid == 0) {
            publish_f32(&sums[ch], a.tag, mass);
            const uint32_t done = __hip_atomic_fetch_add(&a.counters[b], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            s_last = done == static_cast<uint32_t>(nc - 1);
        }
        __syncthreads();
        if (!s_last) return;
    }

    // Last workgroup of the sequence: every chunk mass has been published.
    // Wave 0 stages them in LDS (one round trip; read in place past kSumsLds
    // chunks) and scans them across its lanes for S and the crossing chunk.
    const bool staged = nc <= kSumsLds;
    // The masses were stored before their counter increments but may become
    // visible a little later: a bounded poll on the tags.
    if (tid < kWave) {
        bool fresh = false;
        const uint64_t t0 = wall_clock64();
        for (;;) {
            fresh = true;
            for (int i = tid; i < nc; i += kWave) {
                const uint64_t v = fetch(&sums[i]);
                fresh = fresh && current(v, a.tag);
                if (staged) s_m[i] = word_f32(v);
            }
            fresh = __all(fresh);
            if (fresh || wall_clock64() - t0 > kWaitTicks) break;
            __builtin_amdgcn_s_sleep(2);
        }
        if (tid == 0) s_last = fresh;
    }
    __syncthreads();
    ok = ok && s_last;
    if (tid < kWave) {
        const float S = scan_masses(s_m, sums, nc, staged, 0.f, nullptr, nullptr);
        if (tid == 0) s_S = S;
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
                else publish_f32_sync(&sums[i], a.tag, mass);
            }
        }
        __syncthreads();
        if (tid < kWave) {
            const float S = scan_masses(s_m, sums, nc, staged, 0.f, nullptr, nullptr);
            if (tid == 0) s_S = S;
        }
        __syncthreads();
    }
    if (tid < kWave) {
        const float tau = a.u_sample[b] * s_S;
        int cstar;
        float base;
        scan_masses(s_m, sums, nc, staged, tau, &cstar, &base);
        if (tid == 0) {
            s_cstar = cstar;
            s_base = base;
            s_tau = tau;
        }
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
        // All loads issued before any use; entries past the chunk are clamped
        // to its last vector and get weight 0.
        const uint4 *tp = static_cast<const uint4 *>(a.target);
        const uint4 *dp = w.resid ? static_cast<const uint4 *>(a.draft) : tp;
        const int64_t tb = (w.trow + c0) / VEC, db = ((w.resid ? w.drow : w.trow) + c0) / VEC;
        const int last = n / VEC - 1;
        uint4 rt[NQ], rd[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int o = min((s0 + q * VEC) / VEC, last);
            rt[q] = tp[tb + o];
            rd[q] = dp[db + o];
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int e = s0 + q * VEC;
            float t[VEC], d[VEC];
            unpack<DT>(rt[q], t);
            unpack<DT>(rd[q], d);
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                wt[q * VEC + i] = e < n ? draw_weight(t[i], d[i], a.c, w.rt, w.izt, w.rd, w.izd,
                                                      w.resid)
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

    // Emit x_0..x_{j-1}, then the drawn token, then -1 (all -1 if a word
    // was stale: the statistics phase did not run for this call).
    for (int k = tid; k <= K; k += kWG) {
        int32_t o = -1;
        if (ok) {
            if (k < j) o = my_tok;  // k == tid here: K + 1 <= 65 < kWG
            else if (k == j) o = token;
        }
        a.out_tokens[static_cast<int64_t>(b) * (K + 1) + k] = o;
        if (a.out_diag) {
            float4 dg = make_float4(0.f, 0.f, 0.f, 0.f);
            if (k < K) {
                const float P = s_P[k], Q = s_Q[k];
                dg.x = P;
                dg.y = Q;
                dg.z = Q > 0.f ? P / Q : (P > 0.f ? INFINITY : 0.f);
            }
            if (k == j) dg.w = s_S;
            reinterpret_cast<float4 *>(a.out_diag)[static_cast<int64_t>(b) * (K + 1) + k] = dg;
        }
    }
    if (tid == 0) a.out_accepted[b] = ok ? j : -1;
}

template <class DT, int U>
__global__ __launch_bounds__(kWG) void k_chain_stats(ChainArgs a) {
    const int64_t row = blockIdx.x / a.nchunk;
    const int ch = blockIdx.x % a.nchunk;
    // The tail kernel's per-sequence counters start at zero for this call.
    if (threadIdx.x == 0 && ch == 0 && row % (2 * a.K + 1) == 0)
        a.counters[row / (2 * a.K + 1)] = 0u;
    stats_item<DT, U>(a, row, ch);
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

hipError_t launch_chain_tail(const ChainArgs &a, int dtype, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.nchunk2));
    if (dtype == 1)
        k_chain_tail<Bf16><<<grid, dim3(kWG), 0, s>>>(a);
    else
        k_chain_tail<F32><<<grid, dim3(kWG), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sv
