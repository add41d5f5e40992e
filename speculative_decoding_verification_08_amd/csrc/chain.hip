// Chain verify at T > 0 on gfx950: two kernels in stream order.
//
// k_chain_stats streams every logit of the step once.  One workgroup takes
// one 16 KB vocabulary chunk of one row (target rows 0..K and draft rows
// 0..K-1 of a sequence), folds it into softmax statistics (ref, z) and
// publishes them (and, if its chunk holds the row's drafted token, that
// logit).  This is the HBM-bound pass that carries the bytes; no workgroup of
// it waits for another.
//
// k_chain_draw runs one workgroup per (sequence b, 16 KB chunk of a row).
// Each merges b's row statistics, evaluates the accept test of every drafted
// token (u < p(x)/q(x), French lesson "Décodage spéculatif et Eagle", section
// "La règle de l'exactitude"; forum post "Speculative Decoding: от идеи до
// SOTA", §3) and finds the first rejection j.  It holds its chunk of row j in
// registers and publishes the chunk's draw masses -- max(0, p_j - q_j) after a
// rejection (the residual of the same passages) and p_j, the bonus draw's
// weights when every draft was accepted.  Once every chunk's masses are
// visible, all of b's workgroups find the chunk whose running mass first
// exceeds u * S; that chunk's workgroup picks the token from its registers and
// writes the sequence's outputs.
//
// Hand-over words are 64 bits: the call's tag above a 32-bit value, written
// with device-scope atomic stores and read with device-scope atomic loads; a
// reader checks the tag, so nothing left by an earlier call is taken for
// fresh, and polls (bounded in time) until the word is visible; the
// workspace needs no initialisation.  A draw workgroup waits for the other
// draw workgroups of its sequence, which the hardware dispatches together (a
// sequence has at most 64 of them, far fewer than the chip holds).
#include "device.hpp"
#include "plan.hpp"

namespace sv {
namespace {

// ------------------------------------------------------------ hand-over

constexpr uint64_t kWaitTicks = 200000000ull;  // 2 s of the 100 MHz wall clock

__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t bits) {
    return (static_cast<uint64_t>(tag) << 32) | bits;
}
// Publish without waiting (a device-scope store; readers check the tag).
__device__ __forceinline__ void publish(uint64_t *p, uint32_t tag, uint32_t bits) {
    __hip_atomic_store(p, tagged(tag, bits), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// ------------------------------------------------------------ stats item

// Row r of sequence b (r <= K: target row r; r > K: draft row r - K - 1),
// chunk ch.
template <class DT, int U>
__device__ __forceinline__ void stats_item(const ChainArgs &a, int64_t b, int r, int ch) {
    constexpr int VEC = DT::kVec;
    const int K = a.K, V = a.V, R = 2 * K + 1;
    const int64_t row = b * R + r;
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

// Running masses of a sequence's draw chunks, scanned 64 chunks at a time
// by one wavefront in a fixed order (chunk masses from LDS when staged, else
// from the published words).  Returns S, the total, in every lane.  With
// `cstar`, also finds the crossing chunk: the first whose inclusive running
// mass exceeds tau (the inverse CDF, strict), else the last chunk with mass
// (tau rounded up to S), and `base`, the running mass before it.
__device__ __forceinline__ float scan_masses(const float *s_m, const uint64_t *sums, int nc, bool staged,
                             float tau, int *cstar, float *base) {
    const int lane = threadIdx.x % kWave;
    float carry = 0.f, last_base = 0.f;
    int found = -1, last_pos = 0;
    float found_base = 0.f;
    for (int i0 = 0; i0 < nc; i0 += kWave) {
        const int i = i0 + lane;
        float m = 0.f;
        if (i < nc) m = staged ? s_m[i] : word_f32(fetch(&sums[i]));
        const float incl = carry + wave_incl_sum(m);
        float excl = wave_excl_from_incl(incl);
        if (lane == 0) excl = carry;
        if (cstar) {
            const uint64_t cross = __ballot(i < nc && incl > tau);
            if (found < 0 && cross) {
                const int l = __ffsll(static_cast<unsigned long long>(cross)) - 1;
                found = i0 + l;
                found_base = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(excl), l));
            }
            const uint64_t pos = __ballot(i < nc && m > 0.f);
            if (pos) {
                const int l = 63 - __clzll(static_cast<long long>(pos));
                last_pos = i0 + l;
                last_base = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(excl), l));
            }
        }
        carry = wave_last(incl);
    }
    if (cstar) {
        *cstar = found >= 0 ? found : last_pos;
        *base = found >= 0 ? found_base : last_base;
    }
    return carry;
}

// Resolve of sequence b inside a draw workgroup, from the statistics the
// first kernel left (ordered before this kernel by the stream): merges each
// row's chunks with a fixed DPP tree, evaluates the accept test of every
// drafted token (u < P/Q, strict; Q = 0 accepts iff P > 0) and returns j, the
// first rejected position (K if none), with row j's statistics in `w`.
// `ok` is false if a word was not written for this call.  With `diag` the
// workgroup also writes p_k(x_k), q_k(x_k) and their ratio to out_diag.
template <class DT>
__device__ __forceinline__ int resolve_local(const ChainArgs &a, int b, DrawRow &w, bool &ok,
                                             bool diag, float *lds) {
    float *s_ref = lds, *s_z = s_ref + (2 * kMaxK + 1);
    float *s_pr = s_z + (2 * kMaxK + 1), *s_pz = s_pr + kMergeLds;
    __shared__ int s_j, s_stale;
    const int K = a.K, V = a.V, R = 2 * K + 1, tid = threadIdx.x, lane = tid % kWave;
    const int np = R * a.nchunk;
    const uint64_t *part = a.partial + 2 * static_cast<int64_t>(b) * np;
    const uint64_t *gat = a.gathered + static_cast<int64_t>(b) * R;
    const bool staged = np <= kMergeLds;
    // One round trip: partials, drafted-token logits and uniforms are all
    // loaded (from clamped indices, without branches) before any is used.
    const float *ua = K > 0 ? a.u_accept + static_cast<int64_t>(b) * K : a.u_sample + b;
    float u = ua[min(tid, max(K - 1, 0))];
    const uint64_t wt = gat[min(tid, R - 1)], wd = gat[min(K + 1 + tid, R - 1)];
    const int i0 = min(tid, np - 1);
    const uint64_t wr0 = part[2 * i0], wz0 = part[2 * i0 + 1];
    int stale = 0;
    float lt = 0.f, ld = 0.f;
    if (tid < K) {
        stale |= !current(wt, a.tag) || !current(wd, a.tag);
        lt = word_f32(wt);
        ld = word_f32(wd);
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
    if (tid == 0) s_stale = 0;
    __syncthreads();
    // Row r's chunk statistics are merged by wave r % kWaves: lane i folds
    // chunks i, i + 64, ... in order, then a fixed DPP tree merges the lanes
    // and lane 63's result is the row's.
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
        mz_wave_merge(ref, z);
        if (lane == kWave - 1) {
            s_ref[r] = ref;
            s_z[r] = z;
        }
    }
    if (stale || !fresh) s_stale = 1;  // benign race: every writer stores 1
    __syncthreads();
    ok = !s_stale;
    // Accept test on wave 0 (K <= 64), first rejection by ballot.
    if (tid < kWave) {
        bool reject = false;
        if (tid < K) {
            const float P = exp2_hw(fmaf(lt, a.c, -s_ref[tid])) / s_z[tid];
            const float Q = exp2_hw(fmaf(ld, a.c, -s_ref[K + 1 + tid])) / s_z[K + 1 + tid];
            reject = !(Q > 0.f ? (u < P / Q) : (P > 0.f));
            if (diag && a.out_diag) {
                float *dg = a.out_diag + 4 * (static_cast<int64_t>(b) * (K + 1) + tid);
                dg[0] = P;
                dg[1] = Q;
                dg[2] = Q > 0.f ? P / Q : (P > 0.f ? INFINITY : 0.f);
            }
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

// ------------------------------------------------------------ draw item

// Workgroup (b, ch) of the draw.  It holds entries [ch*C2, ch*C2 + C2) of row
// j in registers (kSeg contiguous entries per thread), publishes the chunk's
// residual mass sum max(0, p_j - q_j) and target mass sum p_j, and prepares
// the running sums inside its chunk while the sequence's other chunks
// publish theirs.  Once all are visible every draw workgroup of the sequence
// computes the same S and the same crossing chunk -- the first whose
// inclusive running mass exceeds u * S (the inverse CDF, strict), else the
// last chunk with mass -- and the workgroup owning it picks the token and
// writes the sequence's outputs.  An all-zero residual (reachable only
// through rounding) draws from p_j; the bonus draw (j = K) always uses p_K.
template <class DT, bool VecOk>
__device__ __forceinline__ void draw_item(const ChainArgs &a, int b, int ch, float *s_m) {
    constexpr int VEC = DT::kVec;
    constexpr int C2 = Chunk2<DT>::kElems;
    constexpr int kSeg = C2 / kWG;  // contiguous entries per thread
    constexpr int NQ = kSeg / VEC;
    const int K = a.K, V = a.V, tid = threadIdx.x;
    const int nc = a.nchunk2;
    __shared__ float s_S, s_tau, s_base;
    __shared__ int s_cstar, s_fresh, s_resid;

    static_assert(kMaxK + 1 <= kWG, "one thread per emitted token");
    // Drafted tokens for the emission, loaded now (thread k emits token k).
    const int32_t *tk = K > 0 ? a.tokens + static_cast<int64_t>(b) * K
                              : reinterpret_cast<const int32_t *>(a.u_sample + b);
    const int32_t my_tok = tk[min(tid, max(K - 1, 0))];

    const float us = a.u_sample[b];

    DrawRow w;
    bool ok;
    const int j = resolve_local<DT>(a, b, w, ok, ch == 0, s_m);

    // This thread's entries of the chunk, both kinds of weight.
    const int64_t c0 = static_cast<int64_t>(ch) * C2;
    const int n = static_cast<int>(min(static_cast<int64_t>(C2), static_cast<int64_t>(V) - c0));
    const int s0 = tid * kSeg;
    uint4 rt[NQ], rd[NQ];
    if constexpr (VecOk) {
        // All loads issued before any use; entries past the chunk are clamped
        // to its last vector and get weight 0.  Without a draft row (bonus
        // draw) the target row is read twice and the copy is unused.
        const uint4 *tp = static_cast<const uint4 *>(a.target);
        const uint4 *dp = w.resid ? static_cast<const uint4 *>(a.draft) : tp;
        const int64_t tb = (w.trow + c0) / VEC, db = ((w.resid ? w.drow : w.trow) + c0) / VEC;
        const int last = n / VEC - 1;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int o = min((s0 + q * VEC) / VEC, last);
            rt[q] = tp[tb + o];
            rd[q] = dp[db + o];
        }
    } else {
        // Unaligned rows: entries one by one, packed into the same layout.
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            uint32_t wt4[4], wd4[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                uint32_t tb = 0, db = 0;
#pragma unroll
                for (int e2 = 0; e2 < VEC / 4; ++e2) {
                    const int e = min(s0 + q * VEC + h * (VEC / 4) + e2, n - 1);
                    const float t = load_one<DT>(a.target, w.trow + c0 + e);
                    const float d = w.resid ? load_one<DT>(a.draft, w.drow + c0 + e) : 0.f;
                    if (VEC == 8) {
                        tb |= (__float_as_uint(t) >> 16) << (16 * e2);
                        db |= (__float_as_uint(d) >> 16) << (16 * e2);
                    } else {
                        tb = __float_as_uint(t);
                        db = __float_as_uint(d);
                    }
                }
                wt4[h] = tb;
                wd4[h] = db;
            }
            rt[q] = make_uint4(wt4[0], wt4[1], wt4[2], wt4[3]);
            rd[q] = make_uint4(wd4[0], wd4[1], wd4[2], wd4[3]);
        }
    }
    // Weights of entry (q, i): p, and max(0, p - q) after a rejection.
    auto weights = [&](int q, float (&wp)[VEC], float (&wr)[VEC]) {
        float t[VEC], d[VEC];
        unpack<DT>(rt[q], t);
        unpack<DT>(rd[q], d);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const bool in = s0 + q * VEC + i < n;
            wp[i] = in ? draw_weight(t[i], 0.f, a.c, w.rt, w.izt, 0.f, 0.f, false) : 0.f;
            wr[i] = in && w.resid
                        ? draw_weight(t[i], d[i], a.c, w.rt, w.izt, w.rd, w.izd, true)
                        : 0.f;
        }
    };
    float lp = 0.f, lr = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        float wp[VEC], wr[VEC];
        weights(q, wp, wr);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            lp += wp[i];
            lr += wr[i];
        }
        asm volatile("" : "+v"(lp), "+v"(lr));  // one slot at a time
    }
    // The raw entries stay in registers for the crossing search; mark them
    // rewritten so the weights are recomputed there instead of kept alive.
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        asm volatile("" : "+v"(rt[q].x), "+v"(rt[q].y), "+v"(rt[q].z), "+v"(rt[q].w));
        asm volatile("" : "+v"(rd[q].x), "+v"(rd[q].y), "+v"(rd[q].z), "+v"(rd[q].w));
    }
    // Running sums inside the chunk and the chunk's masses, both kinds, in
    // one pass (published afterwards: a barrier after a device-scope store
    // would wait for it to complete).
    uint64_t *sums = a.sums + 2 * static_cast<int64_t>(b) * nc;
    float ex_r, ex_p, mr, mp;
    wg_excl_scan2(lr, lp, ex_r, ex_p, mr, mp);
    if (tid == 0) {
        publish_f32(&sums[2 * ch], a.tag, mr);
        publish_f32(&sums[2 * ch + 1], a.tag, mp);
    }

    // Wait (bounded) for every chunk's masses; stage the chosen kind later.
    const bool staged = nc <= kSumsLds;
    if (tid < kWave) {
        bool fresh = false;
        const uint64_t t0 = wall_clock64();
        for (;;) {
            fresh = true;
            for (int i = tid; i < nc; i += kWave) {
                const uint64_t vr = fetch(&sums[2 * i]), vp = fetch(&sums[2 * i + 1]);
                fresh = fresh && current(vr, a.tag) && current(vp, a.tag);
            }
            fresh = __all(fresh);
            if (fresh || wall_clock64() - t0 > kWaitTicks) break;
            __builtin_amdgcn_s_sleep(2);
        }
        if (tid == 0) s_fresh = fresh;
    }
    __syncthreads();
    ok = ok && s_fresh;
    if (!ok) {
        // A bounded wait ran out: the last chunk's workgroup marks the
        // sequence as failed.
        if (ch == nc - 1) {
            for (int k = tid; k <= K; k += kWG)
                a.out_tokens[static_cast<int64_t>(b) * (K + 1) + k] = -1;
            if (tid == 0) a.out_accepted[b] = -1;
        }
        return;
    }
    // Residual or p: the same decision in every workgroup of the sequence.
    if (tid < kWave) {
        for (int i = tid; i < nc; i += kWave)
            if (staged) s_m[i] = word_f32(fetch(&sums[2 * i]));
        float S = staged ? scan_masses(s_m, sums, nc, true, 0.f, nullptr, nullptr) : 0.f;
        if (!staged) {
            float carry = 0.f;
            for (int i0 = 0; i0 < nc; i0 += kWave) {
                const int i = i0 + tid;
                const float m = i < nc ? word_f32(fetch(&sums[2 * i])) : 0.f;
                carry = carry + wave_last(wave_incl_sum(m));
            }
            S = carry;
        }
        const bool resid = w.resid && S > 0.f;
        if (!resid) {
            for (int i = tid; i < nc; i += kWave)
                if (staged) s_m[i] = word_f32(fetch(&sums[2 * i + 1]));
        }
        if (tid == 0) s_resid = resid;
    }
    __syncthreads();
    const bool resid = s_resid;
    if (tid < kWave) {
        // With unstaged masses the scan reads the chosen words in place.
        const uint64_t *src = sums + (resid ? 0 : 1);
        float S;
        if (staged) {
            S = scan_masses(s_m, nullptr, nc, true, 0.f, nullptr, nullptr);
        } else {
            float carry = 0.f;
            for (int i0 = 0; i0 < nc; i0 += kWave) {
                const int i = i0 + tid;
                const float m = i < nc ? word_f32(fetch(&src[2 * i])) : 0.f;
                carry = carry + wave_last(wave_incl_sum(m));
            }
            S = carry;
        }
        const float tau = us * S;
        int cstar = 0;
        float base = 0.f;
        if (staged) {
            scan_masses(s_m, nullptr, nc, true, tau, &cstar, &base);
        } else {
            // In place: the same scan over the chosen words.
            float carry = 0.f, last_base = 0.f, found_base = 0.f;
            int found = -1, last_pos = 0;
            for (int i0 = 0; i0 < nc; i0 += kWave) {
                const int i = i0 + tid;
                const float m = i < nc ? word_f32(fetch(&src[2 * i])) : 0.f;
                const float incl = carry + wave_incl_sum(m);
                float excl = wave_excl_from_incl(incl);
                if (tid == 0) excl = carry;
                const uint64_t cross = __ballot(i < nc && incl > tau);
                if (found < 0 && cross) {
                    const int l = __ffsll(static_cast<unsigned long long>(cross)) - 1;
                    found = i0 + l;
                    found_base = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(excl), l));
                }
                const uint64_t pos = __ballot(i < nc && m > 0.f);
                if (pos) {
                    const int l = 63 - __clzll(static_cast<long long>(pos));
                    last_pos = i0 + l;
                    last_base = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(excl), l));
                }
                carry = wave_last(incl);
            }
            cstar = found >= 0 ? found : last_pos;
            base = found >= 0 ? found_base : last_base;
        }
        if (tid == 0) {
            s_S = S;
            s_tau = tau;
            s_cstar = cstar;
            s_base = base;
        }
    }
    __syncthreads();
    if (s_cstar != ch) return;

    // The crossing chunk: the first entry (index order) whose running mass
    // exceeds tau; if rounding leaves none, the last entry with weight.
    const float tau = s_tau;
    float run = s_base + (resid ? ex_r : ex_p);
    int found = INT32_MAX, last_nz = -1;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        float wp[VEC], wr[VEC];
        weights(q, wp, wr);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const float x = resid ? wr[i] : wp[i];
            run += x;
            if (x > 0.f) {
                if (found == INT32_MAX && run > tau) found = s0 + q * VEC + i;
                last_nz = s0 + q * VEC + i;
            }
        }
        asm volatile("" : "+v"(run), "+v"(found), "+v"(last_nz));  // one slot at a time
    }
    wg_min_max(found, last_nz, found, last_nz);
    const int pick = found != INT32_MAX ? found : max(last_nz, 0);
    const int32_t token = static_cast<int32_t>(c0 + pick);

    // Emit x_0..x_{j-1}, then the drawn token, then -1.
    for (int k = tid; k <= K; k += kWG) {
        int32_t o = -1;
        if (k < j) o = my_tok;  // k == tid here: K + 1 <= 65 < kWG
        else if (k == j) o = token;
        a.out_tokens[static_cast<int64_t>(b) * (K + 1) + k] = o;
        if (a.out_diag) {
            float *dg = a.out_diag + 4 * (static_cast<int64_t>(b) * (K + 1) + k);
            if (k == K) dg[0] = dg[1] = dg[2] = 0.f;
            dg[3] = k == j ? s_S : 0.f;
        }
    }
    if (tid == 0) a.out_accepted[b] = j;
}

template <class DT, int U>
__global__ __launch_bounds__(kWG) void k_chain_stats(ChainArgs a) {
    // 32-bit index arithmetic (the grid is below 2^31 workgroups): a 64-bit
    // division is a long instruction sequence ahead of the first load.
    const uint32_t R = 2 * a.K + 1, S = R * a.nchunk;
    const uint32_t g = blockIdx.x, b = g / S, pos = g - b * S, r = pos / a.nchunk;
    stats_item<DT, U>(a, b, static_cast<int>(r), static_cast<int>(pos - r * a.nchunk));
}

template <class DT, bool VecOk>
__global__ __launch_bounds__(kWG) void k_chain_draw(ChainArgs a) {
    const uint32_t nc = a.nchunk2, g = blockIdx.x, b = g / nc;
    __shared__ float lds[kDrawLds];
    draw_item<DT, VecOk>(a, static_cast<int>(b), static_cast<int>(g - b * nc), lds);
}

}  // namespace

hipError_t launch_chain_stats(const ChainArgs &a, int dtype, hipStream_t s) {
    const dim3 g(static_cast<uint32_t>(static_cast<int64_t>(a.B) * (2 * a.K + 1) * a.nchunk)),
        blk(kWG);
    if (dtype == 1)
        k_chain_stats<Bf16, 4><<<g, blk, 0, s>>>(a);
    else
        k_chain_stats<F32, 4><<<g, blk, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_chain_draw(const ChainArgs &a, int dtype, hipStream_t s) {
    const dim3 g(static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.nchunk2)), blk(kWG);
    if (dtype == 1) {
        if (a.V % Bf16::kVec == 0) k_chain_draw<Bf16, true><<<g, blk, 0, s>>>(a);
        else k_chain_draw<Bf16, false><<<g, blk, 0, s>>>(a);
    } else {
        if (a.V % F32::kVec == 0) k_chain_draw<F32, true><<<g, blk, 0, s>>>(a);
        else k_chain_draw<F32, false><<<g, blk, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace sv
