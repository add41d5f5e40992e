// Chain verify at T > 0 on gfx950.
//
// Statistics items stream every logit of the step once.  One workgroup takes
// one 16 KB vocabulary chunk of one row (target rows 0..K and draft rows
// 0..K-1 of a sequence), folds it into softmax statistics (ref, z) and
// publishes them.  This is the HBM-bound work that carries the bytes; no
// statistics workgroup waits for another.
//
// Draw items run one workgroup per (sequence b, 16 KB chunk of a row).  Each
// merges b's row statistics, reads the logits at the drafted tokens from the
// inputs, evaluates the accept test of every drafted token
// (u < p(x)/q(x), French lesson "Décodage spéculatif et Eagle", section "La
// règle de l'exactitude"; forum post "Speculative Decoding: от идеи до SOTA",
// §3) and finds the first rejection j.  It holds its chunk of row j in
// registers and publishes the chunk's draw masses -- max(0, p_j - q_j) after a
// rejection (the residual of the same passages) and p_j, the bonus draw's
// weights when every draft was accepted.  Once every chunk's masses are
// visible, all of b's workgroups find the chunk whose running mass first
// exceeds u * S; that chunk's workgroup picks the token and writes the
// sequence's outputs.
//
// k_chain_fused runs both kinds of item in one grid (the one-call entry
// point); k_chain_stats and k_chain_draw run them as two kernels in stream
// order (the two-phase entry points).  Both give the same bits.
//
// Hand-over words are 64 bits: the call's tag above a 32-bit value, written
// with device-scope atomic stores and read with device-scope atomic loads; a
// reader checks the tag, so nothing left by an earlier call is taken for
// fresh, and waits (bounded in time) until the word is visible.  Tags are
// never 0, so a workspace zeroed once before first use needs no clearing.  A
// workgroup only waits for workgroups of lower index (dispatched before it)
// or for the draw workgroups of its own sequence (a sequence has at most 64,
// far fewer than the chip holds).
#include "device.hpp"
#include "handover.hpp"
#include "plan.hpp"

namespace sv {
namespace {

// ------------------------------------------------------------ stats item

// Row r of sequence b (r <= K: target row r; r > K: draft row r - K - 1),
// chunk ch.
template <class DT, int U>
__device__ __forceinline__ void stats_item(const ChainArgs &a, int64_t b, int r, int ch) {
    constexpr int VEC = DT::kVec;
    const int K = a.K, V = a.V, R = 2 * K + 1;
    const int64_t row = b * R + r;
    const void *base = r <= K ? a.target : a.draft;
    const int64_t trow = r <= K ? b * (K + 1) + r : b * K + (r - K - 1);
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
    mz_reduce_wg(ref, z);
    if (threadIdx.x == 0) {
        uint64_t *w = a.partial + 2 * (row * a.nchunk + ch);
        publish_f32(w, a.tag, ref);
        publish_f32(w + 1, a.tag, z);
    }
}

// ------------------------------------------------------------ draw weights

// Draw weights of one vocabulary entry of row j: p = 2^(l*c - ref) / z of the
// target row, and the residual max(0, p - q) with q likewise from the draft
// row.  Both passes over an entry (chunk masses, then the search inside the
// crossing chunk) evaluate these same expressions, so they agree bit for bit.
struct DrawRow {
    int64_t trow, drow;  // element offsets of target row j and draft row j
    float rt, izt, rd, izd;
    bool resid;          // j < K: a rejection, draw from the residual
};
__device__ __forceinline__ float weight_p(float t, float c, const DrawRow &w) {
    return __fmul_rn(exp2_hw(fmaf(t, c, -w.rt)), w.izt);
}
__device__ __forceinline__ float weight_r(float p, float d, float c, const DrawRow &w) {
    return fmaxf(fmaf(-exp2_hw(fmaf(d, c, -w.rd)), w.izd, p), 0.f);
}

// Bits of -inf: entries past the end of a row are replaced by them, which
// gives them weight 0 in both kinds (c > 0) without a test per entry.
template <class DT>
struct NegInf;
template <>
struct NegInf<Bf16> {
    static constexpr uint32_t kBits = 0xff80ff80u;
};
template <>
struct NegInf<F32> {
    static constexpr uint32_t kBits = 0xff800000u;
};

// Resolve of sequence b inside a draw workgroup.  Each group of 16 lanes
// merges one row's chunk statistics (lane i folds chunks i, i + 16, ... in
// order, then a fixed DPP tree), every wavefront evaluates the accept test of
// every drafted token (u < P/Q, strict; Q = 0 accepts iff P > 0) and takes j,
// the first rejected position (K if none), by ballot, so no second barrier is
// needed.  The accept tests never read the bonus row (target row K), so j < K
// is decided without it; the bonus row is needed only when j = K, and then
// its per-chunk statistics are left in LDS for the bonus draw.  Row j's
// statistics land in `w`.  Without Live the statistics come from a kernel
// ordered before this one by the stream and are read once; with Live the
// statistics workgroups may still be running, so the words are read with
// device-scope loads, and while a needed word is missing one lane of each
// wavefront that saw it waits for it (bounded) and everything is read again.
// `ok` is false if a needed word was not written for this call in time.
// With `diag` the workgroup also writes p_k(x_k), q_k(x_k) and their ratio to
// out_diag.
template <class DT, bool Live, int Fold, int kPasses>
__device__ __forceinline__ int resolve_local(const ChainArgs &a, int b, DrawRow &w, bool &ok,
                                             bool diag, float *lds) {
    // The loads of kPasses row groups (16 rows each) go out together.
    constexpr int kGroup = 16, kGroups = kWG / kGroup;
    float *s_ref = lds, *s_z = s_ref + (2 * kMaxK + 1);
    float *s_kref = lds + kDrawBonusAt, *s_kz = s_kref + kMaxDrawChunks;
    __shared__ int s_stale[2][kWaves + 1];
    const int K = a.K, V = a.V, R = 2 * K + 1, nch = a.nchunk;
    const int tid = threadIdx.x, lane = tid % kWave, grp = tid / kGroup, gl = tid % kGroup;
    const uint64_t *part = a.partial + 2 * static_cast<int64_t>(b) * R * nch;
    // Lane k's position: its uniform, and the drafted token's logits in target
    // row k and draft row k, read straight from the inputs (every wavefront,
    // clamped indices) before anything waits.
    const int kk = min(lane, max(K - 1, 0));
    const float *ua = K > 0 ? a.u_accept + static_cast<int64_t>(b) * K : a.u_sample + b;
    const float u = ua[kk];
    float lt = 0.f, ld = 0.f;
    if (K > 0) {
        const int x = min(max(a.tokens[static_cast<int64_t>(b) * K + kk], 0), V - 1);
        lt = load_one<DT>(a.target, (static_cast<int64_t>(b) * (K + 1) + kk) * V + x);
        ld = load_one<DT>(a.draft, (static_cast<int64_t>(b) * K + kk) * V + x);
    }
    const uint64_t t0 = Live ? wall_clock64() : 0;
    float P = 0.f, Q = 0.f;
    int j = K;
    for (int it = 0;; ++it) {
        // The first missing word this lane found among the rows the accept
        // tests read, and in the bonus row.
        const uint64_t *miss = nullptr, *miss_k = nullptr;
        for (int r0 = 0; r0 < R; r0 += kGroups * kPasses) {
            float ref[kPasses], z[kPasses];
#pragma unroll
            for (int q = 0; q < kPasses; ++q) {
                ref[q] = -INFINITY;
                z[q] = 0.f;
            }
            for (int i0 = 0; i0 < nch; i0 += kGroup * Fold) {
                uint64_t pr[kPasses][Fold], pz[kPasses][Fold];
#pragma unroll
                for (int q = 0; q < kPasses; ++q) {
                    const int rr = min(r0 + grp + kGroups * q, R - 1);
#pragma unroll
                    for (int f = 0; f < Fold; ++f) {
                        const uint64_t *pw = part + 2 * (rr * nch + min(i0 + gl + kGroup * f, nch - 1));
                        if (Live) {
                            pr[q][f] = fetch(pw);
                            pz[q][f] = fetch(pw + 1);
                        } else {
                            const uint4 v = *reinterpret_cast<const uint4 *>(pw);
                            pr[q][f] = (static_cast<uint64_t>(v.y) << 32) | v.x;
                            pz[q][f] = (static_cast<uint64_t>(v.w) << 32) | v.z;
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < kPasses; ++q) {
                    const int r = r0 + grp + kGroups * q, rr = min(r, R - 1);
#pragma unroll
                    for (int f = 0; f < Fold; ++f) {
                        const int i = i0 + gl + kGroup * f;
                        const bool in = r < R && i < nch;
                        const bool cr = current(pr[q][f], a.tag), cz = current(pz[q][f], a.tag);
                        const float fr = in ? word_f32(pr[q][f]) : -INFINITY;
                        const float fz = in ? word_f32(pz[q][f]) : 0.f;
                        if (in && !(cr && cz)) {
                            const uint64_t *mw = part + 2 * (rr * nch + i) + (cr ? 1 : 0);
                            if (r == K) miss_k = miss_k ? miss_k : mw;
                            else miss = miss ? miss : mw;
                        }
                        if (r == K && in) {
                            s_kref[i] = fr;
                            s_kz[i] = fz;
                        }
                        mz_merge(ref[q], z[q], fr, fz);
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < kPasses; ++q) {
                mz_row_merge(ref[q], z[q]);
                const int r = r0 + grp + kGroups * q;
                if (r < R && gl == kGroup - 1) {
                    s_ref[r] = ref[q];
                    s_z[r] = z[q];
                }
            }
        }
        const uint64_t st = __ballot(miss != nullptr), st_k = __ballot(miss_k != nullptr);
        // Double-buffered by iteration: a wavefront may start the next
        // iteration while another still reads this one's flags.
        if (lane == 0) s_stale[it & 1][tid / kWave] = (st ? 1 : 0) | (st_k ? 2 : 0);
        if (tid == 0) s_stale[it & 1][kWaves] = !Live || wall_clock64() - t0 > kWaitTicks;
        __syncthreads();
        int any = 0;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) any |= s_stale[it & 1][k];
        if (!(any & 1)) {
            bool reject = false;
            if (lane < K) {
                P = exp2_hw(fmaf(lt, a.c, -s_ref[lane])) / s_z[lane];
                Q = exp2_hw(fmaf(ld, a.c, -s_ref[K + 1 + lane])) / s_z[K + 1 + lane];
                reject = !(Q > 0.f ? (u < P / Q) : (P > 0.f));
            }
            const uint64_t m = __ballot(reject);
            j = m ? (__ffsll(static_cast<unsigned long long>(m)) - 1) : K;
            if (j < K || !(any & 2)) {
                ok = true;
                break;
            }
        }
        if (s_stale[it & 1][kWaves]) {
            ok = false;
            break;
        }
        // One lane of each wavefront that missed a needed word waits for it.
        const uint64_t need = (any & 1) ? st : st_k;
        if (need && lane == __ffsll(static_cast<unsigned long long>(need)) - 1)
            wait_word((any & 1) ? miss : miss_k, a.tag, t0);
    }
    if (ok && diag && tid < K && a.out_diag) {
        float *dg = a.out_diag + 4 * (static_cast<int64_t>(b) * (K + 1) + lane);
        dg[0] = P;
        dg[1] = Q;
        dg[2] = Q > 0.f ? P / Q : (P > 0.f ? INFINITY : 0.f);
    }
    w.resid = j < K;
    w.rt = s_ref[j];
    w.izt = 1.f / s_z[j];
    w.rd = w.resid ? s_ref[K + 1 + j] : 0.f;
    w.izd = w.resid ? 1.f / s_z[K + 1 + j] : 0.f;
    w.trow = (static_cast<int64_t>(b) * (K + 1) + j) * V;
    w.drow = w.resid ? (static_cast<int64_t>(b) * K + j) * V : 0;
    return j;
}

// Entries per chunk of the residual / bonus pass: 16 KB of one row.
template <class DT>
struct Chunk2 {
    static constexpr int kElems = kChunk2Bytes / (16 / DT::kVec);
    static constexpr int kSeg = kElems / kWG;    // contiguous entries per thread
    static constexpr int kNQ = kSeg / DT::kVec;  // 16-byte vectors per thread and row
    static constexpr int kRawWords = 4 * kNQ;    // 32-bit words per thread and row
};

// This thread's entries [s0, s0 + kSeg) of chunk c0 of row j (target, and
// draft when Resid), as raw 16-byte vectors; entries past the row's end read
// as -inf.  With V a multiple of the vector width all loads are issued before
// any is used; otherwise entries are read one by one into the same layout.
template <class DT, bool VecOk, bool Resid>
__device__ __forceinline__ void load_chunk(const ChainArgs &a, const DrawRow &w, int64_t c0, int n,
                                           int s0, uint4 (&rt)[Chunk2<DT>::kNQ],
                                           uint4 (&rd)[Chunk2<DT>::kNQ]) {
    constexpr int VEC = DT::kVec, NQ = Chunk2<DT>::kNQ;
    constexpr uint32_t kInf = NegInf<DT>::kBits;
    if constexpr (VecOk) {
        const uint4 *tp = static_cast<const uint4 *>(a.target) + (w.trow + c0) / VEC;
        const uint4 *dp = static_cast<const uint4 *>(a.draft) + (w.drow + c0) / VEC;
        const int last = n / VEC - 1;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int o = min(s0 / VEC + q, last);
            rt[q] = tp[o];
            if (Resid) rd[q] = dp[o];
        }
        if (n < Chunk2<DT>::kElems) {  // the row's last chunk: whole vectors past its end
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (s0 + q * VEC >= n) {
                    rt[q] = make_uint4(kInf, kInf, kInf, kInf);
                    rd[q] = rt[q];
                }
        }
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            uint32_t wt4[4], wd4[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                uint32_t tb = 0, db = 0;
#pragma unroll
                for (int e2 = 0; e2 < VEC / 4; ++e2) {
                    const int e = s0 + q * VEC + h * (VEC / 4) + e2, ec = min(e, n - 1);
                    float t = load_one<DT>(a.target, w.trow + c0 + ec);
                    float d = Resid ? load_one<DT>(a.draft, w.drow + c0 + ec) : 0.f;
                    t = e < n ? t : -INFINITY;
                    d = e < n ? d : -INFINITY;
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
}

// Entry e of a thread's raw words (the layout load_chunk fills), widened.
template <class DT>
__device__ __forceinline__ float raw_entry(const uint32_t *words, int e) {
    if constexpr (DT::kVec == 8) {
        const uint32_t v = words[e >> 1];
        return __uint_as_float((e & 1) ? (v & 0xffff0000u) : (v << 16));
    } else {
        return __uint_as_float(words[e]);
    }
}

// ------------------------------------------------------------ draw item

// Row j's entries of this workgroup's chunk, as draw weights: per-thread
// sums of p and (with Resid) of max(0, p - q), the raw entries staying in
// registers for the crossing search.
template <class DT, bool VecOk, bool Resid>
__device__ __forceinline__ void chunk_weights(const ChainArgs &a, const DrawRow &w, int64_t c0, int n,
                                              int s0, uint4 (&rt)[Chunk2<DT>::kNQ],
                                              uint4 (&rd)[Chunk2<DT>::kNQ], float &lp, float &lr) {
    constexpr int VEC = DT::kVec, NQ = Chunk2<DT>::kNQ;
    load_chunk<DT, VecOk, Resid>(a, w, c0, n, s0, rt, rd);
    lp = 0.f;
    lr = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        float t[VEC], d[VEC];
        unpack<DT>(rt[q], t);
        if (Resid) unpack<DT>(rd[q], d);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const float p = weight_p(t[i], a.c, w);
            lp += p;
            if (Resid) lr += weight_r(p, d[i], a.c, w);
        }
        asm volatile("" : "+v"(lp), "+v"(lr));  // one slot at a time
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        asm volatile("" : "+v"(rt[q].x), "+v"(rt[q].y), "+v"(rt[q].z), "+v"(rt[q].w));
        if (Resid) asm volatile("" : "+v"(rd[q].x), "+v"(rd[q].y), "+v"(rd[q].z), "+v"(rd[q].w));
    }
}

// Wavefront 0: from the chunk masses of the sequence (lane i: chunk i), the
// total S, tau = u * S and the crossing chunk -- the first whose inclusive
// running mass exceeds tau (the inverse CDF, strict), else the last chunk
// with mass -- with the running mass before it.
__device__ __forceinline__ void crossing_chunk(float m, bool in, float us, float &S, float &tau,
                                               int &cstar, float &base) {
    const float incl = wave_incl_sum(m);
    S = wave_last(incl);
    tau = us * S;
    const float excl = wave_excl_from_incl(incl);
    const uint64_t cross = __ballot(in && incl > tau), pos = __ballot(in && m > 0.f);
    cstar = cross ? __ffsll(static_cast<unsigned long long>(cross)) - 1
                  : (pos ? 63 - __clzll(static_cast<long long>(pos)) : 0);
    base = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(excl), cstar));
}

// Workgroup (b, ch) of the draw after the resolve.
//
// After a rejection (Resid) it holds entries [ch*C2, ch*C2 + C2) of rows j in
// registers (kSeg contiguous entries per thread) and publishes the chunk's
// residual mass sum max(0, p_j - q_j) and target mass sum p_j.  Wavefront 0
// reads every chunk's masses of the sequence into its lanes (a sequence has
// at most 64 chunks), and every draw workgroup of the sequence computes the
// same S and the same crossing chunk.  An all-zero residual (reachable only
// through rounding) draws from p_j.
//
// For the bonus draw (j = K) the chunk masses of p_K follow from the bonus
// row's chunk statistics, z_c * 2^(ref_c - ref) / z, with no second read of
// the row; only the crossing chunk's workgroup loads its entries.
//
// In the crossing chunk's workgroup the first thread whose running mass
// passes u * S hands its entries to wavefront 0 through LDS, which finds the
// entry (one lane each) and writes the sequence's outputs.
template <class DT, bool VecOk, bool Resid>
__device__ __forceinline__ void draw_body(const ChainArgs &a, int b, int ch, int j, const DrawRow &w,
                                          bool ok, float us, int32_t my_tok, float *lds) {
    using CK = Chunk2<DT>;
    constexpr int C2 = CK::kElems, kSeg = CK::kSeg, NQ = CK::kNQ;
    static_assert(kSeg <= kWave, "one lane per entry of a thread's segment");
    static_assert(CK::kRawWords <= kDrawRawWords, "a thread's raw entries fit the LDS");
    static_assert(kMaxDrawChunks <= kWave, "one lane per chunk of a sequence");
    const int K = a.K, tid = threadIdx.x, lane = tid % kWave, nc = a.nchunk2;
    __shared__ float s_tau, s_base;
    __shared__ int s_cstar, s_resid, s_ok;

    const int64_t c0 = static_cast<int64_t>(ch) * C2;
    const int n = static_cast<int>(min(static_cast<int64_t>(C2), static_cast<int64_t>(a.V) - c0));
    const int s0 = tid * kSeg;
    uint4 rt[NQ], rd[NQ];
    float lp = 0.f, lr = 0.f, ex_r = 0.f, ex_p = 0.f, S = 0.f;
    if constexpr (Resid) {
        chunk_weights<DT, VecOk, true>(a, w, c0, n, s0, rt, rd, lp, lr);
        // Running sums inside the chunk and the chunk's masses, both kinds,
        // in one pass (published afterwards: a barrier after a device-scope
        // store would wait for it to complete).
        uint64_t *sums = a.sums + 2 * static_cast<int64_t>(b) * nc;
        float mr, mp;
        wg_excl_scan2(lr, lp, ex_r, ex_p, mr, mp);
        if (tid == 0) {
            publish_f32(&sums[2 * ch], a.tag, mr);
            publish_f32(&sums[2 * ch + 1], a.tag, mp);
        }
        if (tid < kWave) {
            const int i = min(lane, nc - 1);
            uint64_t vr, vp;
            bool fresh;
            const uint64_t t0 = wall_clock64();
            // The last chunk's workgroup is dispatched last: wait for its
            // word, then read all (repeating while any is missing).
            if (lane == 0) wait_word(&sums[2 * (nc - 1)], a.tag, t0);
            for (;;) {
                vr = fetch(&sums[2 * i]);
                vp = fetch(&sums[2 * i + 1]);
                fresh = __all(current(vr, a.tag) && current(vp, a.tag));
                if (fresh || wall_clock64() - t0 > kWaitTicks) break;
                __builtin_amdgcn_s_sleep(8);
            }
            const bool in = lane < nc;
            const float m_r = in ? word_f32(vr) : 0.f, m_p = in ? word_f32(vp) : 0.f;
            const bool resid = wave_last(wave_incl_sum(m_r)) > 0.f;
            float tau, base;
            int cstar;
            crossing_chunk(resid ? m_r : m_p, in, us, S, tau, cstar, base);
            if (lane == 0) {
                s_ok = fresh;
                s_cstar = cstar;
                s_base = base;
                s_tau = tau;
                s_resid = resid;
            }
        }
    } else {
        if (tid < kWave) {
            const bool in = lane < nc;
            const float *s_kref = lds + kDrawBonusAt, *s_kz = s_kref + kMaxDrawChunks;
            const int i = min(lane, nc - 1);
            const float m = in ? __fmul_rn(s_kz[i] * exp2_hw(s_kref[i] - w.rt), w.izt) : 0.f;
            float tau, base;
            int cstar;
            crossing_chunk(m, in, us, S, tau, cstar, base);
            if (lane == 0) {
                s_ok = 1;
                s_cstar = cstar;
                s_base = base;
                s_tau = tau;
                s_resid = 0;
            }
        }
    }
    __syncthreads();
    if (!(ok && s_ok)) {
        // A bounded wait ran out: the last chunk's workgroup marks the
        // sequence as failed.
        if (ch == nc - 1) {
            for (int k = tid; k <= K; k += kWG)
                a.out_tokens[static_cast<int64_t>(b) * (K + 1) + k] = -1;
            if (tid == 0) a.out_accepted[b] = -1;
        }
        return;
    }
    if (s_cstar != ch) return;
    if constexpr (!Resid) {
        // The bonus draw's crossing chunk: its entries and running sums now.
        chunk_weights<DT, VecOk, false>(a, w, c0, n, s0, rt, rd, lp, lr);
        float mr, mp;
        wg_excl_scan2(0.f, lp, ex_r, ex_p, mr, mp);
    }

    // The crossing chunk.  The first thread whose running mass passes tau
    // (else the last thread with mass) holds the drawn entry.
    const bool resid = Resid && s_resid;
    const float tau = s_tau;
    const float start = s_base + (resid ? ex_r : ex_p), l = resid ? lr : lp;
    int tf, tl;
    wg_min_max(l > 0.f && start + l > tau ? tid : INT32_MAX, l > 0.f ? tid : -1, tf, tl);
    const int ts = tf != INT32_MAX ? tf : max(tl, 0);
    uint32_t *s_raw = reinterpret_cast<uint32_t *>(lds + kDrawRawAt);
    float *s_start = lds + kDrawRawAt + 2 * kDrawRawWords;
    if (tid == ts) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            reinterpret_cast<uint4 *>(s_raw)[q] = rt[q];
            if (Resid) reinterpret_cast<uint4 *>(s_raw + kDrawRawWords)[q] = rd[q];
        }
        *s_start = start;
    }
    __syncthreads();
    if (tid >= kWave) return;
    // Lane e takes entry e of that thread's segment: the first entry (index
    // order) whose running mass exceeds tau; if rounding leaves none, the
    // last entry with weight.
    const int e = min(lane, kSeg - 1);
    float x = weight_p(raw_entry<DT>(s_raw, e), a.c, w);
    if (Resid && resid) x = weight_r(x, raw_entry<DT>(s_raw + kDrawRawWords, e), a.c, w);
    x = lane < kSeg ? x : 0.f;
    const float run = *s_start + wave_incl_sum(x);
    const uint64_t f = __ballot(x > 0.f && run > tau), nz = __ballot(x > 0.f);
    const int pick = f ? __ffsll(static_cast<unsigned long long>(f)) - 1
                       : (nz ? 63 - __clzll(static_cast<long long>(nz)) : 0);
    const int32_t token = static_cast<int32_t>(c0 + ts * kSeg + pick);

    // Emit x_0..x_{j-1}, then the drawn token, then -1 (lane k: position k).
    for (int k = lane; k <= K; k += kWave) {
        int32_t o = -1;
        if (k < j) o = my_tok;  // k < j <= K <= 64: k is this lane
        else if (k == j) o = token;
        a.out_tokens[static_cast<int64_t>(b) * (K + 1) + k] = o;
        if (a.out_diag) {
            float *dg = a.out_diag + 4 * (static_cast<int64_t>(b) * (K + 1) + k);
            if (k == K) dg[0] = dg[1] = dg[2] = 0.f;
            dg[3] = k == j ? S : 0.f;
        }
    }
    if (lane == 0) a.out_accepted[b] = j;
}

template <class DT, bool VecOk, bool Live>
__device__ __forceinline__ void draw_item(const ChainArgs &a, int b, int ch, float *lds) {
    const int K = a.K;
    // Drafted tokens for the emission (lane k: token k) and the draw's
    // uniform, loaded before the resolve.
    const int32_t *tk = K > 0 ? a.tokens + static_cast<int64_t>(b) * K
                              : reinterpret_cast<const int32_t *>(a.u_sample + b);
    const int32_t my_tok = tk[min(static_cast<int>(threadIdx.x % kWave), max(K - 1, 0))];
    const float us = a.u_sample[b];
    DrawRow w;
    bool ok;
    // One chunk per lane of a 16-lane group when a row has at most 16 (the
    // loads of up to four groups of 16 rows together), else four chunks per
    // lane and load batch.
    const int R = 2 * a.K + 1;
    const int j = a.nchunk > 16 ? resolve_local<DT, Live, 4, 1>(a, b, w, ok, ch == 0, lds)
                  : R <= 16     ? resolve_local<DT, Live, 1, 1>(a, b, w, ok, ch == 0, lds)
                  : R <= 32     ? resolve_local<DT, Live, 1, 2>(a, b, w, ok, ch == 0, lds)
                                : resolve_local<DT, Live, 1, 4>(a, b, w, ok, ch == 0, lds);
    if (w.resid) draw_body<DT, VecOk, true>(a, b, ch, j, w, ok, us, my_tok, lds);
    else draw_body<DT, VecOk, false>(a, b, ch, j, w, ok, us, my_tok, lds);
}

template <class DT, int U>
__global__ __launch_bounds__(kWG) void k_chain_stats(ChainArgs a) {
    if (a.tag_src) a.tag = *a.tag_src;  // a graph replay's tag
    // 32-bit index arithmetic (the grid is below 2^31 workgroups): a 64-bit
    // division is a long instruction sequence ahead of the first load.
    const uint32_t R = 2 * a.K + 1, S = R * a.nchunk;
    const uint32_t g = blockIdx.x, b = g / S, pos = g - b * S, r = pos / a.nchunk;
    stats_item<DT, U>(a, b, static_cast<int>(r), static_cast<int>(pos - r * a.nchunk));
}

template <class DT, bool VecOk>
__global__ __launch_bounds__(kWG) void k_chain_draw(ChainArgs a) {
    if (a.tag_src) a.tag = *a.tag_src;  // a graph replay's tag
    const uint32_t nc = a.nchunk2, g = blockIdx.x, b = g / nc;
    __shared__ __align__(16) float lds[kDrawLds];
    draw_item<DT, VecOk, false>(a, static_cast<int>(b), static_cast<int>(g - b * nc), lds);
}

// The whole chain verify in one launch.  Per sequence there are S = (2K+1) *
// nchunk statistics workgroups and D = nchunk2 draw workgroups.  The hardware
// dispatches workgroups in index order, and a draw workgroup waits only for
// statistics workgroups it needs and for the draw workgroups of its own
// sequence (dispatched together), so the order of the grid decides how draws
// overlap streaming.
//
// With lag < B: blocks of the statistics of sequence b + lag with the draws of
// b in one run among them, after a prologue of the first `lag` sequences'
// statistics and before an epilogue of the last `lag` sequences' draws.  A
// draw only waits for workgroups of lower index; with the lag at least the
// chip's resident window, the statistics it needs have usually finished
// before it starts.
//
// With lag = B: the statistics of every row but the bonus rows (target row K,
// read only by a draw with every draft accepted) come first, sequence by
// sequence, then the bonus rows, then every draw, so draws after a rejection
// can start while the bonus rows stream.  (Placing the draws ahead of the
// bonus rows measured slower.)
template <class DT, bool VecOk>
__global__ __launch_bounds__(kWG) void k_chain_fused(ChainArgs a) {
    if (a.tag_src) a.tag = *a.tag_src;  // a graph replay's tag
    __shared__ __align__(16) float lds[kDrawLds];
    const uint32_t nch = a.nchunk, S = (2 * a.K + 1) * nch, D = a.nchunk2, L = a.lag, B = a.B;
    const uint32_t g = blockIdx.x;
    // Decode the workgroup's item: a draw (b, chunk) or statistics (b, row, chunk).
    uint32_t b, r = 0, ch;
    bool draw;
    if (L == B) {
        const uint32_t Sn = S - nch, nNB = B * Sn, d0 = nNB + B * nch;
        draw = g >= d0;
        if (draw) {
            b = (g - d0) / D;
            ch = g - d0 - b * D;
        } else if (g < nNB) {
            b = g / Sn;
            const uint32_t p = g - b * Sn, rr = p / nch;
            r = rr < static_cast<uint32_t>(a.K) ? rr : rr + 1;
            ch = p - rr * nch;
        } else {
            const uint32_t h = g - nNB;
            b = h / nch;
            r = a.K;
            ch = h - b * nch;
        }
    } else {
        const uint32_t pro = L * S, steady = pro + (B - L) * (S + D);
        uint32_t s;
        if (g < pro) {
            b = g / S;
            s = g - b * S;
            draw = false;
        } else if (g < steady) {
            // Block k: the D draws of sequence k in one run at offset o among
            // the statistics of sequence L + k; o steps by 8 per block, so the
            // run's place in each XCD's share of the order rotates.
            const uint32_t h = g - pro, k = h / (S + D), p = h - k * (S + D);
            const uint32_t o = (8 * k) % (S + 1);
            draw = p >= o && p < o + D;
            b = draw ? k : L + k;
            s = draw ? p - o : (p < o ? p : p - D);
        } else {
            const uint32_t h = g - steady, k = h / D;
            b = B - L + k;
            s = h - k * D;
            draw = true;
        }
        if (draw) {
            ch = s;
        } else {
            r = s / nch;
            ch = s - r * nch;
        }
    }
    if (draw)
        draw_item<DT, VecOk, true>(a, static_cast<int>(b), static_cast<int>(ch), lds);
    else
        stats_item<DT, 4>(a, b, static_cast<int>(r), static_cast<int>(ch));
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

hipError_t launch_chain_fused(const ChainArgs &a, int dtype, hipStream_t s) {
    const int64_t per_seq = static_cast<int64_t>(2 * a.K + 1) * a.nchunk + a.nchunk2;
    const dim3 g(static_cast<uint32_t>(static_cast<int64_t>(a.B) * per_seq)), blk(kWG);
    if (dtype == 1) {
        if (a.V % Bf16::kVec == 0) k_chain_fused<Bf16, true><<<g, blk, 0, s>>>(a);
        else k_chain_fused<Bf16, false><<<g, blk, 0, s>>>(a);
    } else {
        if (a.V % F32::kVec == 0) k_chain_fused<F32, true><<<g, blk, 0, s>>>(a);
        else k_chain_fused<F32, false><<<g, blk, 0, s>>>(a);
    }
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
