// Chain verify at T > 0 on gfx950.
//
// Statistics items stream the logits of the step, each at most once.  One
// workgroup takes one 8 KB vocabulary chunk of one row (target rows 0..K and
// draft rows 0..K-1 of a sequence), folds it into softmax statistics (ref, z)
// and publishes them; in the position-major order a row whose position comes
// after its sequence's first rejection is skipped, and there one workgroup
// takes two or four adjacent chunks after reading its row's gate word.  This
// is the HBM-bound work that carries the bytes; no statistics workgroup
// waits for another.
//
// A resolver per sequence merges the statistics of the rows the accept tests
// read, evaluates the accept test of every drafted token (u < p(x)/q(x),
// French lesson "Décodage spéculatif et Eagle", section "La règle de
// l'exactitude"; forum post "Speculative Decoding: от идеи до SOTA", §3),
// finds the first rejection j and publishes a record: j and row j's
// normalisers.  After a rejection, draw items (one per 8 KB chunk of rows j)
// publish the chunk's mass of the residual max(0, p_j - q_j) (the residual of
// the same passages) and of p_j; the sequence's finisher finds the chunk
// whose running mass first exceeds u * S, reads it again and draws the token.
// When every draft is accepted, the sequence's bonus item draws from p_K,
// whose chunk masses follow from the bonus row's statistics.
//
// k_chain_fused runs every item in one grid (the one-call entry point);
// k_chain_stats and k_chain_draw run them as two kernels in stream order (the
// two-phase entry points).  Both give the same bits.
//
// Hand-over words are 64 bits: the call's tag above a 32-bit value, written
// with device-scope atomic stores and read with device-scope atomic loads; a
// reader checks the tag, so nothing left by an earlier call is taken for
// fresh, and waits (bounded in time) until the word is visible.  Tags are
// never 0, so a workspace zeroed once before first use needs no clearing.  An
// item only waits for workgroups of lower index (dispatched before it).
#include "device.hpp"
#include "handover.hpp"
#include "grid_order.hpp"
#include "plan.hpp"

namespace sv {
namespace {

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

// ------------------------------------------------------------ stats item

// Loads chunk ch of a row (element offset `trow * V` in `base`): thread t
// takes vectors t and t + 256 (one non-temporal 16-byte load each, both in
// flight before any use); returns the chunk's vector count.
template <class DT>
__device__ __forceinline__ int load_stat_chunk(const ChainArgs &a, const void *base, int64_t trow, int ch,
                                               uint4 (&raw)[kStatVecs]) {
    constexpr int VEC = DT::kVec;
    const int64_t e0 = static_cast<int64_t>(ch) * a.chunk;
    const int n = static_cast<int>(min(static_cast<int64_t>(a.chunk), static_cast<int64_t>(a.V) - e0));
    const uint4 *vp = static_cast<const uint4 *>(base) + (trow * a.V + e0) / VEC;
    const int nv = n / VEC, last = nv - 1, tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kStatVecs; ++u) raw[u] = load_nt(vp + min(tid + u * kWG, last));
    return nv;
}

// The softmax statistics of a loaded chunk, published as its partial: the
// vectors past the row's end (in its last chunk) read as -inf.
template <class DT>
__device__ __forceinline__ void reduce_stat_chunk(const ChainArgs &a, int64_t row, int ch,
                                                  uint4 (&raw)[kStatVecs], int nv) {
    constexpr int VEC = DT::kVec, U = kStatVecs, N = U * VEC;
    constexpr uint32_t kInf = NegInf<DT>::kBits;
    const int tid = threadIdx.x;
    if (nv < U * kWG) {  // the row's last chunk
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (tid + u * kWG > nv - 1) raw[u] = make_uint4(kInf, kInf, kInf, kInf);
    }
    float x[N];
#pragma unroll
    for (int u = 0; u < U; ++u) unpack<DT>(raw[u], x + u * VEC);
    float ref = -INFINITY, z = 0.f;
    mz_chunk_wg<N>(x, a.c, ref, z);
    if (tid == 0) {
        const uint32_t tag = a.tag_src ? *a.tag_src : a.tag;  // a graph replay's tag
        uint64_t *w = a.partial + 2 * (row * a.nchunk + ch);
        publish_f32(w, tag, ref);
        publish_f32(w + 1, tag, z);
    }
}

// Statistics item: softmax statistics (ref, z) of one chunk of row r of
// sequence b (r <= K: target row r; r > K: draft row r - K - 1), published as
// tagged words; chunk ch: a.chunk entries, 8 KB, two 16-byte vectors per
// thread.  With V a
// multiple of the vector width every chunk starts on a vector (the vectors
// past the end of a row's last chunk read as -inf); otherwise the entries are
// read one by one.  Loads are non-temporal: a logit is streamed once, and its
// second read by a draw comes from HBM either way.
template <class DT, bool VecOk>
__device__ __forceinline__ void stats_item(const ChainArgs &a, int64_t b, int r, int ch) {
    const int K = a.K, R = 2 * K + 1;
    const int64_t row = b * R + r;
    const void *base = r <= K ? a.target : a.draft;
    const int64_t trow = r <= K ? b * (K + 1) + r : b * K + (r - K - 1);
    if constexpr (VecOk) {
        uint4 raw[kStatVecs];
        const int nv = load_stat_chunk<DT>(a, base, trow, ch, raw);
        reduce_stat_chunk<DT>(a, row, ch, raw, nv);
    } else {
        constexpr int N = kStatVecs * DT::kVec;
        const int64_t e0 = static_cast<int64_t>(ch) * a.chunk;
        const int n = static_cast<int>(min(static_cast<int64_t>(a.chunk), static_cast<int64_t>(a.V) - e0));
        const int64_t g0 = trow * a.V + e0;
        float x[N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int e = threadIdx.x + i * kWG;
            const float v = load_one<DT>(base, g0 + min(e, n - 1));
            x[i] = e < n ? v : -INFINITY;
        }
        float ref = -INFINITY, z = 0.f;
        mz_chunk_wg<N>(x, a.c, ref, z);
        if (threadIdx.x == 0) {
            const uint32_t tag = a.tag_src ? *a.tag_src : a.tag;  // a graph replay's tag
            uint64_t *w = a.partial + 2 * (row * a.nchunk + ch);
            publish_f32(w, tag, ref);
            publish_f32(w + 1, tag, z);
        }
    }
}

// Chunks ch .. ch + G - 1 of row r (those the row has) in one workgroup, all
// their loads in flight together, each chunk reduced and published exactly
// as a statistics item does it.  V a multiple of the vector width.
template <class DT, int G>
__device__ __forceinline__ void stats_group(const ChainArgs &a, int64_t b, int r, int ch) {
    const int K = a.K, R = 2 * K + 1;
    const int64_t row = b * R + r;
    const void *base = r <= K ? a.target : a.draft;
    const int64_t trow = r <= K ? b * (K + 1) + r : b * K + (r - K - 1);
    const int m = min(G, a.nchunk - ch);
    uint4 raw[G][kStatVecs];
    int nv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) nv[g] = g < m ? load_stat_chunk<DT>(a, base, trow, ch + g, raw[g]) : 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (g >= m) return;
        if (g > 0) __syncthreads();  // the reduction's LDS words are reused
        reduce_stat_chunk<DT>(a, row, ch + g, raw[g], nv[g]);
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

// Resolve of sequence b (one workgroup per sequence).  Each group of 16 lanes
// merges the chunk statistics of one of the 2K rows the accept tests read
// (target rows 0..K-1, draft rows 0..K-1; lane i folds chunks i, i + 16, ...
// in order, then a fixed DPP tree, in double precision), every wavefront
// evaluates the accept test of every drafted token (u < P/Q, strict; Q = 0
// accepts iff P > 0) and takes j, the first rejected position (K if none), by
// ballot.  Row j's statistics land in `w` (row K's are the bonus item's).
// Without Live the statistics come from a kernel ordered before this one by
// the stream and are read once; with Live the statistics workgroups may still
// be running, so the words are read with device-scope loads, and while one is
// missing one lane of each wavefront that saw it waits for it (bounded) and
// everything is read again.  `ok` is false if a word was not written in time.
// Statistics words carry `ptag`.  The workgroup also writes p_k(x_k),
// q_k(x_k) and their ratio to out_diag.
template <class DT, bool Live, int Fold, int kPasses>
__device__ __forceinline__ int resolve_local(const ChainArgs &a, int b, uint32_t ptag, DrawRow &w,
                                             bool &ok, float *lds) {
    // The loads of kPasses row groups (16 rows each) go out together.
    constexpr int kGroup = 16, kGroups = kWG / kGroup;
    float *s_ref = lds, *s_z = s_ref + (2 * kMaxK + 1);
    __shared__ int s_stale[2][kWaves + 1];
    const int K = a.K, V = a.V, R = 2 * K + 1, R2 = 2 * K, nch = a.nchunk;
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
    // The statistics items of a sequence are dispatched in row order, the
    // draft row K - 1 last: one lane waits for that row's last word before
    // the whole read.
    if (Live && K > 0 && tid == 0)
        wait_word(part + 2 * ((2 * K) * nch + nch - 1) + 1, ptag, t0);
    float P = 0.f, Q = 0.f;
    int j = K;
    ok = true;
    for (int it = 0; K > 0; ++it) {
        const uint64_t *miss = nullptr;  // the first missing word this lane found
        for (int r0 = 0; r0 < R2; r0 += kGroups * kPasses) {
            float ref[kPasses];
            double z[kPasses];
#pragma unroll
            for (int q = 0; q < kPasses; ++q) {
                ref[q] = -INFINITY;
                z[q] = 0.0;
            }
            for (int i0 = 0; i0 < nch; i0 += kGroup * Fold) {
                uint64_t pr[kPasses][Fold], pz[kPasses][Fold];
#pragma unroll
                for (int q = 0; q < kPasses; ++q) {
                    const int rs = min(r0 + grp + kGroups * q, R2 - 1), rr = rs < K ? rs : rs + 1;
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
                    const int rs = r0 + grp + kGroups * q, rsc = min(rs, R2 - 1), rr = rsc < K ? rsc : rsc + 1;
#pragma unroll
                    for (int f = 0; f < Fold; ++f) {
                        const int i = i0 + gl + kGroup * f;
                        const bool in = rs < R2 && i < nch;
                        const bool cr = current(pr[q][f], ptag), cz = current(pz[q][f], ptag);
                        const float fr = in ? word_f32(pr[q][f]) : -INFINITY;
                        const float fz = in ? word_f32(pz[q][f]) : 0.f;
                        if (in && !(cr && cz) && !miss) miss = part + 2 * (rr * nch + i) + (cr ? 1 : 0);
                        mz_merge_d(ref[q], z[q], fr, static_cast<double>(fz));
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < kPasses; ++q) {
                mz_row_merge_d(ref[q], z[q]);
                const int rs = r0 + grp + kGroups * q;
                if (rs < R2 && gl == kGroup - 1) {
                    const int rr = rs < K ? rs : rs + 1;
                    s_ref[rr] = ref[q];
                    s_z[rr] = static_cast<float>(z[q]);
                }
            }
        }
        const uint64_t st = __ballot(miss != nullptr);
        // Double-buffered by iteration: a wavefront may start the next
        // iteration while another still reads this one's flags.
        if (lane == 0) s_stale[it & 1][tid / kWave] = st ? 1 : 0;
        if (tid == 0) s_stale[it & 1][kWaves] = !Live || wall_clock64() - t0 > kWaitTicks;
        __syncthreads();
        int any = 0;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) any |= s_stale[it & 1][k];
        if (!any) {
            bool reject = false;
            if (lane < K) {
                P = exp2_hw(fmaf(lt, a.c, -s_ref[lane])) / s_z[lane];
                Q = exp2_hw(fmaf(ld, a.c, -s_ref[K + 1 + lane])) / s_z[K + 1 + lane];
                reject = !(Q > 0.f ? (u < P / Q) : (P > 0.f));
            }
            const uint64_t m = __ballot(reject);
            j = m ? (__ffsll(static_cast<unsigned long long>(m)) - 1) : K;
            break;
        }
        if (s_stale[it & 1][kWaves]) {
            ok = false;
            break;
        }
        // One lane of each wavefront that missed a word waits for it.
        if (st && lane == __ffsll(static_cast<unsigned long long>(st)) - 1) wait_word(miss, ptag, t0);
    }
    if (ok && tid < K && a.out_diag) {
        float *dg = a.out_diag + 4 * (static_cast<int64_t>(b) * (K + 1) + lane);
        dg[0] = P;
        dg[1] = Q;
        dg[2] = Q > 0.f ? P / Q : (P > 0.f ? INFINITY : 0.f);
    }
    w.resid = j < K;
    if (w.resid) {
        w.rt = s_ref[j];
        w.izt = 1.f / s_z[j];
        w.rd = s_ref[K + 1 + j];
        w.izd = 1.f / s_z[K + 1 + j];
    }
    return j;
}

// Entries per chunk of the residual / bonus pass: 8 KB of one row, in
// rounds of one 16-byte vector per thread: vector q * kWG + t of the chunk is
// thread t's q-th, so every load instruction of a wavefront reads 1 KB of
// consecutive bytes, and index order is round by round, thread by thread.
template <class DT>
struct Chunk2 {
    static constexpr int kElems = kDrawChunkBytes / (16 / DT::kVec);
    static constexpr int kNQ = kElems / (kWG * DT::kVec);  // rounds: 16-byte vectors per thread and row
};

// This thread's vectors of chunk c0 of row j (target, and draft when Resid),
// raw; entries past the row's end read as -inf.  With V a multiple of the
// vector width all loads are issued before any is used; otherwise entries are
// read one by one into the same layout.
template <class DT, bool VecOk, bool Resid>
__device__ __forceinline__ void load_chunk(const ChainArgs &a, const DrawRow &w, int64_t c0, int n,
                                           uint4 (&rt)[Chunk2<DT>::kNQ],
                                           uint4 (&rd)[Chunk2<DT>::kNQ]) {
    constexpr int VEC = DT::kVec, NQ = Chunk2<DT>::kNQ;
    constexpr uint32_t kInf = NegInf<DT>::kBits;
    const int tid = threadIdx.x;
    if constexpr (VecOk) {
        const uint4 *tp = static_cast<const uint4 *>(a.target) + (w.trow + c0) / VEC;
        const uint4 *dp = static_cast<const uint4 *>(a.draft) + (w.drow + c0) / VEC;
        const int last = n / VEC - 1;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int o = min(tid + q * kWG, last);
            rt[q] = tp[o];
            if (Resid) rd[q] = dp[o];
        }
        // The row's last chunk: whole vectors past its end read as -inf
        // (selects, not branches, so the vectors stay in registers).
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const bool in = tid + q * kWG <= last;
            rt[q].x = in ? rt[q].x : kInf;
            rt[q].y = in ? rt[q].y : kInf;
            rt[q].z = in ? rt[q].z : kInf;
            rt[q].w = in ? rt[q].w : kInf;
            if (Resid) {
                rd[q].x = in ? rd[q].x : kInf;
                rd[q].y = in ? rd[q].y : kInf;
                rd[q].z = in ? rd[q].z : kInf;
                rd[q].w = in ? rd[q].w : kInf;
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
                    const int e = (tid + q * kWG) * VEC + h * (VEC / 4) + e2, ec = min(e, n - 1);
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

// Entry e of one raw 16-byte vector (as 32-bit words), widened.
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

// Row j's entries of this workgroup's chunk, as draw weights: per-thread,
// per-round sums of p and (with Resid) of max(0, p - q), the raw entries
// staying in registers for the crossing search.
template <class DT, bool VecOk, bool Resid>
__device__ __forceinline__ void chunk_weights(const ChainArgs &a, const DrawRow &w, int64_t c0, int n,
                                              uint4 (&rt)[Chunk2<DT>::kNQ],
                                              uint4 (&rd)[Chunk2<DT>::kNQ],
                                              float (&lp)[Chunk2<DT>::kNQ],
                                              float (&lr)[Chunk2<DT>::kNQ]) {
    constexpr int VEC = DT::kVec, NQ = Chunk2<DT>::kNQ;
    load_chunk<DT, VecOk, Resid>(a, w, c0, n, rt, rd);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        float t[VEC], d[VEC];
        unpack<DT>(rt[q], t);
        if (Resid) unpack<DT>(rd[q], d);
        float sp = 0.f, sr = 0.f;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const float p = weight_p(t[i], a.c, w);
            sp += p;
            if (Resid) sr += weight_r(p, d[i], a.c, w);
        }
        lp[q] = sp;
        lr[q] = sr;
    }
    // The raw entries stay in registers for the crossing search.
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        asm volatile("" : "+v"(rt[q].x), "+v"(rt[q].y), "+v"(rt[q].z), "+v"(rt[q].w));
        if (Resid) asm volatile("" : "+v"(rd[q].x), "+v"(rd[q].y), "+v"(rd[q].z), "+v"(rd[q].w));
    }
}

// Exclusive prefix sums in index order (round by round, thread by thread) of
// two kinds of per-thread, per-round masses, and the chunk's two totals; every
// thread gets the totals.  A fixed order, so the draw item that publishes a
// chunk's masses and the workgroup that searches the chunk agree bit for bit.
template <int NQ>
__device__ __forceinline__ void round_scan2(const float (&x)[NQ], const float (&y)[NQ],
                                            float (&ex)[NQ], float (&ey)[NQ], float &tx, float &ty) {
    __shared__ float s_t[2][NQ][kWaves];
    float ix[NQ], iy[NQ];
    const int w = threadIdx.x / kWave;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        ix[q] = wave_incl_sum(x[q]);
        iy[q] = wave_incl_sum(y[q]);
        if (threadIdx.x % kWave == kWave - 1) {
            s_t[0][q][w] = ix[q];
            s_t[1][q][w] = iy[q];
        }
    }
    __syncthreads();
    tx = 0.f;
    ty = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        float bx = 0.f, by = 0.f;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
            if (k == w) {
                bx = tx;
                by = ty;
            }
            tx += s_t[0][q][k];
            ty += s_t[1][q][k];
        }
        ex[q] = bx + wave_excl_from_incl(ix[q]);
        ey[q] = by + wave_excl_from_incl(iy[q]);
    }
}

// Wavefront 0: from the chunk masses of the sequence (lane i: chunks 2i and
// 2i + 1, m0 and m1, zero past the last chunk), the total S, tau = u * S and
// the crossing chunk -- the first whose inclusive running mass exceeds tau
// (the inverse CDF, strict), else the last chunk with mass -- with the
// running mass before it.
__device__ __forceinline__ void crossing_chunk(float m0, float m1, float us, float &S, float &tau,
                                               int &cstar, float &base) {
    const float incl = wave_incl_sum(m0 + m1);
    S = wave_last(incl);
    tau = us * S;
    const float excl = wave_excl_from_incl(incl);
    const uint64_t cross = __ballot(incl > tau), pos = __ballot(m0 > 0.f || m1 > 0.f);
    const int l = cross ? __ffsll(static_cast<unsigned long long>(cross)) - 1
                        : (pos ? 63 - __clzll(static_cast<long long>(pos)) : 0);
    const float e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(excl), l));
    const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m0), l));
    const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m1), l));
    // The pair's first chunk crosses if its own running mass passes tau;
    // without a crossing, the pair's last chunk with mass is taken.
    const bool second = cross ? !(e + a0 > tau) : a1 > 0.f;
    cstar = 2 * l + (second ? 1 : 0);
    base = second ? e + a0 : e;
}

// A sequence whose bounded wait ran out, or whose statistics were not left
// for this call: its outputs read -1 and the workspace's failure count grows.
__device__ __forceinline__ void fail_sequence(const ChainArgs &a, int b) {
    const int K = a.K;
    for (int k = threadIdx.x; k <= K; k += kWG)
        a.out_tokens[static_cast<int64_t>(b) * (K + 1) + k] = -1;
    if (threadIdx.x == 0) {
        a.out_accepted[b] = -1;
        __hip_atomic_fetch_add(a.hdr + kHdrFailures, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The search inside the crossing chunk (entries [c0, c0 + C2) of row j) and
// the emission.  The first vector (index order) whose running mass passes tau
// (else the last vector with mass) is handed by its thread to wavefront 0
// through LDS; lane e takes entry e of it, and the first entry whose running
// mass exceeds tau (else the last with weight) is the drawn token.  Wavefront
// 0 writes x_0..x_{j-1}, the drawn token, then -1.  `start[q]` and `l[q]` are
// the running mass before this thread's vector of round q and its mass.
template <class DT, bool Resid>
__device__ __forceinline__ void search_emit(const ChainArgs &a, int b, int64_t c0, int j,
                                            const DrawRow &w, bool resid, float tau,
                                            const float (&start)[Chunk2<DT>::kNQ],
                                            const float (&l)[Chunk2<DT>::kNQ],
                                            const uint4 (&rt)[Chunk2<DT>::kNQ],
                                            const uint4 (&rd)[Chunk2<DT>::kNQ], float S,
                                            int32_t my_tok, float *lds) {
    constexpr int VEC = DT::kVec, NQ = Chunk2<DT>::kNQ;
    static_assert(VEC <= kWave, "one lane per entry of a vector");
    const int K = a.K, tid = threadIdx.x, lane = tid % kWave;
    int cand = INT32_MAX, last = -1;
#pragma unroll
    for (int q = NQ - 1; q >= 0; --q) {
        if (l[q] > 0.f && start[q] + l[q] > tau) cand = q * kWG + tid;
        if (l[q] > 0.f && last < 0) last = q * kWG + tid;
    }
    int vf, vl;
    wg_min_max(cand, last, vf, vl);
    const int vs = vf != INT32_MAX ? vf : max(vl, 0);  // the vector searched, index in the chunk
    uint32_t *s_raw = reinterpret_cast<uint32_t *>(lds + kDrawRawAt);
    float *s_start = lds + kDrawRawAt + 8;
    // The owner of vector vs stores its round vs / kWG: one store per round,
    // under a uniform condition, so no register array is indexed at run time.
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if (vs / kWG == q && tid == vs % kWG) {
            reinterpret_cast<uint4 *>(s_raw)[0] = rt[q];
            if (Resid) reinterpret_cast<uint4 *>(s_raw)[1] = rd[q];
            *s_start = start[q];
        }
    }
    __syncthreads();
    if (tid >= kWave) return;
    const int e = min(lane, VEC - 1);
    float x = weight_p(raw_entry<DT>(s_raw, e), a.c, w);
    if (Resid && resid) x = weight_r(x, raw_entry<DT>(s_raw + 4, e), a.c, w);
    x = lane < VEC ? x : 0.f;
    const float run = *s_start + wave_incl_sum(x);
    const uint64_t f = __ballot(x > 0.f && run > tau), nz = __ballot(x > 0.f);
    const int pick = f ? __ffsll(static_cast<unsigned long long>(f)) - 1
                       : (nz ? 63 - __clzll(static_cast<long long>(nz)) : 0);
    const int32_t token = static_cast<int32_t>(c0 + static_cast<int64_t>(vs) * VEC + pick);
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

// The tags of an item: `tag` for the words this launch's workgroups hand each
// other, `ptag` for the statistics words (the phase word's tag in the
// two-phase form, else the call's own).
__device__ __forceinline__ void item_tags(const ChainArgs &a, uint32_t &ptag, uint32_t &tag) {
    tag = a.tag_src ? *a.tag_src : a.tag;
    ptag = a.sample_phase ? __hip_atomic_load(a.hdr + kHdrPhaseTag, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT)
                          : tag;
}

// Resolver item of sequence b: the accept tests and j, published as the
// sequence's record -- j, then row j's (ref, 1/z) of the target and the draft
// -- for its draw items and bonus item.  A failed resolve publishes j = -1.
template <class DT, bool Live>
__device__ __forceinline__ void resolver_item(const ChainArgs &a, int b, float *lds) {
    uint32_t ptag, tag;
    item_tags(a, ptag, tag);
    DrawRow w;
    bool ok = false;
    int j = -1;
    if (ptag != 0) {  // else the two-phase form without statistics for this call
        const int R = 2 * a.K + 1;
        j = a.nchunk > 16 ? resolve_local<DT, Live, 4, 1>(a, b, ptag, w, ok, lds)
            : R <= 16     ? resolve_local<DT, Live, 1, 1>(a, b, ptag, w, ok, lds)
            : R <= 32     ? resolve_local<DT, Live, 1, 2>(a, b, ptag, w, ok, lds)
                          : resolve_local<DT, Live, 1, 4>(a, b, ptag, w, ok, lds);
    }
    if (!ok) {
        fail_sequence(a, b);
        j = -1;
    }
    if (threadIdx.x == 0) {
        uint64_t *rec = a.rec + kRecWords * static_cast<int64_t>(b);
        const bool r = ok && j < a.K;
        publish_f32(rec + 1, tag, r ? w.rt : 0.f);
        publish_f32(rec + 2, tag, r ? w.izt : 0.f);
        publish_f32(rec + 3, tag, r ? w.rd : 0.f);
        publish_f32(rec + 4, tag, r ? w.izd : 0.f);
        publish(rec, tag, static_cast<uint32_t>(j));
    }
}

// ------------------------------------------------------------ position-major form

// Statistics of target row k and draft row k of sequence b, merged exactly as
// resolve_local merges a row (lane i of a group of 16 folds chunks i, i + 16,
// ... in order in double precision, then the same DPP tree), so P_k and Q_k
// come out bit for bit as the sequence resolver's.  Group 0 takes the target
// row, group 1 the draft row; wavefront 0 reads until every word carries
// `ptag` (bounded).  Returns false if a word did not come in time.
__device__ __forceinline__ bool pair_stats(const ChainArgs &a, int b, int k, uint32_t ptag, float &rt,
                                           float &zt, float &rd, float &zd) {
    constexpr int kGroup = 16;
    __shared__ float s_ref[2], s_z[2];
    __shared__ int s_ok;
    const int tid = threadIdx.x, K = a.K, nch = a.nchunk;
    if (tid < kWave) {
        const int grp = tid / kGroup, gl = tid % kGroup;
        const int row = grp == 0 ? k : K + 1 + k;
        const uint64_t *part = a.partial + 2 * ((static_cast<int64_t>(b) * (2 * K + 1) + row) * nch);
        const uint64_t t0 = wall_clock64();
        float ref;
        double z;
        bool fresh;
        for (;;) {
            ref = -INFINITY;
            z = 0.0;
            bool mine = true;
            if (grp < 2) {
                for (int i = gl; i < nch; i += kGroup) {
                    const uint64_t pr = fetch(part + 2 * i), pz = fetch(part + 2 * i + 1);
                    mine = mine && current(pr, ptag) && current(pz, ptag);
                    mz_merge_d(ref, z, word_f32(pr), static_cast<double>(word_f32(pz)));
                }
            }
            fresh = __all(mine);
            if (fresh || wall_clock64() - t0 > kWaitTicks) break;
            __builtin_amdgcn_s_sleep(2);
        }
        mz_row_merge_d(ref, z);
        if (grp < 2 && gl == kGroup - 1) {
            s_ref[grp] = ref;
            s_z[grp] = static_cast<float>(z);
        }
        if (tid == 0) s_ok = fresh;
    }
    __syncthreads();
    rt = s_ref[0];
    zt = s_z[0];
    rd = s_ref[1];
    zd = s_z[1];
    return s_ok != 0;
}

// Word offset of the gate line of (sequence b, position k).
__device__ __forceinline__ int64_t gate_line(const ChainArgs &a, int b, int k) {
    return (static_cast<int64_t>(b) * a.K + k) * kGateLineWords;
}

// The accept tests of sequence b ended at position k (a rejection or a
// failure): marks the gate lines of positions k+1..K-1, whose rows are then
// not needed.  Only the position-major orders, which skip rows, mark (a
// compile-time choice: reading a flag for it made the compiler load the flag
// at every workgroup's entry, one memory round trip before any load).
template <bool Gate>
__device__ __forceinline__ void mark_rows_not_needed(const ChainArgs &a, int b, int k, uint32_t tag) {
    if constexpr (!Gate) return;
    uint64_t *g = a.gate + gate_line(a, b, 0);
    for (int i = k + 1; i < a.K; ++i) publish(g + i * kGateLineWords, tag, 1u);
}

// Publishes sequence b's record: j, then row j's (ref, 1/z) of the target and
// the draft (zeros unless 0 <= j < K).
__device__ __forceinline__ void publish_record(const ChainArgs &a, int b, uint32_t tag, int j, float rt,
                                               float izt, float rd, float izd) {
    uint64_t *rec = a.rec + kRecWords * static_cast<int64_t>(b);
    const bool r = j >= 0 && j < a.K;
    publish_f32(rec + 1, tag, r ? rt : 0.f);
    publish_f32(rec + 2, tag, r ? izt : 0.f);
    publish_f32(rec + 3, tag, r ? rd : 0.f);
    publish_f32(rec + 4, tag, r ? izd : 0.f);
    publish(rec, tag, static_cast<uint32_t>(j));
}

// Pair resolver of position k of sequence b (position-major form).  It waits
// (bounded) for the outcomes of positions 0..k-1 of the sequence; if one of
// them ended the accept tests it records a skip and stops.  Otherwise it
// merges the statistics of target row k and draft row k, takes the accept
// test u < P/Q (strict; Q = 0 accepts iff P > 0) as the sequence resolver
// does, and publishes the outcome.  The first rejecting position publishes
// the sequence's record (j = k), and so does the last position when every
// draft is accepted (j = K).  A word that does not come in time fails the
// sequence (record j = -1).
template <class DT, bool Gate>
__device__ __forceinline__ void pair_resolver_item(const ChainArgs &a, int b, int k) {
    __shared__ int s_prev;
    const int K = a.K, V = a.V, tid = threadIdx.x, lane = tid % kWave;
    const uint32_t tag = a.tag_src ? *a.tag_src : a.tag;
    uint64_t *pairs = a.pairs + static_cast<int64_t>(b) * K;
    // The drafted token's logits and the uniform, issued before anything waits.
    float lt = 0.f, ld = 0.f, u = 0.f;
    if (tid == 0) {
        const int x = min(max(a.tokens[static_cast<int64_t>(b) * K + k], 0), V - 1);
        lt = load_one<DT>(a.target, (static_cast<int64_t>(b) * (K + 1) + k) * V + x);
        ld = load_one<DT>(a.draft, (static_cast<int64_t>(b) * K + k) * V + x);
        u = a.u_accept[static_cast<int64_t>(b) * K + k];
    }
    if (tid < kWave) {
        static_assert(kMaxK <= kWave, "one earlier position per lane");
        const uint64_t t0 = wall_clock64();
        uint64_t v;
        bool fresh;
        for (;;) {
            v = lane < k ? fetch(pairs + lane) : tagged(tag, kPairAccept);
            fresh = __all(current(v, tag));
            if (fresh || wall_clock64() - t0 > kWaitTicks) break;
            __builtin_amdgcn_s_sleep(2);
        }
        const bool stop = __any(static_cast<uint32_t>(v) != kPairAccept);
        if (lane == 0) s_prev = !fresh ? 2 : (stop ? 1 : 0);
    }
    __syncthreads();
    if (s_prev != 0) {
        if (s_prev == 2) fail_sequence(a, b);
        if (tid == 0) {
            if (s_prev == 2) {
                publish_record(a, b, tag, -1, 0.f, 0.f, 0.f, 0.f);
                mark_rows_not_needed<Gate>(a, b, k, tag);
            }
            publish(pairs + k, tag, s_prev == 2 ? kPairFail : kPairSkip);
        }
        return;
    }
    float rt, zt, rd, zd;
    if (!pair_stats(a, b, k, tag, rt, zt, rd, zd)) {
        fail_sequence(a, b);
        if (tid == 0) {
            publish_record(a, b, tag, -1, 0.f, 0.f, 0.f, 0.f);
            mark_rows_not_needed<Gate>(a, b, k, tag);
            publish(pairs + k, tag, kPairFail);
        }
        return;
    }
    if (tid == 0) {
        const float P = exp2_hw(fmaf(lt, a.c, -rt)) / zt;
        const float Q = exp2_hw(fmaf(ld, a.c, -rd)) / zd;
        const bool reject = !(Q > 0.f ? (u < P / Q) : (P > 0.f));
        if (a.out_diag) {
            float *dg = a.out_diag + 4 * (static_cast<int64_t>(b) * (K + 1) + k);
            dg[0] = P;
            dg[1] = Q;
            dg[2] = Q > 0.f ? P / Q : (P > 0.f ? INFINITY : 0.f);
        }
        if (reject) {
            mark_rows_not_needed<Gate>(a, b, k, tag);
            publish_record(a, b, tag, k, rt, 1.f / zt, rd, 1.f / zd);
        } else if (k == K - 1) {
            publish_record(a, b, tag, K, 0.f, 0.f, 0.f, 0.f);
        }
        publish(pairs + k, tag, reject ? kPairReject : kPairAccept);
    }
}

// Whether a statistics item of position k of sequence b may skip its
// chunk: an outcome already published for a position below k ended the
// sequence's accept tests, and so marked the gate line of (b, k).  Each
// (sequence, position) has a line of its own, read only by that position's
// items: a line an XCD's L2 holds from a read made before the mark was
// written stays stale there, and would otherwise hide the marks of later
// positions too.  Uniform over the workgroup (thread 0 reads, LDS shares).
__device__ __forceinline__ bool rows_not_needed(const ChainArgs &a, int b, int k) {
    __shared__ int s_skip;
    if (threadIdx.x == 0) {
        const uint32_t tag = a.tag_src ? *a.tag_src : a.tag;
        s_skip = current(plain_word(a.gate + gate_line(a, b, k)), tag);
    }
    __syncthreads();
    return s_skip != 0;
}

// Whether a bonus-row statistics item of sequence b may skip its chunk: the
// sequence's record, already published, says a draft was rejected (or the
// resolve failed).  Uniform over the workgroup.
__device__ __forceinline__ bool bonus_not_needed(const ChainArgs &a, int b) {
    __shared__ int s_skip;
    if (threadIdx.x == 0) {
        const uint32_t tag = a.tag_src ? *a.tag_src : a.tag;
        const uint64_t v = plain_word(a.rec + kRecWords * static_cast<int64_t>(b));
        s_skip = current(v, tag) && static_cast<int32_t>(static_cast<uint32_t>(v)) != a.K;
    }
    __syncthreads();
    return s_skip != 0;
}

// Wavefront 0 waits (bounded) until every word of sequence b's record
// carries `tag`, and shares it through LDS.  Returns false if it did not in
// time; else j (-1 for a failed resolve) and row j's statistics.
__device__ __forceinline__ bool read_record(const ChainArgs &a, int b, uint32_t tag, int &j,
                                            DrawRow &w) {
    __shared__ uint32_t s_rec[kRecWords + 1];
    const int lane = threadIdx.x % kWave;
    if (threadIdx.x < kWave) {
        const uint64_t *rec = a.rec + kRecWords * static_cast<int64_t>(b);
        const uint64_t t0 = wall_clock64();
        uint64_t v;
        bool fresh;
        for (;;) {
            v = lane < 5 ? fetch(rec + lane) : tagged(tag, 0);
            fresh = __all(current(v, tag));
            if (fresh || wall_clock64() - t0 > kWaitTicks) break;
            __builtin_amdgcn_s_sleep(8);
        }
        if (lane < 5) s_rec[lane] = static_cast<uint32_t>(v);
        if (lane == 0) s_rec[kRecWords] = fresh;
    }
    __syncthreads();
    j = static_cast<int32_t>(s_rec[0]);
    w.rt = __uint_as_float(s_rec[1]);
    w.izt = __uint_as_float(s_rec[2]);
    w.rd = __uint_as_float(s_rec[3]);
    w.izd = __uint_as_float(s_rec[4]);
    return s_rec[kRecWords] != 0;
}

// Draw item (b, ch) after a rejection at j < K: the masses of entries
// [ch*C2, ch*C2 + C2) of rows j -- the residual max(0, p_j - q_j) and the
// target p_j -- summed in the order the finisher's scan of the same chunk
// uses, so the two agree bit for bit.  It waits for nothing but the record
// and leaves the draw to the sequence's finisher, unless the row is a single
// chunk: then it draws itself.
template <class DT, bool VecOk>
__device__ __forceinline__ void draw_item(const ChainArgs &a, int b, int ch, float *lds) {
    using CK = Chunk2<DT>;
    constexpr int C2 = CK::kElems, NQ = CK::kNQ;
    const int K = a.K, tid = threadIdx.x;
    uint32_t ptag, tag;
    item_tags(a, ptag, tag);
    int j;
    DrawRow w;
    if (!read_record(a, b, tag, j, w) || j < 0 || j >= K) return;  // the finisher reports failures
    w.resid = true;
    w.trow = (static_cast<int64_t>(b) * (K + 1) + j) * a.V;
    w.drow = (static_cast<int64_t>(b) * K + j) * a.V;
    const int64_t c0 = static_cast<int64_t>(ch) * C2;
    const int n = static_cast<int>(min(static_cast<int64_t>(C2), static_cast<int64_t>(a.V) - c0));
    uint4 rt[NQ], rd[NQ];
    float lp[NQ], lr[NQ], ex_r[NQ], ex_p[NQ], mr, mp;
    chunk_weights<DT, VecOk, true>(a, w, c0, n, rt, rd, lp, lr);
    round_scan2<NQ>(lr, lp, ex_r, ex_p, mr, mp);
    if (a.nchunk2 == 1) {
        // The row is one chunk and this workgroup holds all of it: it draws
        // here, through the crossing and search a finisher would run on the
        // same masses (so the same bits), with no hand-over and no reload.
        __shared__ float s_tau1, s_base1, s_S1;
        __shared__ int s_resid1;
        const int lane = tid % kWave;
        const int32_t my_tok = a.tokens[static_cast<int64_t>(b) * K + min(lane, K - 1)];
        if (tid < kWave) {
            const float r0 = lane == 0 ? mr : 0.f, p0 = lane == 0 ? mp : 0.f;
            const bool resid = wave_last(wave_incl_sum(r0)) > 0.f;
            float S, tau, base;
            int cstar;
            crossing_chunk(resid ? r0 : p0, 0.f, a.u_sample[b], S, tau, cstar, base);
            if (lane == 0) {
                s_tau1 = tau;
                s_base1 = base;
                s_S1 = S;
                s_resid1 = resid;
            }
        }
        __syncthreads();
        const bool resid = s_resid1;
        float start[NQ], l[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            start[q] = s_base1 + (resid ? ex_r[q] : ex_p[q]);
            l[q] = resid ? lr[q] : lp[q];
        }
        search_emit<DT, true>(a, b, c0, j, w, resid, s_tau1, start, l, rt, rd, s_S1, my_tok, lds);
        return;
    }
    if (tid == 0) {
        uint64_t *sums = a.sums + 2 * (static_cast<int64_t>(b) * a.nchunk2 + ch);
        publish_f32(sums, tag, mr);
        publish_f32(sums + 1, tag, mp);
    }
}

// Finisher of sequence b after a rejection at j < K.  Wavefront 0 waits
// (bounded) until every chunk's masses carry the call's tag (lane i: chunk i;
// a sequence has at most 64 chunks), takes the total S of the residual (of
// p_j if the residual is all zero, reachable only through rounding), tau = u
// * S and the crossing chunk; the workgroup then loads that chunk of rows j
// again and searches it.
template <class DT, bool VecOk>
__device__ __forceinline__ void finisher_item(const ChainArgs &a, int b, float *lds) {
    using CK = Chunk2<DT>;
    constexpr int C2 = CK::kElems, NQ = CK::kNQ;
    static_assert(kMaxDrawChunks <= 2 * kWave, "two chunks per lane of a sequence");
    const int K = a.K, tid = threadIdx.x, lane = tid % kWave, nc = a.nchunk2;
    __shared__ float s_tau, s_base, s_S;
    __shared__ int s_cstar, s_resid, s_ok;
    const int32_t *tk = K > 0 ? a.tokens + static_cast<int64_t>(b) * K
                              : reinterpret_cast<const int32_t *>(a.u_sample + b);
    const int32_t my_tok = tk[min(lane, max(K - 1, 0))];
    const float us = a.u_sample[b];
    uint32_t ptag, tag;
    item_tags(a, ptag, tag);
    int j;
    DrawRow w;
    if (!read_record(a, b, tag, j, w)) {
        fail_sequence(a, b);
        return;
    }
    if (j < 0 || j >= K) return;  // a failed resolve (reported), or the bonus item's draw
    if (nc == 1) return;          // a one-chunk row: its draw item drew
    w.resid = true;
    w.trow = (static_cast<int64_t>(b) * (K + 1) + j) * a.V;
    w.drow = (static_cast<int64_t>(b) * K + j) * a.V;
    if (tid < kWave) {
        const uint64_t *sums = a.sums + 2 * static_cast<int64_t>(b) * nc;
        const int i0 = min(2 * lane, nc - 1), i1 = min(2 * lane + 1, nc - 1);
        const bool in0 = 2 * lane < nc, in1 = 2 * lane + 1 < nc;
        uint64_t w[4];
        bool fresh;
        const uint64_t t0 = wall_clock64();
        for (;;) {
            w[0] = fetch(&sums[2 * i0]);
            w[1] = fetch(&sums[2 * i0 + 1]);
            w[2] = fetch(&sums[2 * i1]);
            w[3] = fetch(&sums[2 * i1 + 1]);
            fresh = __all(current(w[0], tag) && current(w[1], tag) && current(w[2], tag) &&
                          current(w[3], tag));
            if (fresh || wall_clock64() - t0 > kWaitTicks) break;
            __builtin_amdgcn_s_sleep(8);
        }
        const float r0 = in0 ? word_f32(w[0]) : 0.f, p0 = in0 ? word_f32(w[1]) : 0.f;
        const float r1 = in1 ? word_f32(w[2]) : 0.f, p1 = in1 ? word_f32(w[3]) : 0.f;
        const bool resid = wave_last(wave_incl_sum(r0 + r1)) > 0.f;
        float S, tau, base;
        int cstar;
        crossing_chunk(resid ? r0 : p0, resid ? r1 : p1, us, S, tau, cstar, base);
        if (lane == 0) {
            s_ok = fresh;
            s_cstar = cstar;
            s_base = base;
            s_tau = tau;
            s_S = S;
            s_resid = resid;
        }
    }
    __syncthreads();
    if (!s_ok) {
        fail_sequence(a, b);
        return;
    }
    const int ch = s_cstar;
    const bool resid = s_resid;
    const int64_t c0 = static_cast<int64_t>(ch) * C2;
    const int n = static_cast<int>(min(static_cast<int64_t>(C2), static_cast<int64_t>(a.V) - c0));
    uint4 rt[NQ], rd[NQ];
    float lp[NQ], lr[NQ], ex_r[NQ], ex_p[NQ], mr, mp, start[NQ], l[NQ];
    chunk_weights<DT, VecOk, true>(a, w, c0, n, rt, rd, lp, lr);
    round_scan2<NQ>(lr, lp, ex_r, ex_p, mr, mp);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        start[q] = s_base + (resid ? ex_r[q] : ex_p[q]);
        l[q] = resid ? lr[q] : lp[q];
    }
    search_emit<DT, true>(a, b, c0, j, w, resid, s_tau, start, l, rt, rd, s_S, my_tok, lds);
}

// The bonus row's statistics of sequence b, on wavefront 0: per statistics
// chunk into LDS (lane i holds chunks i and i + 64), and merged in double
// precision into the row's (ref, 1/z).  With Live the words are read with
// device-scope loads until all carry `ptag` (bounded).  Returns false if a
// word was not written in time.
template <bool Live>
__device__ __forceinline__ bool bonus_row(const ChainArgs &a, int b, uint32_t ptag, float &rt,
                                          float &izt, float *lds) {
    static_assert(kMaxStatChunks <= 2 * kWave, "two statistics chunks per lane");
    __shared__ float s_rt, s_izt;
    __shared__ int s_okb;
    const int K = a.K, nch = a.nchunk, lane = threadIdx.x % kWave;
    float *s_kref = lds + kDrawBonusAt, *s_kz = s_kref + kMaxStatChunks;
    if (threadIdx.x < kWave) {
        const uint64_t *part = a.partial + 2 * ((static_cast<int64_t>(b) * (2 * K + 1) + K) * nch);
        const int i0 = min(lane, nch - 1), i1 = min(lane + kWave, nch - 1);
        const bool in0 = lane < nch, in1 = lane + kWave < nch;
        const uint64_t t0 = Live ? wall_clock64() : 0;
        uint64_t w[4];
        bool fresh;
        for (;;) {
            w[0] = fetch(part + 2 * i0);
            w[1] = fetch(part + 2 * i0 + 1);
            w[2] = fetch(part + 2 * i1);
            w[3] = fetch(part + 2 * i1 + 1);
            fresh = __all((!in0 || (current(w[0], ptag) && current(w[1], ptag))) &&
                          (!in1 || (current(w[2], ptag) && current(w[3], ptag))));
            if (fresh || !Live || wall_clock64() - t0 > kWaitTicks) break;
            __builtin_amdgcn_s_sleep(8);
        }
        const float r0 = in0 ? word_f32(w[0]) : -INFINITY, z0 = in0 ? word_f32(w[1]) : 0.f;
        const float r1 = in1 ? word_f32(w[2]) : -INFINITY, z1 = in1 ? word_f32(w[3]) : 0.f;
        if (in0) {
            s_kref[lane] = r0;
            s_kz[lane] = z0;
        }
        if (in1) {
            s_kref[lane + kWave] = r1;
            s_kz[lane + kWave] = z1;
        }
        float ref = r0;
        double z = z0;
        mz_merge_d(ref, z, r1, z1);
        mz_wave_merge_d(ref, z);
        if (lane == kWave - 1) {
            s_rt = ref;
            s_izt = 1.f / static_cast<float>(z);
            s_okb = fresh;
        }
    }
    __syncthreads();
    rt = s_rt;
    izt = s_izt;
    return s_okb != 0;
}

// Bonus item of sequence b: if every draft was accepted, it draws the bonus
// token from p_K.  The mass of each draw chunk follows from the bonus row's
// statistics, z_c * 2^(ref_c - ref) / z over the two statistics chunks it
// covers, with no second read of the row; only the crossing chunk's entries
// are loaded.
template <class DT, bool VecOk, bool Live>
__device__ __forceinline__ void bonus_item(const ChainArgs &a, int b, float *lds) {
    using CK = Chunk2<DT>;
    constexpr int C2 = CK::kElems, NQ = CK::kNQ;
    const int K = a.K, tid = threadIdx.x, lane = tid % kWave, nc = a.nchunk2;
    __shared__ float s_tau, s_base, s_S;
    __shared__ int s_cstar;
    const int32_t *tk = K > 0 ? a.tokens + static_cast<int64_t>(b) * K
                              : reinterpret_cast<const int32_t *>(a.u_sample + b);
    const int32_t my_tok = tk[min(lane, max(K - 1, 0))];
    const float us = a.u_sample[b];
    uint32_t ptag, tag;
    item_tags(a, ptag, tag);
    int j;
    DrawRow w;
    if (!read_record(a, b, tag, j, w)) {
        fail_sequence(a, b);
        return;
    }
    if (j != K) return;  // a residual draw, or a failed resolve (reported)
    if (!bonus_row<Live>(a, b, ptag, w.rt, w.izt, lds)) {
        fail_sequence(a, b);
        return;
    }
    w.resid = false;
    w.trow = (static_cast<int64_t>(b) * (K + 1) + K) * a.V;
    w.drow = 0;
    w.rd = w.izd = 0.f;
    if (tid < kWave) {
        // A draw chunk is a statistics chunk: its mass of p_K follows from
        // the chunk's (ref, z).
        const float *s_kref = lds + kDrawBonusAt, *s_kz = s_kref + kMaxStatChunks;
        const int i0 = min(2 * lane, nc - 1), i1 = min(2 * lane + 1, nc - 1);
        const float m0 = 2 * lane < nc ? __fmul_rn(s_kz[i0] * exp2_hw(s_kref[i0] - w.rt), w.izt) : 0.f;
        const float m1 = 2 * lane + 1 < nc ? __fmul_rn(s_kz[i1] * exp2_hw(s_kref[i1] - w.rt), w.izt) : 0.f;
        float S, tau, base;
        int cstar;
        crossing_chunk(m0, m1, us, S, tau, cstar, base);
        if (lane == 0) {
            s_cstar = cstar;
            s_base = base;
            s_tau = tau;
            s_S = S;
        }
    }
    __syncthreads();
    const int ch = s_cstar;
    const int64_t c0 = static_cast<int64_t>(ch) * C2;
    const int n = static_cast<int>(min(static_cast<int64_t>(C2), static_cast<int64_t>(a.V) - c0));
    uint4 rt[NQ], rd[NQ];
    float lp[NQ], lr[NQ], ex_r[NQ], ex_p[NQ], mr, mp, start[NQ];
    chunk_weights<DT, VecOk, false>(a, w, c0, n, rt, rd, lp, lr);
    round_scan2<NQ>(lr, lp, ex_r, ex_p, mr, mp);
#pragma unroll
    for (int q = 0; q < NQ; ++q) start[q] = s_base + ex_p[q];
    search_emit<DT, false>(a, b, c0, K, w, false, s_tau, start, lp, rt, rd, s_S, my_tok, lds);
}

// Grid (chunk, row, sequence): the hardware hands out the item, so nothing
// stands between a workgroup's start and its first loads.  Workgroup (0, 0,
// 0) records the call's tag in the workspace header for the draws.
template <class DT, bool VecOk>
__global__ __launch_bounds__(kWG) void k_chain_stats(ChainArgs a) {
    stats_item<DT, VecOk>(a, blockIdx.z, static_cast<int>(blockIdx.y), static_cast<int>(blockIdx.x));
    if ((blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0)
        a.hdr[kHdrPhaseTag] = a.tag_src ? *a.tag_src : a.tag;
}

// The draws of the two-phase form: B resolvers, B * D draw items, B
// finishers and B bonus items (each waits only for items of lower index).
template <class DT, bool VecOk>
__global__ __launch_bounds__(kWG) void k_chain_draw(ChainArgs a) {
    __shared__ __align__(16) float lds[kDrawLds];
    const ChainItem it = chain_draw_item(blockIdx.x, a);
    const int b = static_cast<int>(it.b);
    if (it.kind == kItemResolver) resolver_item<DT, false>(a, b, lds);
    else if (it.kind == kItemDraw) draw_item<DT, VecOk>(a, b, static_cast<int>(it.p), lds);
    else if (it.kind == kItemFinisher) finisher_item<DT, VecOk>(a, b, lds);
    else bonus_item<DT, VecOk, false>(a, b, lds);
}

// The whole chain verify in one launch, in one of three orders (each its own
// kernel, so that each carries only its own decode and item kinds: an unused
// branch measured 4 us slower on 64 x 5 x 128256 bf16 through the scalar
// registers it cost the statistics items):
//   kSeqMajor        chain_fused_item on a 1D grid, one resolver per sequence;
//   kPosMajor        chain_pm_item on a 3D grid, one pair resolver per
//                    position of each sequence; statistics items of position
//                    k >= 2 skip their chunk after a published rejection
//                    below k;
//   kPosMajorGate1   the same, and items of position 1 skip too (positions
//                    whose rows stream long enough for position 0's
//                    outcomes to come out early in position 1).
// Sequence-major: each resolver finds its statistics done or nearly so, and
// the stream of logits runs undisturbed: draws placed among the statistics
// measured slower at every lag tried (their second read of row j takes slots
// and bandwidth from the stream), so the second reads all come after it,
// where the bonus draws, which need none, also run.
enum ChainOrder : int { kSeqMajor = 0, kPosMajor = 1, kPosMajorGate1 = 2 };

template <class DT, bool VecOk, int Order>
__global__ __launch_bounds__(kWG, 8) void k_chain_fused(ChainArgs a) {
    __shared__ __align__(16) float lds[kDrawLds];
    // The statistics items' arguments are loaded with the schedule's, in one
    // batch ahead of the decode: otherwise the compiler sinks them into the
    // item's branch, and every workgroup waits for a second round of argument
    // loads before its first logit load.
    asm volatile("" ::"s"(a.target), "s"(a.draft), "s"(a.partial), "s"(a.c), "s"(a.V), "s"(a.chunk),
                 "s"(a.tag), "s"(a.tag_src));
    int row = 0, ch = 0;
    const ChainItem it = Order == kSeqMajor ? chain_fused_item(blockIdx.x, a)
                                            : chain_pm_item(blockIdx.x, blockIdx.y, blockIdx.z, a, row, ch);
    const int b = static_cast<int>(it.b);
    if (it.kind == kItemStats) {
        if constexpr (Order == kSeqMajor) chain_stats_row(it.p, a, row, ch);
        if constexpr (Order != kSeqMajor) {
            const int pos = static_cast<int>(blockIdx.z);
            if (pos >= (Order == kPosMajorGate1 ? 1 : 2)) {
                if constexpr (VecOk) {
                    // In a gated position the item of chunk ch, ch a multiple
                    // of G, streams chunks ch .. ch + G - 1 after one gate
                    // read; the other items return at once.  1/G of the gate
                    // reads, and a skipped row costs 1/G of the workgroup
                    // lives.  G = 2 for short positions, 4 for long ones
                    // (64 x 5 x 128256 bf16: 33.5 us with pairs, 35.7 with
                    // fours; 256 x 8 x 151936 fp32: 253 us with pairs, 243
                    // with fours).
                    constexpr int G = Order == kPosMajorGate1 ? 4 : 2;
                    if (ch % G != 0) return;
                    if (rows_not_needed(a, b, pos)) return;
                    stats_group<DT, G>(a, it.b, row, ch);
                    return;
                }
                if (rows_not_needed(a, b, pos)) return;
            }
        }
        stats_item<DT, VecOk>(a, it.b, row, ch);
    } else if (Order != kSeqMajor && it.kind == kItemNone) {
        return;
    } else if (it.kind == kItemBonusStats) {
        // The bonus row matters only when every draft is accepted; after a
        // rejection already recorded its chunk is not read.
        if (a.gate_bonus && bonus_not_needed(a, b)) return;
        stats_item<DT, VecOk>(a, it.b, a.K, static_cast<int>(it.p));
    } else if (Order != kSeqMajor && it.kind == kItemPair) {
        pair_resolver_item<DT, Order != kSeqMajor>(a, b, static_cast<int>(it.p));
    } else if (Order == kSeqMajor && it.kind == kItemResolver) {
        resolver_item<DT, true>(a, b, lds);
    } else if (it.kind == kItemDraw) {
        draw_item<DT, VecOk>(a, b, static_cast<int>(it.p), lds);
    } else if (it.kind == kItemFinisher) {
        finisher_item<DT, VecOk>(a, b, lds);
    } else {
        bonus_item<DT, VecOk, true>(a, b, lds);
    }
}

template <class DT, bool VecOk>
void launch_fused_order(const ChainArgs &a, dim3 g, hipStream_t s) {
    if (!a.early_exit) k_chain_fused<DT, VecOk, kSeqMajor><<<g, kWG, 0, s>>>(a);
    else if (!a.gate_pos1) k_chain_fused<DT, VecOk, kPosMajor><<<g, kWG, 0, s>>>(a);
    else k_chain_fused<DT, VecOk, kPosMajorGate1><<<g, kWG, 0, s>>>(a);
}

}  // namespace

hipError_t launch_chain_stats(const ChainArgs &a, int dtype, hipStream_t s) {
    const dim3 g(a.nchunk, 2 * a.K + 1, a.B), blk(kWG);
    if (dtype == 1) {
        if (a.V % Bf16::kVec == 0) k_chain_stats<Bf16, true><<<g, blk, 0, s>>>(a);
        else k_chain_stats<Bf16, false><<<g, blk, 0, s>>>(a);
    } else {
        if (a.V % F32::kVec == 0) k_chain_stats<F32, true><<<g, blk, 0, s>>>(a);
        else k_chain_stats<F32, false><<<g, blk, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_chain_fused(const ChainArgs &a, int dtype, hipStream_t s) {
    const Grid3 pm = chain_pm_grid(a);
    const dim3 g = a.early_exit ? dim3(pm.x, pm.y, pm.z) : dim3(chain_fused_grid(a));
    if (dtype == 1) {
        if (a.V % Bf16::kVec == 0) launch_fused_order<Bf16, true>(a, g, s);
        else launch_fused_order<Bf16, false>(a, g, s);
    } else {
        if (a.V % F32::kVec == 0) launch_fused_order<F32, true>(a, g, s);
        else launch_fused_order<F32, false>(a, g, s);
    }
    return hipGetLastError();
}

hipError_t launch_chain_draw(const ChainArgs &a, int dtype, hipStream_t s) {
    const dim3 g(chain_draw_grid(a)), blk(kWG);
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
