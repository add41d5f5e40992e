// Chain verify at T > 0 on gfx950: two kernels.
//
// k_chain_stats streams every logit of the step once.  One workgroup takes one
// vocabulary chunk of one row (target rows 0..K and draft rows 0..K-1 of a
// sequence), folds it into softmax statistics (ref, z) and writes them to the
// workspace.  This is the HBM-bound pass that carries almost all the bytes.
//
// k_chain_sample runs one workgroup per (sequence, chunk).  Each one merges the
// sequence's row statistics, evaluates the accept test of every drafted token
// (u < p(x)/q(x), French lesson "La règle de l'exactitude"; forum post §3) and
// finds the first rejection j.  It then sums the draw weights of its chunk of
// row j: max(0, p_j - q_j) for a rejection (the residual of the same passages)
// or p_K for the bonus draw when every draft was accepted.  The last workgroup
// of a sequence to finish (device-scope counter) locates the chunk whose
// running mass crosses u * S, stages that chunk's weights in LDS, scans them
// and writes the emitted tokens.
#include "device.hpp"
#include "plan.hpp"

namespace sv {
namespace {

template <class DT, int U>
__global__ __launch_bounds__(kWG) void k_chain_stats(ChainArgs a) {
    constexpr int VEC = DT::kVec;
    const int K = a.K, V = a.V, R = 2 * K + 1;
    const int64_t row = blockIdx.x / a.nchunk;
    const int ch = blockIdx.x % a.nchunk;
    const int64_t b = row / R;
    const int r = static_cast<int>(row % R);

    const void *base;
    int64_t trow;
    if (r <= K) {
        base = a.target;
        trow = b * (K + 1) + r;
    } else {
        base = a.draft;
        trow = b * K + (r - K - 1);
    }
    const int64_t g0 = trow * V + static_cast<int64_t>(ch) * a.chunk;
    const int64_t g1 = min(g0 + a.chunk, trow * V + V);
    const Span s = split_span<VEC>(g0, g1);

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
        a.partial[row * a.nchunk + ch] = make_float2(ref, z);
        // The second kernel elects its last workgroup per sequence with this counter.
        if (r == 0 && ch == 0) a.counters[b] = 0u;
    }
}

// Draw weight of one vocabulary entry of row j.
__device__ __forceinline__ float draw_weight(float t, float d, float c, float rt, float izt,
                                             float rd, float izd, bool resid) {
    const float p = __fmul_rn(exp2_hw(fmaf(t, c, -rt)), izt);
    if (!resid) return p;
    const float q = __fmul_rn(exp2_hw(fmaf(d, c, -rd)), izd);
    return fmaxf(p - q, 0.f);
}

// Sum of the draw weights of elements [e0, e1) of row j, valid in thread 0.
template <class DT>
__device__ float chunk_mass(const ChainArgs &a, int64_t trow, int64_t drow, int64_t e0,
                            int64_t e1, float rt, float izt, float rd, float izd, bool resid) {
    constexpr int VEC = DT::kVec;
    float acc = 0.f;
    if (a.V % VEC == 0) {
        // Rows and chunk bounds are vector aligned: 16-byte loads.
        const uint4 *tp = static_cast<const uint4 *>(a.target);
        const uint4 *dp = static_cast<const uint4 *>(a.draft);
        const int64_t v0 = (trow + e0) / VEC, v1 = (trow + e1) / VEC;
        const int64_t w0 = (drow + e0) / VEC;
        for (int64_t v = v0 + threadIdx.x; v < v1; v += kWG) {
            float t[VEC], d[VEC];
            unpack<DT>(tp[v], t);
            if (resid) unpack<DT>(dp[w0 + (v - v0)], d);
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                acc += draw_weight(t[i], resid ? d[i] : 0.f, a.c, rt, izt, rd, izd, resid);
        }
    } else {
        for (int64_t e = e0 + threadIdx.x; e < e1; e += kWG) {
            const float t = load_one<DT>(a.target, trow + e);
            const float d = resid ? load_one<DT>(a.draft, drow + e) : 0.f;
            acc += draw_weight(t, d, a.c, rt, izt, rd, izd, resid);
        }
    }
    return sum_wg(acc);
}

constexpr int kSeg = kChunk2 / kWG;                  // elements per thread in the final scan
__host__ __device__ constexpr int lds_pad(int e) { return e + e / 32; }

template <class DT>
__global__ __launch_bounds__(kWG) void k_chain_sample(ChainArgs a) {
    const int K = a.K, V = a.V, R = 2 * K + 1;
    const int b = blockIdx.x / a.nchunk2;
    const int ch = blockIdx.x % a.nchunk2;
    const int tid = threadIdx.x;

    __shared__ float s_ref[2 * kMaxK + 1], s_z[2 * kMaxK + 1];
    __shared__ float s_P[kMaxK], s_Q[kMaxK];
    __shared__ int s_j, s_last, s_cstar;
    __shared__ float s_S, s_tau, s_base;
    __shared__ float s_w[lds_pad(kChunk2)];

    // Row statistics of the sequence: merge the per-chunk pairs in chunk order.
    for (int r = tid; r < R; r += kWG) {
        const float2 *p = a.partial + (static_cast<int64_t>(b) * R + r) * a.nchunk;
        float ref = -INFINITY, z = 0.f;
        for (int i = 0; i < a.nchunk; ++i) {
            const float2 q = p[i];
            mz_merge(ref, z, q.x, q.y);
        }
        s_ref[r] = ref;
        s_z[r] = z;
    }
    __syncthreads();

    // Accept test of every drafted token; j = first rejection (wave 0, K <= 64).
    if (tid < kWave) {
        bool reject = false;
        if (tid < K) {
            const int x = min(max(a.tokens[b * K + tid], 0), V - 1);
            const float lt = load_one<DT>(a.target, (static_cast<int64_t>(b) * (K + 1) + tid) * V + x);
            const float ld = load_one<DT>(a.draft, (static_cast<int64_t>(b) * K + tid) * V + x);
            const float P = exp2_hw(fmaf(lt, a.c, -s_ref[tid])) / s_z[tid];
            const float Q = exp2_hw(fmaf(ld, a.c, -s_ref[K + 1 + tid])) / s_z[K + 1 + tid];
            const float u = a.u_accept[b * K + tid];
            const bool accept = Q > 0.f ? (u < P / Q) : (P > 0.f);
            reject = !accept;
            s_P[tid] = P;
            s_Q[tid] = Q;
        }
        const uint64_t m = __ballot(reject);
        if (tid == 0) s_j = m ? (__ffsll(static_cast<unsigned long long>(m)) - 1) : K;
    }
    __syncthreads();
    const int j = s_j;
    bool resid = j < K;
    const float rt = s_ref[j], izt = 1.f / s_z[j];
    const float rd = resid ? s_ref[K + 1 + j] : 0.f;
    const float izd = resid ? 1.f / s_z[K + 1 + j] : 0.f;
    const int64_t trow = (static_cast<int64_t>(b) * (K + 1) + j) * V;
    const int64_t drow = resid ? (static_cast<int64_t>(b) * K + j) * V : 0;

    // This workgroup's share: the draw mass of one chunk of row j.
    {
        const int64_t e0 = static_cast<int64_t>(ch) * kChunk2;
        const int64_t e1 = min(static_cast<int64_t>(V), e0 + kChunk2);
        const float mass = chunk_mass<DT>(a, trow, drow, e0, e1, rt, izt, rd, izd, resid);
        if (tid == 0) {
            a.sums[static_cast<int64_t>(b) * a.nchunk2 + ch] = mass;
            __threadfence();
            const uint32_t done = atomicAdd(&a.counters[b], 1u);
            s_last = (done == static_cast<uint32_t>(a.nchunk2 - 1));
        }
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();  // acquire: every chunk's mass of this sequence is visible

    float *sums = a.sums + static_cast<int64_t>(b) * a.nchunk2;
    if (tid == 0) {
        float S = 0.f;
        for (int i = 0; i < a.nchunk2; ++i) S += sums[i];
        s_S = S;
    }
    __syncthreads();
    if (resid && s_S == 0.f) {
        // All-zero residual (only reachable through rounding): draw from p_j.
        resid = false;
        for (int i = 0; i < a.nchunk2; ++i) {
            const int64_t e0 = static_cast<int64_t>(i) * kChunk2;
            const int64_t e1 = min(static_cast<int64_t>(V), e0 + kChunk2);
            const float mass = chunk_mass<DT>(a, trow, drow, e0, e1, rt, izt, rd, izd, false);
            if (tid == 0) sums[i] = mass;
        }
        if (tid == 0) {
            float S = 0.f;
            for (int i = 0; i < a.nchunk2; ++i) S += sums[i];
            s_S = S;
        }
        __syncthreads();
    }

    // Crossing chunk: the first whose inclusive running mass exceeds u * S.
    if (tid == 0) {
        const float S = s_S;
        const float tau = a.u_sample[b] * S;
        float cum = 0.f;
        int cstar = -1, last_pos = 0;
        float base = 0.f, base_last = 0.f;
        for (int i = 0; i < a.nchunk2; ++i) {
            const float m = sums[i];
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
        if (cstar < 0) {  // u * S rounded up to S: take the last chunk with mass
            cstar = last_pos;
            base = base_last;
        }
        s_cstar = cstar;
        s_base = base;
        s_tau = tau;
    }
    __syncthreads();

    // Stage the crossing chunk's weights in LDS and scan them in index order.
    const int64_t c0 = static_cast<int64_t>(s_cstar) * kChunk2;
    const int n = static_cast<int>(min(static_cast<int64_t>(kChunk2), static_cast<int64_t>(V) - c0));
    for (int e = tid; e < n; e += kWG) {
        const float t = load_one<DT>(a.target, trow + c0 + e);
        const float d = resid ? load_one<DT>(a.draft, drow + c0 + e) : 0.f;
        s_w[lds_pad(e)] = draw_weight(t, d, a.c, rt, izt, rd, izd, resid);
    }
    __syncthreads();
    const int s0 = tid * kSeg;
    float local = 0.f;
    for (int e = s0; e < min(s0 + kSeg, n); ++e) local += s_w[lds_pad(e)];
    float run = s_base + exclusive_scan_wg(local);
    const float tau = s_tau;
    int found = INT32_MAX, last_nz = -1;
    for (int e = s0; e < min(s0 + kSeg, n); ++e) {
        const float w = s_w[lds_pad(e)];
        run += w;
        if (found == INT32_MAX && run > tau) found = e;
        if (w > 0.f) last_nz = e;
    }
    found = min_wg(found);
    last_nz = max_wg(last_nz);
    const int pick = (found != INT32_MAX) ? found : max(last_nz, 0);
    const int32_t token = static_cast<int32_t>(c0 + pick);

    // Emit x_0..x_{j-1}, then the drawn token, then -1.
    for (int k = tid; k <= K; k += kWG) {
        int32_t o = -1;
        if (k < j) o = a.tokens[b * K + k];
        else if (k == j) o = token;
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
    if (tid == 0) a.out_accepted[b] = j;
}

}  // namespace

hipError_t launch_chain_stats(const ChainArgs &a, int dtype, hipStream_t s) {
    const int64_t grid = static_cast<int64_t>(a.B) * (2 * a.K + 1) * a.nchunk;
    if (dtype == 1)
        k_chain_stats<Bf16, 8><<<dim3(static_cast<uint32_t>(grid)), dim3(kWG), 0, s>>>(a);
    else
        k_chain_stats<F32, 8><<<dim3(static_cast<uint32_t>(grid)), dim3(kWG), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_chain_sample(const ChainArgs &a, int dtype, hipStream_t s) {
    const int64_t grid = static_cast<int64_t>(a.B) * a.nchunk2;
    if (dtype == 1)
        k_chain_sample<Bf16><<<dim3(static_cast<uint32_t>(grid)), dim3(kWG), 0, s>>>(a);
    else
        k_chain_sample<F32><<<dim3(static_cast<uint32_t>(grid)), dim3(kWG), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sv
