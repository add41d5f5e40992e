// Greedy verify at T = 0 on gfx950: a row-argmax streaming pass, then a small
// per-sequence resolve (French lesson, "La règle de l'exactitude", greedy case,
// for the chain; "Vérifie l'attention des arbres" and the EAGLE section for the
// tree: one target pass scores every candidate and the longest accepted branch
// wins).
//
// k_row_argmax: one workgroup per vocabulary chunk of one row; 16-byte loads,
// per-lane (max, lowest index) kept in index order, then a workgroup reduce.
// Values are compared as floats widened exactly from bf16, so ties and -0.0 ==
// +0.0 behave as on the raw logits.
#include "device.hpp"
#include "plan.hpp"

namespace sv {
namespace {

template <class DT, int U>
__global__ __launch_bounds__(kWG) void k_row_argmax(ArgmaxArgs a) {
    constexpr int VEC = DT::kVec;
    const int64_t row = blockIdx.x / a.nchunk;
    const int ch = blockIdx.x % a.nchunk;
    const int64_t rbase = row * a.V;
    const int64_t g0 = rbase + static_cast<int64_t>(ch) * a.chunk;
    const int64_t g1 = min(g0 + a.chunk, rbase + a.V);
    const Span s = split_span<VEC>(g0, g1);

    // Each lane visits its elements in increasing index order, so a strict
    // comparison keeps the lowest index among equal values.
    float bv = -INFINITY;
    int32_t bi = INT32_MAX;
    {
        const int64_t h = s.h0 + threadIdx.x;
        if (h < s.h1) {
            const float x = load_one<DT>(a.logits, h);
            if (vi_better(x, static_cast<int32_t>(h - rbase), bv, bi)) {
                bv = x;
                bi = static_cast<int32_t>(h - rbase);
            }
        }
    }
    const uint4 *vp = static_cast<const uint4 *>(a.logits);
    int64_t v = s.va + threadIdx.x;
    for (; v + (U - 1) * kWG < s.vb; v += U * kWG) {
        uint4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = vp[v + u * kWG];
        float x[U * VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) unpack<DT>(raw[u], x + u * VEC);
        float m = x[0];
#pragma unroll
        for (int i = 1; i < U * VEC; ++i) m = fmaxf(m, x[i]);
        if (m > bv) {
            // Rare after the first batches: locate the first element equal to m.
            int at = 0;
#pragma unroll
            for (int i = U * VEC - 1; i >= 0; --i)
                if (x[i] == m) at = i;
            bv = m;
            bi = static_cast<int32_t>((v + (at / VEC) * kWG) * VEC + (at % VEC) - rbase);
        }
    }
    for (; v < s.vb; v += kWG) {
        float x[VEC];
        unpack<DT>(vp[v], x);
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            if (x[i] > bv) {
                bv = x[i];
                bi = static_cast<int32_t>(v * VEC + i - rbase);
            }
    }
    {
        const int64_t t = s.t0 + threadIdx.x;
        if (t < s.t1) {
            const float x = load_one<DT>(a.logits, t);
            if (vi_better(x, static_cast<int32_t>(t - rbase), bv, bi)) {
                bv = x;
                bi = static_cast<int32_t>(t - rbase);
            }
        }
    }
    vi_reduce_wg(bv, bi);
    if (threadIdx.x == 0) a.partial[row * a.nchunk + ch] = make_int2(__float_as_int(bv), bi);
}

// argmax of one row from its chunk partials (chunks in index order).
__device__ __forceinline__ int32_t merge_argmax(const int2 *p, int nchunk) {
    float bv = -INFINITY;
    int32_t bi = INT32_MAX;
    for (int i = 0; i < nchunk; ++i) {
        const float v = __int_as_float(p[i].x);
        if (vi_better(v, p[i].y, bv, bi)) {
            bv = v;
            bi = p[i].y;
        }
    }
    return bi == INT32_MAX ? 0 : bi;  // an all -inf row (outside the contract) maps to 0
}

constexpr int kGreedyThreads = 2 * kWave;  // rows 0..K with K <= 64

__global__ __launch_bounds__(kGreedyThreads) void k_greedy_resolve(GreedyArgs a) {
    const int b = blockIdx.x, k = threadIdx.x, K = a.K;
    __shared__ int32_t s_a[kMaxK + 1];
    __shared__ int s_j;
    if (k <= K) s_a[k] = merge_argmax(a.partial + (static_cast<int64_t>(b) * (K + 1) + k) * a.nchunk, a.nchunk);
    __syncthreads();
    if (k < kWave) {
        const bool mismatch = k < K && a.tokens[b * K + k] != s_a[k];
        const uint64_t m = __ballot(mismatch);
        if (k == 0) s_j = m ? (__ffsll(static_cast<unsigned long long>(m)) - 1) : K;
    }
    __syncthreads();
    const int j = s_j;
    if (k <= K) {
        int32_t o = -1;
        if (k < j) o = a.tokens[b * K + k];
        else if (k == j) o = s_a[k];
        a.out_tokens[static_cast<int64_t>(b) * (K + 1) + k] = o;
    }
    if (k == 0) a.out_accepted[b] = j;
}

__global__ __launch_bounds__(kMaxTreeNodes) void k_tree_resolve(TreeArgs a) {
    const int b = blockIdx.x, v = threadIdx.x;
    const int N = a.tree.N, D = a.tree.D;
    __shared__ int32_t s_a[kMaxTreeNodes];
    __shared__ int s_ok[kMaxTreeNodes];
    __shared__ int s_anc[kMaxTreeNodes];
    __shared__ int s_best;
    __shared__ int s_path[kMaxTreeNodes];
    if (v < N) s_a[v] = merge_argmax(a.partial + (static_cast<int64_t>(b) * N + v) * a.nchunk, a.nchunk);
    __syncthreads();
    // match[v]: v's token equals its parent's argmax; accepted = all matches
    // on the path to the root, folded by pointer jumping (depth <= 255).
    int par = v < N ? a.tree.parent[v] : -1;
    if (v < N) {
        s_ok[v] = (v == 0) ? 1 : (a.tokens[static_cast<int64_t>(b) * N + v] == s_a[par]);
        s_anc[v] = par;
    }
    __syncthreads();
    for (int step = 1; step < kMaxTreeNodes; step <<= 1) {
        int ok = 0, anc = -1;
        if (v < N) {
            anc = s_anc[v];
            ok = s_ok[v];
            if (anc >= 0) {
                ok &= s_ok[anc];
                anc = s_anc[anc];
            }
        }
        __syncthreads();
        if (v < N) {
            s_ok[v] = ok;
            s_anc[v] = anc;
        }
        __syncthreads();
    }
    // Deepest accepted node, lowest index among equals.
    const int key = (v < N && s_ok[v]) ? ((a.tree.depth[v] << 16) | (0xFFFF - v)) : -1;
    const int best_key = max_wg(key);
    if (v == 0) s_best = 0xFFFF - (best_key & 0xFFFF);
    __syncthreads();
    if (v == 0) {
        const int best = s_best;
        const int d = a.tree.depth[best];
        int *path = s_path;
        int node = best;
        for (int i = d; i >= 0; --i) {
            path[i] = node;
            node = a.tree.parent[node];
        }
        int32_t *ot = a.out_tokens + static_cast<int64_t>(b) * (D + 1);
        for (int i = 0; i <= D; ++i) {
            int32_t o = -1;
            if (i < d) o = a.tokens[static_cast<int64_t>(b) * N + path[i + 1]];
            else if (i == d) o = s_a[best];
            ot[i] = o;
        }
        if (a.out_path) {
            int32_t *op = a.out_path + static_cast<int64_t>(b) * (D + 1);
            for (int i = 0; i <= D; ++i) op[i] = i <= d ? path[i] : -1;
        }
        a.out_depth[b] = d;
    }
}

}  // namespace

hipError_t launch_row_argmax(const ArgmaxArgs &a, int dtype, hipStream_t s) {
    const int64_t grid = a.rows * a.nchunk;
    if (dtype == 1)
        k_row_argmax<Bf16, 4><<<dim3(static_cast<uint32_t>(grid)), dim3(kWG), 0, s>>>(a);
    else
        k_row_argmax<F32, 4><<<dim3(static_cast<uint32_t>(grid)), dim3(kWG), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_greedy_resolve(const GreedyArgs &a, hipStream_t s) {
    k_greedy_resolve<<<dim3(static_cast<uint32_t>(a.B)), dim3(kGreedyThreads), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_tree_resolve(const TreeArgs &a, hipStream_t s) {
    k_tree_resolve<<<dim3(static_cast<uint32_t>(a.B)), dim3(kMaxTreeNodes), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace sv
