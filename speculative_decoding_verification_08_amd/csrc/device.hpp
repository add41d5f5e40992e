// Device-side building blocks of the verify kernels for gfx950 (wave64).
//
// Logit rows are streamed as 16-byte vectors (8 bf16 or 4 fp32 per lane and
// load), widened to fp32 in registers.  Softmax statistics are kept as a pair
// (ref, z): ref is a reference point in the exponent domain, ref = m * c with
// c = log2(e) / T and m the largest logit seen, and z = sum_i 2^(l_i*c - ref).
// All exponentials of one row are taken against the same rounded reference,
// so the rounding of m * c cancels between a probability's numerator and the
// row sum.  Every reduction runs in a fixed order: results are bitwise
// reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWG = 256;    // threads per workgroup of the streaming kernels
constexpr int kWave = 64;   // CDNA wavefront
constexpr int kWaves = kWG / kWave;

struct Bf16 {
    static constexpr int kVec = 8;  // elements per 16-byte vector
};
struct F32 {
    static constexpr int kVec = 4;
};

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// A 16-byte load marked non-temporal, for data read once (streamed logits,
// KV rows on their way to the cache): it should not displace data that is
// reused from the caches, and it streams faster than a plain load.
__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// One element of a logit array, widened exactly to fp32.
template <class DT>
__device__ __forceinline__ float load_one(const void *base, int64_t i);
template <>
__device__ __forceinline__ float load_one<Bf16>(const void *base, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(base)[i]) << 16);
}
template <>
__device__ __forceinline__ float load_one<F32>(const void *base, int64_t i) {
    return static_cast<const float *>(base)[i];
}

// A 16-byte vector widened to fp32, element order preserved.
template <class DT>
__device__ __forceinline__ void unpack(const uint4 &v, float *x);
template <>
__device__ __forceinline__ void unpack<Bf16>(const uint4 &v, float *x) {
    x[0] = __uint_as_float(v.x << 16);
    x[1] = __uint_as_float(v.x & 0xffff0000u);
    x[2] = __uint_as_float(v.y << 16);
    x[3] = __uint_as_float(v.y & 0xffff0000u);
    x[4] = __uint_as_float(v.z << 16);
    x[5] = __uint_as_float(v.z & 0xffff0000u);
    x[6] = __uint_as_float(v.w << 16);
    x[7] = __uint_as_float(v.w & 0xffff0000u);
}
template <>
__device__ __forceinline__ void unpack<F32>(const uint4 &v, float *x) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
}

// Element range [g0, g1) of a flat array split into a scalar head, whole
// 16-byte vectors [va, vb) (vector indices from the array base) and a scalar
// tail.  The array base is 16-byte aligned.
struct Span {
    int64_t h0, h1, va, vb, t0, t1;
};
template <int VEC>
__device__ __forceinline__ Span split_span(int64_t g0, int64_t g1) {
    const int64_t a = (g0 + VEC - 1) / VEC * VEC;
    if (a >= g1) return Span{g0, g1, 0, 0, g1, g1};
    const int64_t e = g1 / VEC * VEC;
    return Span{g0, a, a / VEC, e / VEC, e, g1};
}

// ------------------------------------------------------------------ softmax

// Merge two (ref, z) pairs.  A pair with ref = -inf is empty.
__device__ __forceinline__ void mz_merge(float &ref, float &z, float ref2, float z2) {
    const float m = fmaxf(ref, ref2);
    const float r = (m == -INFINITY) ? 0.f : m;
    z = z * exp2_hw(ref - r) + z2 * exp2_hw(ref2 - r);
    ref = m;
}

// The same with z in double precision.  A row's sum of exponentials is
// formed from per-thread fp32 sums of a few dozen terms, and every sum above
// that level (across lanes, wavefronts and chunks) is taken in double: the
// residual max(0, p - q) cancels most of p and q, so an error in either
// normaliser reaches the residual's mass amplified by 1 / mass.
__device__ __forceinline__ void mz_merge_d(float &ref, double &z, float ref2, double z2) {
    const float m = fmaxf(ref, ref2);
    const float r = (m == -INFINITY) ? 0.f : m;
    z = z * static_cast<double>(exp2_hw(ref - r)) + z2 * static_cast<double>(exp2_hw(ref2 - r));
    ref = m;
}

// Fold N logits into (ref, z): one max over the batch, one rescale, then one
// exp2 per element against the new reference.
template <int N>
__device__ __forceinline__ void mz_batch(const float *x, float c, float &ref, float &z) {
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) bm = fmaxf(bm, x[i]);
    const float rn = fmaxf(ref, bm * c);
    const float r = (rn == -INFINITY) ? 0.f : rn;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < N; ++i) s[i & 3] += exp2_hw(fmaf(x[i], c, -r));
    z = z * exp2_hw(ref - r) + ((s[0] + s[1]) + (s[2] + s[3]));
    ref = rn;
}

// Workgroup merge of (ref, z); the result is valid in thread 0.  Defined
// after the DPP helpers below.
__device__ __forceinline__ void mz_reduce_wg(float &ref, float &z);

// ------------------------------------------------------------------ argmax

// (value, index) with the larger value winning and the lower index breaking
// ties; -0.0 and +0.0 compare equal.
struct ValIdx {
    float v;
    int32_t i;
};
__device__ __forceinline__ bool vi_better(float v, int32_t i, float bv, int32_t bi) {
    return v > bv || (v == bv && i < bi);
}

// Workgroup argmax; the result is valid in thread 0.
__device__ __forceinline__ void vi_reduce_wg(float &v, int32_t &i) {
    __shared__ float s_v[kWaves];
    __shared__ int32_t s_i[kWaves];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const float v2 = __shfl_xor(v, off);
        const int32_t i2 = __shfl_xor(i, off);
        if (vi_better(v2, i2, v, i)) {
            v = v2;
            i = i2;
        }
    }
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) {
        s_v[w] = v;
        s_i[w] = i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < kWaves; ++k)
            if (vi_better(s_v[k], s_i[k], v, i)) {
                v = s_v[k];
                i = s_i[k];
            }
    }
    __syncthreads();
}

// ------------------------------------------------------------------ sums

// Workgroup sum in a fixed order; the result is valid in thread 0.
__device__ __forceinline__ float sum_wg(float x) {
    __shared__ float s_x[kWaves];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if ((threadIdx.x % kWave) == 0) s_x[threadIdx.x / kWave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        x = s_x[0];
        for (int k = 1; k < kWaves; ++k) x += s_x[k];
    }
    __syncthreads();
    return x;
}

// Exclusive prefix sum over the workgroup's threads in thread order.
__device__ __forceinline__ float exclusive_scan_wg(float x) {
    __shared__ float s_tot[kWaves];
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    float inc = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    if (lane == kWave - 1) s_tot[w] = inc;
    float ex = __shfl_up(inc, 1);
    if (lane == 0) ex = 0.f;
    __syncthreads();
    float base = 0.f;
    for (int k = 0; k < w; ++k) base += s_tot[k];
    __syncthreads();
    return base + ex;
}

__device__ __forceinline__ int min_wg(int x) {
    __shared__ int s_x[kWaves];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off));
    if ((threadIdx.x % kWave) == 0) s_x[threadIdx.x / kWave] = x;
    __syncthreads();
    int r = s_x[0];
    for (int k = 1; k < kWaves; ++k) r = min(r, s_x[k]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ int max_wg(int x) {
    __shared__ int s_x[kWaves];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
    if ((threadIdx.x % kWave) == 0) s_x[threadIdx.x / kWave] = x;
    __syncthreads();
    int r = s_x[0];
    for (int k = 1; k < kWaves; ++k) r = max(r, s_x[k]);
    __syncthreads();
    return r;
}


// ------------------------------------------------------------------ DPP

// Wavefront primitives on data-parallel-primitive (DPP) lane moves: each step
// is one VALU operation instead of an LDS-crossbar shuffle.  Row = 16 lanes.
// Lanes whose DPP source is out of range keep `identity`.
namespace dpp {
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kWaveShr1 = 0x138, kRowBcast15 = 0x142, kRowBcast31 = 0x143;

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ float mov_f(float identity, float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(x),
                                                      Ctrl, RowMask, 0xF, false));
}
template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ int mov_i(int identity, int x) {
    return __builtin_amdgcn_update_dpp(identity, x, Ctrl, RowMask, 0xF, false);
}
template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ double mov_d(double identity, double x) {
    const long long xi = __double_as_longlong(x), ii = __double_as_longlong(identity);
    const int lo = __builtin_amdgcn_update_dpp(static_cast<int>(ii), static_cast<int>(xi), Ctrl,
                                               RowMask, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(static_cast<int>(ii >> 32), static_cast<int>(xi >> 32),
                                               Ctrl, RowMask, 0xF, false);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<uint32_t>(lo));
}
}  // namespace dpp

// Inclusive sum over lanes 0..lane of a wavefront, in a fixed order: within
// rows of 16 by doubling shifts, then the rows' totals carried upward.
__device__ __forceinline__ float wave_incl_sum(float x) {
    x += dpp::mov_f<dpp::kRowShr1>(0.f, x);
    x += dpp::mov_f<dpp::kRowShr2>(0.f, x);
    x += dpp::mov_f<dpp::kRowShr4>(0.f, x);
    x += dpp::mov_f<dpp::kRowShr8>(0.f, x);
    x += dpp::mov_f<dpp::kRowBcast15, 0xA>(0.f, x);
    x += dpp::mov_f<dpp::kRowBcast31, 0xC>(0.f, x);
    return x;
}
// The same in double precision.
__device__ __forceinline__ double wave_incl_sum_d(double x) {
    x += dpp::mov_d<dpp::kRowShr1>(0.0, x);
    x += dpp::mov_d<dpp::kRowShr2>(0.0, x);
    x += dpp::mov_d<dpp::kRowShr4>(0.0, x);
    x += dpp::mov_d<dpp::kRowShr8>(0.0, x);
    x += dpp::mov_d<dpp::kRowBcast15, 0xA>(0.0, x);
    x += dpp::mov_d<dpp::kRowBcast31, 0xC>(0.0, x);
    return x;
}
__device__ __forceinline__ double wave_last_d(double x) {
    const long long v = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(v), 63);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), 63);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<uint32_t>(lo));
}
// Value of lane 63 (uniform).
__device__ __forceinline__ float wave_last(float x) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
}
__device__ __forceinline__ int wave_last_i(int x) { return __builtin_amdgcn_readlane(x, kWave - 1); }

// Minimum / maximum over the wavefront (uniform result).
__device__ __forceinline__ int wave_min_i(int x) {
    x = min(x, dpp::mov_i<dpp::kRowShr1>(INT32_MAX, x));
    x = min(x, dpp::mov_i<dpp::kRowShr2>(INT32_MAX, x));
    x = min(x, dpp::mov_i<dpp::kRowShr4>(INT32_MAX, x));
    x = min(x, dpp::mov_i<dpp::kRowShr8>(INT32_MAX, x));
    x = min(x, dpp::mov_i<dpp::kRowBcast15, 0xA>(INT32_MAX, x));
    x = min(x, dpp::mov_i<dpp::kRowBcast31, 0xC>(INT32_MAX, x));
    return wave_last_i(x);
}
__device__ __forceinline__ int wave_max_i(int x) {
    x = max(x, dpp::mov_i<dpp::kRowShr1>(INT32_MIN, x));
    x = max(x, dpp::mov_i<dpp::kRowShr2>(INT32_MIN, x));
    x = max(x, dpp::mov_i<dpp::kRowShr4>(INT32_MIN, x));
    x = max(x, dpp::mov_i<dpp::kRowShr8>(INT32_MIN, x));
    x = max(x, dpp::mov_i<dpp::kRowBcast15, 0xA>(INT32_MIN, x));
    x = max(x, dpp::mov_i<dpp::kRowBcast31, 0xC>(INT32_MIN, x));
    return wave_last_i(x);
}

// Exclusive prefix within the wavefront from an inclusive one (lane 0: 0).
__device__ __forceinline__ float wave_excl_from_incl(float incl) {
    return dpp::mov_f<dpp::kWaveShr1>(0.f, incl);
}

// Two workgroup sums at once, in a fixed order; every thread gets both.
__device__ __forceinline__ void wg_sum2(float a, float b, float &sa, float &sb) {
    __shared__ float s_t[2][kWaves];
    a = wave_last(wave_incl_sum(a));
    b = wave_last(wave_incl_sum(b));
    const int w = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) {
        s_t[0][w] = a;
        s_t[1][w] = b;
    }
    __syncthreads();
    sa = s_t[0][0];
    sb = s_t[1][0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) {
        sa += s_t[0][k];
        sb += s_t[1][k];
    }
}

// Two exclusive prefix sums over the workgroup's threads in thread order,
// with both totals; every thread gets the totals.  One barrier.
__device__ __forceinline__ void wg_excl_scan2(float a, float b, float &ea, float &eb, float &ta,
                                              float &tb) {
    __shared__ float s_t[2][kWaves];
    const float ia = wave_incl_sum(a), ib = wave_incl_sum(b);
    const int w = threadIdx.x / kWave;
    if (threadIdx.x % kWave == kWave - 1) {
        s_t[0][w] = ia;
        s_t[1][w] = ib;
    }
    __syncthreads();
    float ba = 0.f, bb = 0.f;
    ta = 0.f;
    tb = 0.f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
        if (k == w) {
            ba = ta;
            bb = tb;
        }
        ta += s_t[0][k];
        tb += s_t[1][k];
    }
    ea = ba + wave_excl_from_incl(ia);
    eb = bb + wave_excl_from_incl(ib);
}

// Workgroup minimum of one int and maximum of another; every thread gets both.
__device__ __forceinline__ void wg_min_max(int mn, int mx, int &rmin, int &rmax) {
    __shared__ int s_t[2][kWaves];
    mn = wave_min_i(mn);
    mx = wave_max_i(mx);
    const int w = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) {
        s_t[0][w] = mn;
        s_t[1][w] = mx;
    }
    __syncthreads();
    rmin = s_t[0][0];
    rmax = s_t[1][0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) {
        rmin = min(rmin, s_t[0][k]);
        rmax = max(rmax, s_t[1][k]);
    }
}

// Merge of (ref, z) on DPP moves in a fixed order.  The row form merges each
// row of 16 lanes (result valid in the row's last lane); the wavefront form
// continues across rows (result valid in lane 63, read it with wave_last).
#define SV_MZ_STEP(CTRL, MASK)                                                   \
    {                                                                            \
        const float r2 = dpp::mov_f<CTRL, MASK>(-INFINITY, ref);                \
        const float z2 = dpp::mov_f<CTRL, MASK>(0.f, z);                        \
        mz_merge(ref, z, r2, z2);                                                \
    }
__device__ __forceinline__ void mz_row_merge(float &ref, float &z) {
    SV_MZ_STEP(dpp::kRowShr1, 0xF)
    SV_MZ_STEP(dpp::kRowShr2, 0xF)
    SV_MZ_STEP(dpp::kRowShr4, 0xF)
    SV_MZ_STEP(dpp::kRowShr8, 0xF)
}
__device__ __forceinline__ void mz_wave_merge(float &ref, float &z) {
    mz_row_merge(ref, z);
    SV_MZ_STEP(dpp::kRowBcast15, 0xA)
    SV_MZ_STEP(dpp::kRowBcast31, 0xC)
}
#define SV_MZ_STEP_D(CTRL, MASK)                                                 \
    {                                                                            \
        const float r2 = dpp::mov_f<CTRL, MASK>(-INFINITY, ref);                \
        const double z2 = dpp::mov_d<CTRL, MASK>(0.0, z);                       \
        mz_merge_d(ref, z, r2, z2);                                              \
    }
__device__ __forceinline__ void mz_row_merge_d(float &ref, double &z) {
    SV_MZ_STEP_D(dpp::kRowShr1, 0xF)
    SV_MZ_STEP_D(dpp::kRowShr2, 0xF)
    SV_MZ_STEP_D(dpp::kRowShr4, 0xF)
    SV_MZ_STEP_D(dpp::kRowShr8, 0xF)
}
__device__ __forceinline__ void mz_wave_merge_d(float &ref, double &z) {
    mz_row_merge_d(ref, z);
    SV_MZ_STEP_D(dpp::kRowBcast15, 0xA)
    SV_MZ_STEP_D(dpp::kRowBcast31, 0xC)
}
#undef SV_MZ_STEP_D
#undef SV_MZ_STEP

__device__ __forceinline__ void mz_reduce_wg(float &ref, float &z) {
    __shared__ float s_ref[kWaves], s_z[kWaves];
    mz_wave_merge(ref, z);
    const int w = threadIdx.x / kWave;
    if (threadIdx.x % kWave == kWave - 1) {
        s_ref[w] = ref;
        s_z[w] = z;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        ref = s_ref[0];
        z = s_z[0];
        for (int i = 1; i < kWaves; ++i) mz_merge(ref, z, s_ref[i], s_z[i]);
    }
}


// Maximum over the wavefront (uniform result).
__device__ __forceinline__ float wave_max_f(float x) {
    x = fmaxf(x, dpp::mov_f<dpp::kRowShr1>(-INFINITY, x));
    x = fmaxf(x, dpp::mov_f<dpp::kRowShr2>(-INFINITY, x));
    x = fmaxf(x, dpp::mov_f<dpp::kRowShr4>(-INFINITY, x));
    x = fmaxf(x, dpp::mov_f<dpp::kRowShr8>(-INFINITY, x));
    x = fmaxf(x, dpp::mov_f<dpp::kRowBcast15, 0xA>(-INFINITY, x));
    x = fmaxf(x, dpp::mov_f<dpp::kRowBcast31, 0xC>(-INFINITY, x));
    return wave_last(x);
}

// Softmax statistics of N logits per thread over the workgroup, valid in
// thread 0.  Every wavefront takes its largest logit as the reference, so
// each logit costs one exp2 and no rescaling; the four wavefronts' (ref, z)
// are then merged in order by thread 0.
template <int N>
__device__ __forceinline__ void mz_chunk_wg(const float *x, float c, float &ref, float &z) {
    __shared__ float s_ref[kWaves];
    __shared__ double s_z[kWaves];
    float m = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) m = fmaxf(m, x[i]);
    const float rw = wave_max_f(m) * c;
    const float r = rw == -INFINITY ? 0.f : rw;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < N; ++i) s[i & 3] += exp2_hw(fmaf(x[i], c, -r));
    const double zw =
        wave_last_d(wave_incl_sum_d(static_cast<double>((s[0] + s[1]) + (s[2] + s[3]))));
    const int w = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) {
        s_ref[w] = rw;
        s_z[w] = zw;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        ref = s_ref[0];
        double zd = s_z[0];
        for (int i = 1; i < kWaves; ++i) mz_merge_d(ref, zd, s_ref[i], s_z[i]);
        z = static_cast<float>(zd);
    }
}

}  // namespace sv
