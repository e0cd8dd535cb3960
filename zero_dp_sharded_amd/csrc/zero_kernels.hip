// gfx950 kernels of the owner-rank ZeRO-DP step.
//
// Everything here is HBM-bound elementwise streaming (about 0.5 flop per byte
// against a ridge near 20), so there is no MFMA and no LDS staging of data:
// each lane moves 16-byte vectors (8 two-byte values, or 2 x 4 fp32 values),
// the loads of one vector run are all issued before their arithmetic, and the
// only cross-lane work is the fixed-shape reduction of the overflow flag and
// the squared gradient norm (wave butterfly, then one LDS slot per wave).
//
// Floating point: built with -ffp-contract=off, correctly rounded fp32 divide
// and square root, fp32 denormals kept, and packed-fp32 instructions disabled.
// Every per-element operation therefore rounds to nearest even exactly once,
// in the order written.

#include "zero_kernels.h"

namespace zk {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

template <int LP> struct Fmt;
template <> struct Fmt<1> {            // IEEE binary16
    using T = _Float16;
    using V = h8;
    static constexpr unsigned short kExp = 0x7c00;
};
template <> struct Fmt<2> {            // bfloat16
    using T = __bf16;
    using V = b8;
    static constexpr unsigned short kExp = 0x7f80;
};

template <int LP>
__device__ __forceinline__ typename Fmt<LP>::V load_v(const void* base, int64_t e)
{
    using F = Fmt<LP>;
    return *reinterpret_cast<const typename F::V*>(static_cast<const typename F::T*>(base) + e);
}

template <int LP>
__device__ __forceinline__ void store_v(void* base, int64_t e, typename Fmt<LP>::V x)
{
    using F = Fmt<LP>;
    *reinterpret_cast<typename F::V*>(static_cast<typename F::T*>(base) + e) = x;
}

template <int LP>
__device__ __forceinline__ float load_s(const void* base, int64_t e)
{
    using F = Fmt<LP>;
    return static_cast<float>(static_cast<const typename F::T*>(base)[e]);
}

// Overflow flag and squared unscaled norm of stored 2-byte values.
template <int LP>
__device__ __forceinline__ void check_v(typename Fmt<LP>::V o, float inv_scale, int& flag,
                                        double& ss)
{
    using F = Fmt<LP>;
    u16x8 bits = __builtin_bit_cast(u16x8, o);
    f8 of = __builtin_convertvector(o, f8);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        flag |= (bits[k] & F::kExp) == F::kExp;
        float u = of[k] * inv_scale;
        ss += (double)u * (double)u;
    }
}

template <int LP>
__device__ __forceinline__ void check_s(typename Fmt<LP>::T o, float inv_scale, int& flag,
                                        double& ss)
{
    using F = Fmt<LP>;
    unsigned short bits = __builtin_bit_cast(unsigned short, o);
    flag |= (bits & F::kExp) == F::kExp;
    float u = static_cast<float>(o) * inv_scale;
    ss += (double)u * (double)u;
}

// Reduce of one 8-element run: fp32 sum over r in ascending order from +0,
// times fp32(1/R), rounded to the 2-byte format.
template <int LP, int RT>
__device__ __forceinline__ void reduce_v(const ReduceLaunch& L, int64_t e, int& flag, double& ss)
{
    using F = Fmt<LP>;
    using V = typename F::V;
    f8 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if constexpr (RT > 0) {
        V x[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) x[r] = load_v<LP>(L.c.p[r], e);
#pragma unroll
        for (int r = 0; r < RT; ++r) acc = acc + __builtin_convertvector(x[r], f8);
    } else {
        for (int r0 = 0; r0 < L.R; r0 += 8) {
            const int cnt = L.R - r0 < 8 ? L.R - r0 : 8;
            V x[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (k < cnt) x[k] = load_v<LP>(L.c.p[r0 + k], e);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (k < cnt) acc = acc + __builtin_convertvector(x[k], f8);
        }
    }
    acc = acc * L.inv_r;
    V o = __builtin_convertvector(acc, V);
    store_v<LP>(L.out, e, o);
    check_v<LP>(o, L.inv_scale, flag, ss);
}

template <int LP>
__device__ __forceinline__ void reduce_s(const ReduceLaunch& L, int64_t e, int& flag, double& ss)
{
    using F = Fmt<LP>;
    float acc = 0.f;
    for (int r = 0; r < L.R; ++r) acc = acc + load_s<LP>(L.c.p[r], e);
    typename F::T o = static_cast<typename F::T>(acc * L.inv_r);
    static_cast<typename F::T*>(L.out)[e] = o;
    check_s<LP>(o, L.inv_scale, flag, ss);
}

// Fold the lane values of a workgroup into its partial slot.  The shape of the
// reduction is fixed, so the result is bitwise reproducible.  On the first
// bucket of a step the slot is overwritten and the slots past the grid are
// cleared; later buckets add to them in stream order.
__device__ __forceinline__ void block_partial(double* ps, int32_t* pf, int first, int flag,
                                              double ss)
{
    __shared__ double sh_ss[kBlock / 64];
    __shared__ int sh_f[kBlock / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        ss += __shfl_xor(ss, off, 64);
        flag |= __shfl_xor(flag, off, 64);
    }
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    if (lane == 0) {
        sh_ss[w] = ss;
        sh_f[w] = flag;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = sh_ss[0];
        int f = sh_f[0];
#pragma unroll
        for (int k = 1; k < kBlock / 64; ++k) {
            s += sh_ss[k];
            f |= sh_f[k];
        }
        const int b = blockIdx.x;
        if (first) {
            ps[b] = s;
            pf[b] = f;
        } else {
            ps[b] += s;
            pf[b] |= f;
        }
    }
    if (first) {
        for (int k = gridDim.x + blockIdx.x * kBlock + threadIdx.x; k < kSlots;
             k += gridDim.x * kBlock) {
            ps[k] = 0.0;
            pf[k] = 0;
        }
    }
}

template <int LP, int RT>
__global__ __launch_bounds__(kBlock) void reduce_kernel(ReduceLaunch L)
{
    const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int flag = 0;
    double ss = 0.0;
    if (L.vec_ok) {
        for (int64_t v = gid; v < L.nvec; v += stride)
            reduce_v<LP, RT>(L, L.head + v * 8, flag, ss);
        const int64_t tail0 = L.head + L.nvec * 8;
        const int64_t nsc = L.head + (L.n - tail0);
        if (gid < nsc)
            reduce_s<LP>(L, gid < L.head ? gid : tail0 + (gid - L.head), flag, ss);
    } else {
        for (int64_t e = gid; e < L.n; e += stride) reduce_s<LP>(L, e, flag, ss);
    }
    block_partial(L.part_sumsq, L.part_flag, L.first, flag, ss);
}

template <int LP>
__global__ __launch_bounds__(kBlock) void scan_kernel(ScanLaunch L)
{
    using F = Fmt<LP>;
    const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int flag = 0;
    double ss = 0.0;
    if (L.vec_ok) {
        for (int64_t v = gid; v < L.nvec; v += stride)
            check_v<LP>(load_v<LP>(L.g, L.head + v * 8), L.inv_scale, flag, ss);
        const int64_t tail0 = L.head + L.nvec * 8;
        const int64_t nsc = L.head + (L.n - tail0);
        if (gid < nsc) {
            const int64_t e = gid < L.head ? gid : tail0 + (gid - L.head);
            check_s<LP>(static_cast<const typename F::T*>(L.g)[e], L.inv_scale, flag, ss);
        }
    } else {
        for (int64_t e = gid; e < L.n; e += stride)
            check_s<LP>(static_cast<const typename F::T*>(L.g)[e], L.inv_scale, flag, ss);
    }
    block_partial(L.part_sumsq, L.part_flag, 1, flag, ss);
}

// One workgroup sums the kSlots partials in a fixed order.
__global__ __launch_bounds__(kBlock) void finalize_kernel(const double* ps, const int32_t* pf,
                                                          CheckResult* out)
{
    double s = 0.0;
    int f = 0;
    for (int k = threadIdx.x; k < kSlots; k += kBlock) {
        s += ps[k];
        f |= pf[k];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        s += __shfl_xor(s, off, 64);
        f |= __shfl_xor(f, off, 64);
    }
    __shared__ double sh_s[kBlock / 64];
    __shared__ int sh_f[kBlock / 64];
    if ((threadIdx.x & 63) == 0) {
        sh_s[threadIdx.x >> 6] = s;
        sh_f[threadIdx.x >> 6] = f;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = sh_s[0];
        int g = sh_f[0];
        for (int k = 1; k < kBlock / 64; ++k) {
            t += sh_s[k];
            g |= sh_f[k];
        }
        out->sumsq = t;
        out->flag = g;
        out->pad = 0;
    }
}

// Textbook Adam on one element (Kingma & Ba 2015, Algorithm 1), in the order
// the public header states; p, m, v are updated in place.
template <int WD>
__device__ __forceinline__ void adam_e(float graw, float& p, float& m, float& v,
                                       const AdamLaunch& a)
{
    float g = graw * a.inv_scale;
    if constexpr (WD == kWdL2) g = g + a.wd * p;
    m = a.b1 * m + a.omb1 * g;
    v = a.b2 * v + a.omb2 * (g * g);
    const float mh = m / a.bc1;
    const float vh = v / a.bc2;
    float u = mh / (sqrtf(vh) + a.eps);
    if constexpr (WD == kWdDecoupled) u = u + a.wd * p;
    p = p - a.lr * u;
}

template <int LP, int WD>
__device__ __forceinline__ void adam_v(const AdamLaunch& a, int64_t e)
{
    using F = Fmt<LP>;
    using V = typename F::V;
    const V gv = load_v<LP>(a.grad, e);
    f4* mp = reinterpret_cast<f4*>(a.master + e);
    f4* m1p = reinterpret_cast<f4*>(a.m + e);
    f4* v2p = reinterpret_cast<f4*>(a.v + e);
    const f4 p0 = mp[0], p1 = mp[1];
    const f4 m0 = m1p[0], m1 = m1p[1];
    const f4 v0 = v2p[0], v1 = v2p[1];
    const f8 g = __builtin_convertvector(gv, f8);
    f8 p = __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7);
    f8 m = __builtin_shufflevector(m0, m1, 0, 1, 2, 3, 4, 5, 6, 7);
    f8 v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        float pk = p[k], mk = m[k], vk = v[k];
        adam_e<WD>(g[k], pk, mk, vk, a);
        p[k] = pk;
        m[k] = mk;
        v[k] = vk;
    }
    mp[0] = __builtin_shufflevector(p, p, 0, 1, 2, 3);
    mp[1] = __builtin_shufflevector(p, p, 4, 5, 6, 7);
    m1p[0] = __builtin_shufflevector(m, m, 0, 1, 2, 3);
    m1p[1] = __builtin_shufflevector(m, m, 4, 5, 6, 7);
    v2p[0] = __builtin_shufflevector(v, v, 0, 1, 2, 3);
    v2p[1] = __builtin_shufflevector(v, v, 4, 5, 6, 7);
    store_v<LP>(a.param, e, __builtin_convertvector(p, V));
}

template <int LP, int WD>
__device__ __forceinline__ void adam_s(const AdamLaunch& a, int64_t e)
{
    using F = Fmt<LP>;
    float p = a.master[e], m = a.m[e], v = a.v[e];
    adam_e<WD>(load_s<LP>(a.grad, e), p, m, v, a);
    a.master[e] = p;
    a.m[e] = m;
    a.v[e] = v;
    static_cast<typename F::T*>(a.param)[e] = static_cast<typename F::T>(p);
}

template <int LP, int WD>
__global__ __launch_bounds__(kBlock) void adam_kernel(AdamLaunch a)
{
    const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    if (a.vec_ok) {
        for (int64_t v = gid; v < a.nvec; v += stride) adam_v<LP, WD>(a, a.head + v * 8);
        const int64_t tail0 = a.head + a.nvec * 8;
        const int64_t nsc = a.head + (a.n - tail0);
        if (gid < nsc) adam_s<LP, WD>(a, gid < a.head ? gid : tail0 + (gid - a.head));
    } else {
        for (int64_t e = gid; e < a.n; e += stride) adam_s<LP, WD>(a, e);
    }
}

// Grid of a grid-stride launch: enough workgroups for `work` lane items,
// capped at `cap`, at least one.
inline unsigned grid_for(int64_t work, int64_t cap)
{
    int64_t g = (work + kBlock - 1) / kBlock;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (unsigned)g;
}

template <int LP>
hipError_t reduce_dispatch(const ReduceLaunch& L, unsigned grid, hipStream_t s)
{
    switch (L.vec_ok ? L.R : 0) {
    case 1: reduce_kernel<LP, 1><<<grid, kBlock, 0, s>>>(L); break;
    case 2: reduce_kernel<LP, 2><<<grid, kBlock, 0, s>>>(L); break;
    case 4: reduce_kernel<LP, 4><<<grid, kBlock, 0, s>>>(L); break;
    case 8: reduce_kernel<LP, 8><<<grid, kBlock, 0, s>>>(L); break;
    case 16: reduce_kernel<LP, 16><<<grid, kBlock, 0, s>>>(L); break;
    default: reduce_kernel<LP, 0><<<grid, kBlock, 0, s>>>(L); break;
    }
    return hipGetLastError();
}

template <int LP>
hipError_t adam_dispatch(const AdamLaunch& a, unsigned grid, hipStream_t s)
{
    switch (a.wd_kind) {
    case kWdDecoupled: adam_kernel<LP, kWdDecoupled><<<grid, kBlock, 0, s>>>(a); break;
    case kWdL2: adam_kernel<LP, kWdL2><<<grid, kBlock, 0, s>>>(a); break;
    default: adam_kernel<LP, kWdNone><<<grid, kBlock, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const ReduceLaunch& L, hipStream_t s)
{
    const int64_t work = L.vec_ok ? (L.nvec > 16 ? L.nvec : 16) : L.n;
    const unsigned grid = grid_for(work, kSlots);
    return L.lp == 2 ? reduce_dispatch<2>(L, grid, s) : reduce_dispatch<1>(L, grid, s);
}

hipError_t launch_scan(const ScanLaunch& L, hipStream_t s)
{
    const int64_t work = L.vec_ok ? (L.nvec > 16 ? L.nvec : 16) : L.n;
    const unsigned grid = grid_for(work, kSlots);
    if (L.lp == 2)
        scan_kernel<2><<<grid, kBlock, 0, s>>>(L);
    else
        scan_kernel<1><<<grid, kBlock, 0, s>>>(L);
    return hipGetLastError();
}

hipError_t launch_finalize(const double* ps, const int32_t* pf, CheckResult* out, hipStream_t s)
{
    finalize_kernel<<<1, kBlock, 0, s>>>(ps, pf, out);
    return hipGetLastError();
}

hipError_t launch_adam(const AdamLaunch& a, hipStream_t s)
{
    const int64_t work = a.vec_ok ? (a.nvec > 16 ? a.nvec : 16) : a.n;
    const unsigned grid = grid_for(work, int64_t(1) << 20);
    return a.lp == 2 ? adam_dispatch<2>(a, grid, s) : adam_dispatch<1>(a, grid, s);
}

}  // namespace zk
