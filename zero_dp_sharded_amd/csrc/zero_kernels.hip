// gfx950 kernels of the owner-rank ZeRO-DP step.
//
// Everything here is HBM-bound elementwise streaming (about 0.5 flop per byte
// against a ridge near 20), so there is no MFMA and no LDS staging of data.
// The shapes were chosen by measurement on MI355X:
//  - one tile per lane on an exact grid (no grid-stride loop): the workgroups
//    in flight then sweep each array as one narrow front, which keeps DRAM
//    row locality; grid-stride launches lost about 15 points of bandwidth;
//  - every load and store instruction of a wave covers one contiguous span
//    (lane-consecutive 16-byte or 8-byte pieces);
//  - nontemporal loads and stores (each byte is touched once per step);
//  - a cap on resident workgroups per CU, set by reserving dynamic LDS the
//    kernels never touch: with the 5 to 7 concurrent streams of these kernels,
//    fewer resident waves (8 per CU for Adam, 16 for the reduce) sustain more
//    HBM bandwidth than full occupancy.
// The only cross-lane work is the fixed-shape reduction of the overflow flag
// and the squared gradient norm: wave butterfly, one LDS slot per wave, one
// fp64 partial per workgroup, then a fixed-order two-level fold.
//
// Floating point: built with -ffp-contract=off, correctly rounded fp32 divide
// and square root, fp32 denormals kept, and packed-fp32 instructions disabled.
// Every per-element operation rounds to nearest even exactly once, in the
// order written.

#include "zero_kernels.h"

namespace zk {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef __bf16 b4 __attribute__((ext_vector_type(4)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

template <int LP> struct Fmt;
template <> struct Fmt<1> {            // IEEE binary16
    using T = _Float16;
    using V8 = h8;
    using V4 = h4;
    static constexpr unsigned short kExp = 0x7c00;
};
template <> struct Fmt<2> {            // bfloat16
    using T = __bf16;
    using V8 = b8;
    using V4 = b4;
    static constexpr unsigned short kExp = 0x7f80;
};

template <typename V>
__device__ __forceinline__ V ld_nt(const void* base, int64_t idx)
{
    return __builtin_nontemporal_load(static_cast<const V*>(base) + idx);
}

template <typename V>
__device__ __forceinline__ void st_nt(void* base, int64_t idx, V x)
{
    __builtin_nontemporal_store(x, static_cast<V*>(base) + idx);
}

template <int LP>
__device__ __forceinline__ float load_s(const void* base, int64_t e)
{
    return static_cast<float>(static_cast<const typename Fmt<LP>::T*>(base)[e]);
}

// ----------------------------------------------------------------- check

// Overflow flag and squared unscaled norm of stored 2-byte values.
template <int LP>
__device__ __forceinline__ void check_v(typename Fmt<LP>::V8 o, float inv_scale, int& flag,
                                        double& ss)
{
    using F = Fmt<LP>;
    const u16x8 bits = __builtin_bit_cast(u16x8, o);
    const f8 of = __builtin_convertvector(o, f8);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        flag |= (bits[k] & F::kExp) == F::kExp;
        const float u = of[k] * inv_scale;
        ss += (double)u * (double)u;
    }
}

template <int LP>
__device__ __forceinline__ void check_s(typename Fmt<LP>::T o, float inv_scale, int& flag,
                                        double& ss)
{
    using F = Fmt<LP>;
    const unsigned short bits = __builtin_bit_cast(unsigned short, o);
    flag |= (bits & F::kExp) == F::kExp;
    const float u = static_cast<float>(o) * inv_scale;
    ss += (double)u * (double)u;
}

// One fp64 partial per workgroup: the sum of its lanes' squares, or NaN when
// any lane saw a non-finite stored value.  Fixed reduction shape, so the
// value is bitwise reproducible.
template <int BS>
__device__ __forceinline__ void block_partial(double* slot, int flag, double ss)
{
    __shared__ double sh_ss[BS / 64];
    __shared__ int sh_f[BS / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        ss += __shfl_xor(ss, off, 64);
        flag |= __shfl_xor(flag, off, 64);
    }
    if ((threadIdx.x & 63) == 0) {
        sh_ss[threadIdx.x >> 6] = ss;
        sh_f[threadIdx.x >> 6] = flag;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = sh_ss[0];
        int f = sh_f[0];
#pragma unroll
        for (int k = 1; k < BS / 64; ++k) {
            s += sh_ss[k];
            f |= sh_f[k];
        }
        *slot = f ? __builtin_nan("") : s;
    }
}

// ----------------------------------------------------------------- element lists

// The element-wise kernels walk a list of at most two index ranges: the
// unaligned head [0, a_len) and the tail [b_start, b_start + b_len) of a
// vector layout, or the whole array as range a.
struct Ranges {
    int64_t a_len;
    int64_t b_start;
    int64_t b_len;
    __device__ __forceinline__ int64_t count() const { return a_len + b_len; }
    __device__ __forceinline__ int64_t at(int64_t k) const
    {
        return k < a_len ? k : b_start + (k - a_len);
    }
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ----------------------------------------------------------------- reduce

// Finish the 8-element run vi of the vector body (elements head + 8 vi ..):
// acc holds the fp32 sum over r = 0..R-1 in order from +0; scale by
// fp32(1/R), round to the 2-byte format, store, check.
template <int LP>
__device__ __forceinline__ void reduce_finish(const ReduceLaunch& L, int64_t vi, f8 acc, int& flag,
                                              double& ss)
{
    using V8 = typename Fmt<LP>::V8;
    acc = acc * L.inv_r;
    const V8 o = __builtin_convertvector(acc, V8);
    st_nt<V8>(static_cast<char*>(L.out) + 2 * L.head, vi, o);
    check_v<LP>(o, L.inv_scale, flag, ss);
}

template <int LP>
__device__ __forceinline__ void reduce_s(const ReduceLaunch& L, int64_t e, int& flag, double& ss)
{
    using T = typename Fmt<LP>::T;
    float acc = 0.f;
    for (int r = 0; r < L.R; ++r) acc = acc + load_s<LP>(L.c.p[r], e);
    const T o = static_cast<T>(acc * L.inv_r);
    static_cast<T*>(L.out)[e] = o;
    check_s<LP>(o, L.inv_scale, flag, ss);
}

// Vector body: workgroup b covers runs [b*B*U, (b+1)*B*U) for B lanes and U
// runs per lane; lane l owns runs b*B*U + u*B + l.  Element offsets past `head`
// are multiples of 8, so contribution and output pointers advanced by `head`
// are 16-byte aligned and are indexed in units of 8 elements.
template <int LP, int RT>
__global__ __launch_bounds__(kRedBlock) void reduce_vec_kernel(ReduceLaunch L)
{
    using V8 = typename Fmt<LP>::V8;
    int flag = 0;
    double ss = 0.0;
    const int64_t v0 = (int64_t)blockIdx.x * (kRedBlock * kRedRuns) + threadIdx.x;
    if constexpr (RT > 0 && RT * kRedRuns <= 16) {
        // every load of both runs in flight before the arithmetic
        V8 x[kRedRuns][RT];
#pragma unroll
        for (int u = 0; u < kRedRuns; ++u) {
            const int64_t vi = v0 + u * kRedBlock;
            if (vi < L.nvec) {
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    x[u][r] = ld_nt<V8>(static_cast<const char*>(L.c.p[r]) + 2 * L.head, vi);
            }
        }
#pragma unroll
        for (int u = 0; u < kRedRuns; ++u) {
            const int64_t vi = v0 + u * kRedBlock;
            if (vi < L.nvec) {
                f8 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < RT; ++r) acc = acc + __builtin_convertvector(x[u][r], f8);
                reduce_finish<LP>(L, vi, acc, flag, ss);
            }
        }
    } else {
        for (int u = 0; u < kRedRuns; ++u) {
            const int64_t vi = v0 + u * kRedBlock;
            if (vi >= L.nvec) break;
            f8 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if constexpr (RT > 0) {
                V8 x[RT];
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    x[r] = ld_nt<V8>(static_cast<const char*>(L.c.p[r]) + 2 * L.head, vi);
#pragma unroll
                for (int r = 0; r < RT; ++r) acc = acc + __builtin_convertvector(x[r], f8);
            } else {
                for (int r0 = 0; r0 < L.R; r0 += 8) {
                    const int cnt = L.R - r0 < 8 ? L.R - r0 : 8;
                    V8 x[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        if (k < cnt)
                            x[k] = ld_nt<V8>(static_cast<const char*>(L.c.p[r0 + k]) + 2 * L.head, vi);
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        if (k < cnt) acc = acc + __builtin_convertvector(x[k], f8);
                }
            }
            reduce_finish<LP>(L, vi, acc, flag, ss);
        }
    }
    block_partial<kRedBlock>(L.partial + L.slot_base + blockIdx.x, flag, ss);
}

template <int LP>
__global__ __launch_bounds__(kScalarBlock) void reduce_elem_kernel(ReduceLaunch L, Ranges rg,
                                                                    int64_t slot)
{
    int flag = 0;
    double ss = 0.0;
    const int64_t cnt = rg.count();
#pragma unroll 2
    for (int j = 0; j < (int)(kScalarElemsPerBlock / kScalarBlock); ++j) {
        const int64_t k = (int64_t)blockIdx.x * kScalarElemsPerBlock + j * kScalarBlock + threadIdx.x;
        if (k < cnt) reduce_s<LP>(L, rg.at(k), flag, ss);
    }
    block_partial<kScalarBlock>(L.partial + slot + blockIdx.x, flag, ss);
}

template <int LP>
__global__ __launch_bounds__(kRedBlock) void scan_vec_kernel(ScanLaunch L)
{
    using V8 = typename Fmt<LP>::V8;
    int flag = 0;
    double ss = 0.0;
    const int64_t v0 = (int64_t)blockIdx.x * (kRedBlock * kRedRuns) + threadIdx.x;
    V8 x[kRedRuns];
#pragma unroll
    for (int u = 0; u < kRedRuns; ++u) {
        const int64_t vi = v0 + u * kRedBlock;
        if (vi < L.nvec) x[u] = ld_nt<V8>(static_cast<const char*>(L.g) + 2 * L.head, vi);
    }
#pragma unroll
    for (int u = 0; u < kRedRuns; ++u)
        if (v0 + u * kRedBlock < L.nvec) check_v<LP>(x[u], L.inv_scale, flag, ss);
    block_partial<kRedBlock>(L.partial + L.slot_base + blockIdx.x, flag, ss);
}

template <int LP>
__global__ __launch_bounds__(kScalarBlock) void scan_elem_kernel(ScanLaunch L, Ranges rg,
                                                                  int64_t slot)
{
    using T = typename Fmt<LP>::T;
    int flag = 0;
    double ss = 0.0;
    const int64_t cnt = rg.count();
    for (int j = 0; j < (int)(kScalarElemsPerBlock / kScalarBlock); ++j) {
        const int64_t k = (int64_t)blockIdx.x * kScalarElemsPerBlock + j * kScalarBlock + threadIdx.x;
        if (k < cnt) check_s<LP>(static_cast<const T*>(L.g)[rg.at(k)], L.inv_scale, flag, ss);
    }
    block_partial<kScalarBlock>(L.partial + slot + blockIdx.x, flag, ss);
}

// Workgroup b sums in[b*chunk, min(n, (b+1)*chunk)) with a fixed shape.
__global__ __launch_bounds__(kFoldBlock) void fold_kernel(const double* in, int64_t n, int64_t chunk,
                                                          double* out)
{
    const int64_t lo = (int64_t)blockIdx.x * chunk;
    const int64_t hi = lo + chunk < n ? lo + chunk : n;
    double s = 0.0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += kFoldBlock) s += in[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    __shared__ double sh[kFoldBlock / 64];
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = sh[0];
#pragma unroll
        for (int k = 1; k < kFoldBlock / 64; ++k) t += sh[k];
        out[blockIdx.x] = t;
    }
}

// ----------------------------------------------------------------- Adam

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

// Vector body: groups of 4 elements past `head` (fp32 pointers advanced by
// head are 16-byte aligned, 2-byte pointers 8-byte aligned).  Workgroup b
// covers groups [b*B*G, (b+1)*B*G) for B lanes and G groups per lane; lane l
// owns groups b*B*G + u*B + l, u < G, and issues all loads before any
// arithmetic.
// Device-side skip of a gated launch: the fold leaves NaN in the result when
// any stored gradient is not finite.  The vector kernel reads the gate after
// issuing its loads (a skipped step then costs the 14 load bytes per element
// but writes nothing); the element-wise kernel reads it first.
__device__ __forceinline__ bool gated_off(const AdamLaunch& a)
{
    return a.gate != nullptr && __builtin_isnan(a.gate->sumsq);
}

template <int LP, int WD>
__global__ __launch_bounds__(kAdamBlock) void adam_vec_kernel(AdamLaunch a)
{
    using V4 = typename Fmt<LP>::V4;
    const void* gb = static_cast<const char*>(a.grad) + 2 * a.head;
    void* qb = static_cast<char*>(a.param) + 2 * a.head;
    float* pb = a.master + a.head;
    float* mb = a.m + a.head;
    float* vb = a.v + a.head;
    const int64_t q0 = (int64_t)blockIdx.x * (kAdamBlock * kAdamGroups) + threadIdx.x;
    V4 g[kAdamGroups];
    f4 p[kAdamGroups], m[kAdamGroups], v[kAdamGroups];
#pragma unroll
    for (int u = 0; u < kAdamGroups; ++u) {
        const int64_t q = q0 + u * kAdamBlock;
        if (q < a.ngroups) {
            g[u] = ld_nt<V4>(gb, q);
            p[u] = ld_nt<f4>(pb, q);
            m[u] = ld_nt<f4>(mb, q);
            v[u] = ld_nt<f4>(vb, q);
        }
    }
    // The gate is read after the loads are issued, so its latency overlaps
    // them; on a skipped step the workgroup returns before any store.
    if (gated_off(a)) return;
#pragma unroll
    for (int u = 0; u < kAdamGroups; ++u) {
        const int64_t q = q0 + u * kAdamBlock;
        if (q < a.ngroups) {
            const f4 gf = __builtin_convertvector(g[u], f4);
            f4 pp = p[u], mm = m[u], vv = v[u];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float pk = pp[k], mk = mm[k], vk = vv[k];
                adam_e<WD>(gf[k], pk, mk, vk, a);
                pp[k] = pk;
                mm[k] = mk;
                vv[k] = vk;
            }
            st_nt<f4>(pb, q, pp);
            st_nt<f4>(mb, q, mm);
            st_nt<f4>(vb, q, vv);
            st_nt<V4>(qb, q, __builtin_convertvector(pp, V4));
        }
    }
}

template <int LP, int WD>
__global__ __launch_bounds__(kScalarBlock) void adam_elem_kernel(AdamLaunch a, Ranges rg)
{
    using T = typename Fmt<LP>::T;
    if (gated_off(a)) return;
    const int64_t cnt = rg.count();
    for (int j = 0; j < (int)(kScalarElemsPerBlock / kScalarBlock); ++j) {
        const int64_t k = (int64_t)blockIdx.x * kScalarElemsPerBlock + j * kScalarBlock + threadIdx.x;
        if (k < cnt) {
            const int64_t e = rg.at(k);
            float p = a.master[e], m = a.m[e], v = a.v[e];
            adam_e<WD>(load_s<LP>(a.grad, e), p, m, v, a);
            a.master[e] = p;
            a.m[e] = m;
            a.v[e] = v;
            static_cast<T*>(a.param)[e] = static_cast<T>(p);
        }
    }
}

// Element lists of a layout: head and tail of the vector path, or everything.
Ranges ranges_of(int64_t n, int64_t head, int64_t body, int32_t vec_ok)
{
    Ranges rg;
    if (!vec_ok) {
        rg.a_len = n;
        rg.b_start = n;
        rg.b_len = 0;
    } else {
        rg.a_len = head;
        rg.b_start = head + body;
        rg.b_len = n - (head + body);
    }
    return rg;
}

template <int LP>
hipError_t reduce_vec_launch(const ReduceLaunch& L, unsigned grid, hipStream_t s)
{
    const unsigned lds = L.lds_reserve;
    switch (L.R) {
    case 1: reduce_vec_kernel<LP, 1><<<grid, kRedBlock, lds, s>>>(L); break;
    case 2: reduce_vec_kernel<LP, 2><<<grid, kRedBlock, lds, s>>>(L); break;
    case 4: reduce_vec_kernel<LP, 4><<<grid, kRedBlock, lds, s>>>(L); break;
    case 8: reduce_vec_kernel<LP, 8><<<grid, kRedBlock, lds, s>>>(L); break;
    case 16: reduce_vec_kernel<LP, 16><<<grid, kRedBlock, lds, s>>>(L); break;
    default: reduce_vec_kernel<LP, 0><<<grid, kRedBlock, lds, s>>>(L); break;
    }
    return hipGetLastError();
}

template <int LP>
hipError_t reduce_dispatch(const ReduceLaunch& L, hipStream_t s)
{
    const int64_t runs_per_block = (int64_t)kRedBlock * kRedRuns;
    const int64_t vblocks = L.vec_ok ? ceil_div(L.nvec, runs_per_block) : 0;
    // consecutive launches of at most kMaxLaunchItems work-items; each starts
    // its runs and its partial slots where the previous one stopped
    const int64_t max_blocks = kMaxLaunchItems / kRedBlock;
    for (int64_t b0 = 0; b0 < vblocks; b0 += max_blocks) {
        const int64_t nb = vblocks - b0 < max_blocks ? vblocks - b0 : max_blocks;
        ReduceLaunch part = L;
        part.head = L.head + 8 * runs_per_block * b0;
        part.nvec = L.nvec - runs_per_block * b0;
        part.slot_base = L.slot_base + b0;
        hipError_t e = reduce_vec_launch<LP>(part, (unsigned)nb, s);
        if (e != hipSuccess) return e;
    }
    const Ranges rg = ranges_of(L.n, L.head, 8 * L.nvec, L.vec_ok);
    const int64_t sblocks = ceil_div(rg.a_len + rg.b_len, kScalarElemsPerBlock);
    if (sblocks > 0)
        reduce_elem_kernel<LP><<<(unsigned)sblocks, kScalarBlock, 0, s>>>(L, rg, L.slot_base + vblocks);
    return hipGetLastError();
}

template <int LP, int WD>
hipError_t adam_dispatch(const AdamLaunch& a, hipStream_t s)
{
    const int64_t groups_per_block = (int64_t)kAdamBlock * kAdamGroups;
    const int64_t vblocks = a.vec_ok ? ceil_div(a.ngroups, groups_per_block) : 0;
    const int64_t max_blocks = kMaxLaunchItems / kAdamBlock;
    for (int64_t b0 = 0; b0 < vblocks; b0 += max_blocks) {
        const int64_t nb = vblocks - b0 < max_blocks ? vblocks - b0 : max_blocks;
        AdamLaunch part = a;
        part.head = a.head + 4 * groups_per_block * b0;
        part.ngroups = a.ngroups - groups_per_block * b0;
        adam_vec_kernel<LP, WD><<<(unsigned)nb, kAdamBlock, a.lds_reserve, s>>>(part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const Ranges rg = ranges_of(a.n, a.head, 4 * a.ngroups, a.vec_ok);
    const int64_t sblocks = ceil_div(rg.a_len + rg.b_len, kScalarElemsPerBlock);
    if (sblocks > 0) adam_elem_kernel<LP, WD><<<(unsigned)sblocks, kScalarBlock, 0, s>>>(a, rg);
    return hipGetLastError();
}

template <int LP>
hipError_t adam_dispatch_wd(const AdamLaunch& a, hipStream_t s)
{
    switch (a.wd_kind) {
    case kWdDecoupled: return adam_dispatch<LP, kWdDecoupled>(a, s);
    case kWdL2: return adam_dispatch<LP, kWdL2>(a, s);
    default: return adam_dispatch<LP, kWdNone>(a, s);
    }
}

template <int LP>
hipError_t scan_dispatch(const ScanLaunch& L, hipStream_t s)
{
    const int64_t runs_per_block = (int64_t)kRedBlock * kRedRuns;
    const int64_t vblocks = L.vec_ok ? ceil_div(L.nvec, runs_per_block) : 0;
    const int64_t max_blocks = kMaxLaunchItems / kRedBlock;
    for (int64_t b0 = 0; b0 < vblocks; b0 += max_blocks) {
        const int64_t nb = vblocks - b0 < max_blocks ? vblocks - b0 : max_blocks;
        ScanLaunch part = L;
        part.head = L.head + 8 * runs_per_block * b0;
        part.nvec = L.nvec - runs_per_block * b0;
        part.slot_base = L.slot_base + b0;
        scan_vec_kernel<LP><<<(unsigned)nb, kRedBlock, L.lds_reserve, s>>>(part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const Ranges rg = ranges_of(L.n, L.head, 8 * L.nvec, L.vec_ok);
    const int64_t sblocks = ceil_div(rg.a_len + rg.b_len, kScalarElemsPerBlock);
    if (sblocks > 0)
        scan_elem_kernel<LP><<<(unsigned)sblocks, kScalarBlock, 0, s>>>(L, rg, L.slot_base + vblocks);
    return hipGetLastError();
}

}  // namespace

int64_t reduce_blocks(int64_t n, int64_t head, int64_t nvec, int32_t vec_ok)
{
    const int64_t vblocks = vec_ok ? ceil_div(nvec, (int64_t)kRedBlock * kRedRuns) : 0;
    const int64_t scalars = vec_ok ? n - 8 * nvec : n;
    return vblocks + ceil_div(scalars, kScalarElemsPerBlock);
}

hipError_t launch_reduce(const ReduceLaunch& L, hipStream_t s)
{
    return L.lp == 2 ? reduce_dispatch<2>(L, s) : reduce_dispatch<1>(L, s);
}

hipError_t launch_scan(const ScanLaunch& L, hipStream_t s)
{
    return L.lp == 2 ? scan_dispatch<2>(L, s) : scan_dispatch<1>(L, s);
}

hipError_t launch_finalize(const double* partial, int64_t nslots, double* level1,
                           CheckResult* out, hipStream_t s)
{
    int64_t g1 = ceil_div(nslots, 1024);
    if (g1 < 1) g1 = 1;
    if (g1 > kFoldMaxBlocks) g1 = kFoldMaxBlocks;
    const int64_t chunk = ceil_div(nslots, g1);
    fold_kernel<<<(unsigned)g1, kFoldBlock, 0, s>>>(partial, nslots, chunk, level1);
    fold_kernel<<<1, kFoldBlock, 0, s>>>(level1, g1, g1, &out->sumsq);
    return hipGetLastError();
}

hipError_t launch_adam(const AdamLaunch& a, hipStream_t s)
{
    return a.lp == 2 ? adam_dispatch_wd<2>(a, s) : adam_dispatch_wd<1>(a, s);
}

}  // namespace zk
