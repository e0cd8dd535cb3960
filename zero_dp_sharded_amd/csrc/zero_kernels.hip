// gfx950 kernels of the owner-rank ZeRO-DP step.
//
// Everything here is HBM-bound elementwise streaming (about 0.5 flop per byte
// against a ridge near 20), so there is no MFMA and no LDS staging of data.
// The shapes were chosen by measurement on MI355X:
//  - one tile per lane on an exact grid (no grid-stride loop): the workgroups
//    in flight then sweep each array as one narrow front, which keeps DRAM
//    row locality; grid-stride launches lost about 15 points of bandwidth;
//  - every load and store instruction of a wave covers one contiguous span
//    (lane-consecutive 16-byte runs, or the 8-byte groups of four 2-byte
//    values of the update);
//  - nontemporal loads and stores (each byte is touched once per step), but
//    for the one word per wave of 2-byte data that the shift reduce reads
//    twice (the next workgroup of its XCD reads the same line): cached, and
//    issued first;
//  - a cap on resident workgroups per CU, set by reserving dynamic LDS the
//    kernels never touch: with the 3 to 17 concurrent streams of the update
//    and reduce kernels, fewer resident waves (10 per CU for Adam, 16 or 24
//    for SGD, 6 to 12 for the reduce, 12 to 16 for the shift reduce) sustain
//    more HBM bandwidth than full occupancy; the one-stream scan keeps 32
//    waves with 4 runs per lane;
//  - in the reduce, loads issued in measured groups (a run of up to 8
//    contributions in groups of 4, several runs one run at a time), each group
//    ahead of its arithmetic;
//  - shards of at most 8M elements, whose step fits the caches, instead run
//    256-lane workgroups with one run or group per lane and plain (cached)
//    loads and stores in every bucket reduce and in the update.
// Cross-lane work: the shift reduce takes each lane's next 16-byte word from
// the neighbouring lane (DPP); the overflow flag and the squared gradient norm
// go through a fixed-shape reduction: wave butterfly, one LDS slot per wave,
// one fp64 partial per workgroup, then a fixed-order fold of one or two levels
// whose last lane also computes the clipping coefficient and, in the
// device-resident flow, decides the step.  A device-resident step of at most
// 1024 partials has no fold launch: every update workgroup repeats the fold in
// the same order and takes the same decision (see InlineFold).
//
// Storage formats: fp16 and bf16 (2-byte grads and params beside the fp32
// master copy) and fp32 (4-byte grads; the fp32 master is the parameter and
// no low-precision copy is written).  A 16-byte run holds 8 two-byte or 4 fp32
// elements.
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
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

// Per storage format: element type T, the 16-byte run VW of W elements with
// its fp32 image FW, and the 4-element group V4 of the update kernels.
template <int LP> struct Fmt;
template <> struct Fmt<1> {            // IEEE binary16
    using T = _Float16;
    static constexpr int W = 8;
    using VW = h8;
    using FW = f8;
    using V4 = h4;
};
template <> struct Fmt<2> {            // bfloat16
    using T = __bf16;
    static constexpr int W = 8;
    using VW = b8;
    using FW = f8;
    using V4 = b4;
};
template <> struct Fmt<3> {            // IEEE binary32
    using T = float;
    static constexpr int W = 4;
    using VW = f4;
    using FW = f4;
    using V4 = f4;
};

// A 16-byte run as four raw dwords.
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

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

// Vector load / store: nontemporal (NT = 1, large shards: each byte is touched
// once per step) or plain (NT = 0, small cache-resident shards).
template <typename V, int NT>
__device__ __forceinline__ V ld_v(const void* base, int64_t idx)
{
    if constexpr (NT) return ld_nt<V>(base, idx);
    else return static_cast<const V*>(base)[idx];
}

template <typename V, int NT>
__device__ __forceinline__ void st_v(void* base, int64_t idx, V x)
{
    if constexpr (NT) st_nt<V>(base, idx, x);
    else static_cast<V*>(base)[idx] = x;
}

template <int LP>
__device__ __forceinline__ float load_s(const void* base, int64_t e)
{
    return static_cast<float>(static_cast<const typename Fmt<LP>::T*>(base)[e]);
}

// Base pointer advanced by `elems` elements of the storage format.
template <int LP>
__device__ __forceinline__ const void* adv(const void* p, int64_t elems)
{
    return static_cast<const char*>(p) + (int64_t)sizeof(typename Fmt<LP>::T) * elems;
}

template <int LP>
__device__ __forceinline__ void* adv(void* p, int64_t elems)
{
    return static_cast<char*>(p) + (int64_t)sizeof(typename Fmt<LP>::T) * elems;
}

// An fp32 result held as a rounded fp32 value before it is narrowed.  Without
// it the compiler may fuse the multiply that produced it with the conversion to
// fp16 (v_fma_mixlo_f16 rounds the exact product once, straight to fp16), which
// skips the fp32 rounding in between and differs in the last fp16 bit whenever
// the fp32 product falls on an fp16 rounding tie.
__device__ __forceinline__ float pin_f32(float x)
{
    asm("" : "+v"(x));
    return x;
}

// ----------------------------------------------------------------- check

// The check runs on the unscaled value u = f32(stored) * fp32(1/scale): the
// flag marks a u that is not finite.  A stored inf or NaN always gives one,
// and so does a finite stored value that unscales past the fp32 range under a
// loss scale below 1.
__device__ __forceinline__ void check_u(float u, int& flag, double& ss)
{
    flag |= (__builtin_bit_cast(unsigned int, u) & 0x7f800000u) == 0x7f800000u;
    ss += (double)u * (double)u;
}

// Overflow flag and squared unscaled norm of one stored run.
template <int LP>
__device__ __forceinline__ void check_v(typename Fmt<LP>::VW o, float inv_scale, int& flag,
                                        double& ss)
{
    using F = Fmt<LP>;
    const typename F::FW of = __builtin_convertvector(o, typename F::FW);
#pragma unroll
    for (int k = 0; k < F::W; ++k) check_u(of[k] * inv_scale, flag, ss);
}

template <int LP>
__device__ __forceinline__ void check_s(typename Fmt<LP>::T o, float inv_scale, int& flag,
                                        double& ss)
{
    check_u(static_cast<float>(o) * inv_scale, flag, ss);
}

// One fp64 partial per workgroup: the sum of its lanes' squares, or NaN when
// any lane saw a non-finite unscaled value.  Fixed reduction shape, so the
// value is bitwise reproducible.
// Wave butterflies.  Each lane adds (or ORs) its partner's value at lane
// distance 32, 16, 8, 4, 2 and 1, in that order, and ends with the total of
// the wave, as a butterfly of xor shuffles computes it (the same operations
// on the same values, so the same bits).  The first two steps cross rows of 16
// lanes by shuffle; the last four stay inside rows and use DPP: row_ror:8
// hands lane l the value of lane l ^ 8; after that step lanes l and l ^ 8
// agree, so row_ror:4 hands it the value of lane l ^ 4; quad_perm swaps lanes
// l and l ^ 2, then l and l ^ 1.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint64_t lo = dpp_u32<CTRL>((uint32_t)u), hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
    return __builtin_bit_cast(double, (hi << 32) | lo);
}

constexpr int kDppRowRor8 = 0x128, kDppRowRor4 = 0x124;
constexpr int kDppQuadXor2 = 0x4E, kDppQuadXor1 = 0xB1;   // quad_perm [2,3,0,1], [1,0,3,2]

__device__ __forceinline__ double wave_sum(double x)
{
    x += __shfl_xor(x, 32, 64);
    x += __shfl_xor(x, 16, 64);
    x += dpp_f64<kDppRowRor8>(x);
    x += dpp_f64<kDppRowRor4>(x);
    x += dpp_f64<kDppQuadXor2>(x);
    x += dpp_f64<kDppQuadXor1>(x);
    return x;
}

__device__ __forceinline__ int wave_or(int f)
{
    f |= __shfl_xor(f, 32, 64);
    f |= __shfl_xor(f, 16, 64);
    f |= (int)dpp_u32<kDppRowRor8>((uint32_t)f);
    f |= (int)dpp_u32<kDppRowRor4>((uint32_t)f);
    f |= (int)dpp_u32<kDppQuadXor2>((uint32_t)f);
    f |= (int)dpp_u32<kDppQuadXor1>((uint32_t)f);
    return f;
}

template <int BS>
__device__ __forceinline__ void block_partial(double* slot, int flag, double ss)
{
    __shared__ double sh_ss[BS / 64];
    __shared__ int sh_f[BS / 64];
    ss = wave_sum(ss);
    flag = wave_or(flag);
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

// Whether a reduce's element-wise elements go to its last vector workgroup
// (one per lane) instead of an element-wise launch.
__host__ __device__ inline bool scalars_inline(int64_t vblocks, int64_t scalars, int BS)
{
    return vblocks >= 1 && scalars <= BS;
}

// Finish run vi of the vector body (elements head + W vi ..): acc holds the
// fp32 sum over r = 0..R-1 in order from +0; scale by fp32(1/R), convert to
// the storage format (round to nearest even), store, check.
template <int LP, int NT>
__device__ __forceinline__ void reduce_finish(const ReduceLaunch& L, int64_t vi,
                                              typename Fmt<LP>::FW acc, float inv_scale, int& flag,
                                              double& ss)
{
    using VW = typename Fmt<LP>::VW;
    // (no pin_f32 here: hipcc converts the vector with plain conversions, which
    // a codegen test checks, and the pin costs about 3% of the reduce)
    acc = acc * L.inv_r;
    const VW o = __builtin_convertvector(acc, VW);
    st_v<VW, NT>(adv<LP>(L.out, L.head), vi, o);
    check_v<LP>(o, inv_scale, flag, ss);
}

template <int LP>
__device__ __forceinline__ void reduce_s(const ReduceLaunch& L, int64_t e, float inv_scale, int& flag,
                                         double& ss)
{
    using T = typename Fmt<LP>::T;
    float acc = 0.f;
    for (int r = 0; r < L.R; ++r) acc = acc + load_s<LP>(L.c.p[r], e);
    const T o = static_cast<T>(pin_f32(acc * L.inv_r));
    static_cast<T*>(L.out)[e] = o;
    check_s<LP>(o, inv_scale, flag, ss);
}

// The last workgroup of a launch with L.sc_inline set reduces the element-wise
// elements, lane k the k-th of them, into its own flag and sum.
template <int LP>
__device__ __forceinline__ void reduce_scalars_inline(const ReduceLaunch& L, float inv_scale,
                                                      int& flag, double& ss)
{
    if (L.sc_inline && blockIdx.x == gridDim.x - 1) {
        const int64_t k = threadIdx.x;
        if (k < L.sc_a_len + L.sc_b_len)
            reduce_s<LP>(L, k < L.sc_a_len ? k : L.sc_b_start + (k - L.sc_a_len), inv_scale, flag,
                         ss);
    }
}

// Device-resident steps: workgroup 0 of each reduce or scan launch copies the
// step's starting state for an inline-fold update (see InlineFold; the copies
// are identical, and nothing reads the snapshot before the update).
__device__ __forceinline__ void snapshot_state(const DevState* dev, DevState* snap)
{
    if (snap != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *snap = *dev;
}
// The unscale factor of a check: the launch argument, or the device state's.
// The vector reduce and scan kernels read it after issuing their loads (but
// for a contribution count that is not compiled in): read first, its scalar
// load made every wave wait for that round trip before loading (a wave waits
// for all its outstanding scalar loads at once, and the loads' addresses come
// from scalar loads of the launch arguments).
__device__ __forceinline__ float check_inv_scale(float arg, const DevState* dev)
{
    return dev != nullptr ? dev->inv_scale : arg;
}

// Vector body: workgroup b covers runs [b*BS*U, (b+1)*BS*U) for BS lanes and
// U runs per lane; lane l owns runs b*BS*U + u*BS + l.  Element offsets past `head`
// are multiples of W, so contribution and output pointers advanced by `head`
// are 16-byte aligned and are indexed in units of runs.  NT: nontemporal
// loads and stores (large buckets) or plain ones (small buckets).
template <int LP, int RT, int U, int BS, int SNAP, int NT>
__global__ __launch_bounds__(BS) void reduce_vec_kernel(ReduceLaunch L)
{
    using VW = typename Fmt<LP>::VW;
    using FW = typename Fmt<LP>::FW;
    int flag = 0;
    double ss = 0.0;
    float inv_scale;
    const int64_t v0 = (int64_t)blockIdx.x * (BS * U) + threadIdx.x;
    if constexpr (RT > 0 && RT <= 8 && U == 1) {
        // One run per lane, up to 8 contributions: their loads in groups of
        // kRedGroup, each group in flight together before its arithmetic.
        // Lanes past the body load the body's last run again (a cache hit)
        // and discard it: with the loads under a condition the compiler moved
        // a run's first conversion and add in among them, so that the last
        // load waited for the first.  Measured for R = 8 (fp16 / bf16 / fp32):
        // groups of 4 beat all 8 at once by 1.5-3 points and groups of 2 by
        // 6-8.
        constexpr int G = RT < kRedGroup ? RT : kRedGroup;
        const int64_t vc = v0 < L.nvec ? v0 : L.nvec - 1;
        FW acc = (FW)(0.f);
#pragma unroll
        for (int r0 = 0; r0 < RT; r0 += G) {
            // (L.R == RT: the test only keeps a later group's loads below the
            // earlier group's arithmetic, where the compiler would hoist them)
            if (r0 == 0 || r0 < L.R) {
                VW x[G];
#pragma unroll
                for (int k = 0; k < G; ++k) x[k] = ld_v<VW, NT>(adv<LP>(L.c.p[r0 + k], L.head), vc);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 0; k < G; ++k) acc = acc + __builtin_convertvector(x[k], FW);
            }
        }
        inv_scale = check_inv_scale(L.inv_scale, L.dev);
        if (v0 < L.nvec) reduce_finish<LP, NT>(L, v0, acc, inv_scale, flag, ss);
    } else if constexpr (RT > 0) {
        // Several runs per lane, or 16 contributions.  Each run's loads sit
        // under its own condition, and the compiler widens each contribution
        // as it arrives: with several runs, one run in flight at a time before
        // every sum and store; with 16 contributions, a window of 6-10 loads.
        // (Issuing all runs' loads first measured 3.4% slower for the R = 4
        // reduce of three runs per lane, storing each run before the next
        // one's loads 0.9% slower; for R = 16, groups of 8 loads measured 1.7%
        // slower, all 16 at once 3.5%.)
        VW x[U][RT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t vi = v0 + u * BS;
            if (vi < L.nvec) {
#pragma unroll
                for (int r = 0; r < RT; ++r) x[u][r] = ld_v<VW, NT>(adv<LP>(L.c.p[r], L.head), vi);
            }
        }
        inv_scale = check_inv_scale(L.inv_scale, L.dev);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t vi = v0 + u * BS;
            if (vi < L.nvec) {
                FW acc = (FW)(0.f);
#pragma unroll
                for (int r = 0; r < RT; ++r) acc = acc + __builtin_convertvector(x[u][r], FW);
                reduce_finish<LP, NT>(L, vi, acc, inv_scale, flag, ss);
            }
        }
    } else {
        // a contribution count known only at run time: batches of 8
        inv_scale = check_inv_scale(L.inv_scale, L.dev);
        for (int u = 0; u < U; ++u) {
            const int64_t vi = v0 + u * BS;
            if (vi >= L.nvec) break;
            FW acc = (FW)(0.f);
            for (int r0 = 0; r0 < L.R; r0 += 8) {
                const int cnt = L.R - r0 < 8 ? L.R - r0 : 8;
                VW x[8];
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (k < cnt) x[k] = ld_v<VW, NT>(adv<LP>(L.c.p[r0 + k], L.head), vi);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (k < cnt) acc = acc + __builtin_convertvector(x[k], FW);
            }
            reduce_finish<LP, NT>(L, vi, acc, inv_scale, flag, ss);
        }
    }
    reduce_scalars_inline<LP>(L, inv_scale, flag, ss);
    if constexpr (SNAP) snapshot_state(L.dev, L.snapshot);
    block_partial<BS>(L.partial + L.slot_base + blockIdx.x, flag, ss);
}

// The 16 bytes at byte offset 4*D + b (b = 0 or, for 2-byte data, 2) of the
// 32-byte window lo:hi, lo at the lower address: the five dwords from dword D
// on, and for 2-byte data a byte funnel shift of each pair (v_alignbyte_b32
// takes the high dword first).
template <int LP, int D>
__device__ __forceinline__ u4 cut16(u4 lo, u4 hi, uint32_t b)
{
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    if constexpr (LP == 3) {
        (void)b;
        return u4{w[D], w[D + 1], w[D + 2], w[D + 3]};
    } else {
        return u4{__builtin_amdgcn_alignbyte(w[D + 1], w[D], b),
                  __builtin_amdgcn_alignbyte(w[D + 2], w[D + 1], b),
                  __builtin_amdgcn_alignbyte(w[D + 3], w[D + 2], b),
                  __builtin_amdgcn_alignbyte(w[D + 4], w[D + 3], b)};
    }
}

// Lane i's value of x from lane i + 1 of its wave (DPP wave_shl:1); lane 63,
// which has no such lane, keeps `old`.
__device__ __forceinline__ uint32_t from_next_lane(uint32_t old, uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, 0x130, 0xf, 0xf, false);
}

// acc[u] += the fp32 image of the run cut at dword D from lo[u] and the word
// after it: the next lane's lo[u]; for lane 63, lane 0's lo[u + 1], or nx at
// the last run.  Only the dwords the cut reads are exchanged.
template <int LP, int U, int D>
__device__ __forceinline__ void add_cut(typename Fmt<LP>::FW (&acc)[U], const u4 (&lo)[U],
                                        const u4& nx, uint32_t b)
{
    using VW = typename Fmt<LP>::VW;
    using FW = typename Fmt<LP>::FW;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        u4 hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t old =
                u == U - 1 ? nx[e] : __builtin_amdgcn_readlane(lo[u + 1 < U ? u + 1 : u][e], 0);
            hi[e] = from_next_lane(old, lo[u][e]);
        }
        // lanes past the body add what they hold: their sums are never stored
        acc[u] = acc[u] + __builtin_convertvector(__builtin_bit_cast(VW, cut16<LP, D>(lo[u], hi, b)), FW);
    }
}

// Vector body of a bucket whose contributions do not all share the output's
// address phase modulo 16 bytes (for example contributions carved back to back
// from one buffer when the shard size is not a multiple of 8).  The output
// runs are 16-byte aligned from `head`, with the workgroups, runs per lane and
// partial slots of reduce_vec_kernel.  Contribution r's run vi starts
// s_r = (its address at head) mod 16 bytes past a 16-byte boundary, inside the
// aligned words vi and vi + 1 from base_r, and is cut out of them at the
// wave-uniform offset s_r (a uniform branch on its dword part).  Each lane
// loads word vi, also for vi = nvec (the word after the body, which the run
// before it needs), and takes word vi + 1 from the next lane; lane 63 of a wave
// takes it from lane 0's next run, or at its last run loads it.  So every word
// crosses the memory path once, as in the aligned kernel, plus one word per
// wave.  The host keeps head >= s_r / esz for every r and one whole run after
// the body, so every word lies inside the bucket.  Contributions are taken K at
// a time with every load in flight before the arithmetic and added in
// ascending r from +0: each element's result is the vector kernel's.
template <int LP, int RT, int U, int BS, int SNAP, int NT>
__global__ __launch_bounds__(BS) void reduce_shift_kernel(ReduceLaunch L)
{
    using FW = typename Fmt<LP>::FW;
    constexpr int K = kRedShiftK;
    constexpr bool kNxEarly = LP == 3 ? kRedShiftNxEarlyF32 : kRedShiftNxEarly2B;
    static_assert(U == 1 || BS == 64, "runs of one lane chain across one wave only");
    int flag = 0;
    double ss = 0.0;
    const unsigned blk = shift_block<shift_group<BS, U>()>(blockIdx.x, gridDim.x);
    const int64_t v0 = (int64_t)blk * (BS * U) + threadIdx.x;
    const bool last_lane = (threadIdx.x & 63) == 63;
    FW acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = (FW)(0.f);
    // lane 63's words past its last run, cleared once here: a clear inside a
    // batch loop makes the loads of the next batch wait for this one's
    u4 nx[K];
#pragma unroll
    for (int k = 0; k < K; ++k) nx[k] = u4{0u, 0u, 0u, 0u};
    // Contributions r0 .. r0 + cnt - 1, every load in flight before the
    // arithmetic: lanes past the word after the body load that word again (a
    // cache hit) rather than branch around their loads.  Lane 63's extra words
    // go out before the others with the default cache policy for 2-byte data,
    // after them and nontemporal for fp32 (kRedShiftNxEarly*).
    auto batch = [&](int r0, int cnt) {
        u4 lo[K][U];
        auto load_nx = [&]() {
            if (last_lane && v0 + (U - 1) * BS < L.nvec) {
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    if (k < cnt) {
                        const char* p = static_cast<const char*>(adv<LP>(L.c.p[r0 + k], L.head));
                        const void* base = p - ((uintptr_t)p & 15u);
                        nx[k] = ld_v<u4, kNxEarly ? 0 : NT>(base, v0 + (U - 1) * BS + 1);
                    }
                }
            }
        };
        if constexpr (kNxEarly) load_nx();
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (k < cnt) {
                const char* p = static_cast<const char*>(adv<LP>(L.c.p[r0 + k], L.head));
                const void* base = p - ((uintptr_t)p & 15u);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t vi = v0 + u * BS;
                    lo[k][u] = ld_v<u4, NT>(base, vi <= L.nvec ? vi : L.nvec);
                }
            }
        }
        if constexpr (!kNxEarly) load_nx();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (k < cnt) {
                const uint32_t sh = (uint32_t)(uintptr_t)adv<LP>(L.c.p[r0 + k], L.head) & 15u;
                const uint32_t b = sh & 3u;
                switch (sh >> 2) {
                case 0: add_cut<LP, U, 0>(acc, lo[k], nx[k], b); break;
                case 1: add_cut<LP, U, 1>(acc, lo[k], nx[k], b); break;
                case 2: add_cut<LP, U, 2>(acc, lo[k], nx[k], b); break;
                default: add_cut<LP, U, 3>(acc, lo[k], nx[k], b); break;
                }
            }
        }
    };
    if constexpr (RT > 0) {
        // a known contribution count: straight-line batches
#pragma unroll
        for (int r0 = 0; r0 < RT; r0 += K) batch(r0, RT - r0 < K ? RT - r0 : K);
    } else {
        for (int r0 = 0; r0 < L.R; r0 += K) batch(r0, L.R - r0 < K ? L.R - r0 : K);
    }
    const float inv_scale = check_inv_scale(L.inv_scale, L.dev);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t vi = v0 + u * BS;
        if (vi < L.nvec) reduce_finish<LP, NT>(L, vi, acc[u], inv_scale, flag, ss);
    }
    reduce_scalars_inline<LP>(L, inv_scale, flag, ss);
    if constexpr (SNAP) snapshot_state(L.dev, L.snapshot);
    block_partial<BS>(L.partial + L.slot_base + blk, flag, ss);
}

template <int LP>
__global__ __launch_bounds__(kScalarBlock) void reduce_elem_kernel(ReduceLaunch L, Ranges rg,
                                                                    int64_t slot)
{
    int flag = 0;
    double ss = 0.0;
    const float inv_scale = check_inv_scale(L.inv_scale, L.dev);
    const int64_t cnt = rg.count();
#pragma unroll 2
    for (int j = 0; j < (int)(kScalarElemsPerBlock / kScalarBlock); ++j) {
        const int64_t k = (int64_t)blockIdx.x * kScalarElemsPerBlock + j * kScalarBlock + threadIdx.x;
        if (k < cnt) reduce_s<LP>(L, rg.at(k), inv_scale, flag, ss);
    }
    snapshot_state(L.dev, L.snapshot);
    block_partial<kScalarBlock>(L.partial + slot + blockIdx.x, flag, ss);
}

template <int LP, int SNAP>
__global__ __launch_bounds__(kScanBlock) void scan_vec_kernel(ScanLaunch L)
{
    using VW = typename Fmt<LP>::VW;
    int flag = 0;
    double ss = 0.0;
    const int64_t v0 = (int64_t)blockIdx.x * (kScanBlock * kScanRuns) + threadIdx.x;
    VW x[kScanRuns];
#pragma unroll
    for (int u = 0; u < kScanRuns; ++u) {
        const int64_t vi = v0 + u * kScanBlock;
        if (vi < L.nvec) x[u] = ld_nt<VW>(adv<LP>(L.g, L.head), vi);
    }
    const float inv_scale = check_inv_scale(L.inv_scale, L.dev);
#pragma unroll
    for (int u = 0; u < kScanRuns; ++u)
        if (v0 + u * kScanBlock < L.nvec) check_v<LP>(x[u], inv_scale, flag, ss);
    if constexpr (SNAP) snapshot_state(L.dev, L.snapshot);
    block_partial<kScanBlock>(L.partial + L.slot_base + blockIdx.x, flag, ss);
}

template <int LP>
__global__ __launch_bounds__(kScalarBlock) void scan_elem_kernel(ScanLaunch L, Ranges rg,
                                                                  int64_t slot)
{
    using T = typename Fmt<LP>::T;
    int flag = 0;
    double ss = 0.0;
    const float inv_scale = check_inv_scale(L.inv_scale, L.dev);
    const int64_t cnt = rg.count();
    for (int j = 0; j < (int)(kScalarElemsPerBlock / kScalarBlock); ++j) {
        const int64_t k = (int64_t)blockIdx.x * kScalarElemsPerBlock + j * kScalarBlock + threadIdx.x;
        if (k < cnt) check_s<LP>(static_cast<const T*>(L.g)[rg.at(k)], inv_scale, flag, ss);
    }
    snapshot_state(L.dev, L.snapshot);
    block_partial<kScalarBlock>(L.partial + slot + blockIdx.x, flag, ss);
}

// Decide the checked step in device memory, as the host flows do: overflow
// when the check's sum is not finite (a flagged partial is NaN); an applied step advances t and the fp64 beta
// powers and sets the bias corrections of its update; the loss scale halves on
// overflow (not below min_scale) and doubles after growth_interval clean
// steps.  The update reads upd_inv_scale (this step's), the next check
// inv_scale (the next step's).  One lane runs it.
__device__ void prepare_step(DevState* d, double ss, const PrepareArgs& a)
{
    const bool overflow = !__builtin_isfinite(ss);
    DevState s = *d;
    s.last_sumsq = ss;
    s.last_scale = s.scale;
    s.upd_inv_scale = s.inv_scale;
    s.skip = overflow ? 1 : 0;
    if (!overflow) {
        s.t += 1;
        s.pw1 = s.pw1 * a.b1;
        s.pw2 = s.pw2 * a.b2;
        s.bc1 = a.bias_correction ? (float)(1.0 - s.pw1) : 1.0f;
        s.bc2 = a.bias_correction ? (float)(1.0 - s.pw2) : 1.0f;
    }
    if (a.dynamic) {
        if (overflow) {
            double sc = s.scale / 2.0;
            s.scale = sc < a.min_scale ? a.min_scale : sc;
            s.good = 0;
        } else {
            s.good += 1;
            if (s.good == a.growth_interval) {
                s.scale = s.scale * 2.0;
                s.good = 0;
            }
        }
    }
    s.inv_scale = (float)(1.0 / s.scale);
    s.steps_run += 1;
    *d = s;
}

// Textbook global-norm clipping coefficient min(1, max_norm / (norm + 1e-6)),
// in fp64 and rounded to fp32; 1 when clipping is off or the sum is not
// finite (overflow: the step is skipped).
__device__ __forceinline__ float clip_coef(double sumsq, double max_norm)
{
    float coef = 1.0f;
    if (max_norm > 0.0 && __builtin_isfinite(sumsq)) {
        const double c = max_norm / (sqrt(sumsq) + 1e-6);
        if (c < 1.0) coef = (float)c;
    }
    return coef;
}

// Workgroup b sums in[b*chunk, min(n, (b+1)*chunk)) with a fixed shape into
// out[b]; the last level (res set, one workgroup) writes the check result and
// the clipping coefficient instead, and with dev set also decides the step.
__global__ __launch_bounds__(kFoldBlock) void fold_kernel(const double* in, int64_t n, int64_t chunk,
                                                          double* out, CheckResult* res,
                                                          double max_norm, DevState* dev,
                                                          PrepareArgs pa)
{
    const int64_t lo = (int64_t)blockIdx.x * chunk;
    const int64_t hi = lo + chunk < n ? lo + chunk : n;
    // lane l adds in[lo + l], in[lo + l + 256], ... in that order; eight loads
    // are issued before their adds, so the lane waits for memory once per
    // eight partials, not once per partial
    double s = 0.0;
    int64_t i = lo + threadIdx.x;
    for (; i + 7 * kFoldBlock < hi; i += 8 * kFoldBlock) {
        double x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = in[i + k * kFoldBlock];
#pragma unroll
        for (int k = 0; k < 8; ++k) s += x[k];
    }
    for (; i < hi; i += kFoldBlock) s += in[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    __shared__ double sh[kFoldBlock / 64];
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = sh[0];
#pragma unroll
        for (int k = 1; k < kFoldBlock / 64; ++k) t += sh[k];
        if (res == nullptr) {
            out[blockIdx.x] = t;
        } else {
            res->sumsq = t;
            res->clip = clip_coef(t, max_norm);
            res->pad = 0.0f;
            if (dev != nullptr) prepare_step(dev, t, pa);
        }
    }
}

// ----------------------------------------------------------------- update scalars

// Per-step values of an update: from the launch (host flows) or from device
// memory (the check result's clipping coefficient and NaN gate; the device
// state's scale, bias corrections and decision).  The vector kernels read them
// after issuing their loads, so their latency overlaps the loads (a skipped
// step costs the load bytes but writes nothing); the element-wise kernels read
// them first.
struct StepVals {
    float inv_scale, bc1, bc2, clip;
    bool skip;
};

__device__ __forceinline__ StepVals step_vals(const StepSource& src, float inv_scale, float bc1,
                                              float bc2)
{
    StepVals v{inv_scale, bc1, bc2, src.clip, false};
    if (src.res != nullptr) {
        v.clip = src.res->clip;
        if (src.gate) v.skip = !__builtin_isfinite(src.res->sumsq);
    }
    if (src.dev != nullptr) {
        v.inv_scale = src.dev->upd_inv_scale;
        v.bc1 = src.dev->bc1;
        v.bc2 = src.dev->bc2;
        v.skip = src.dev->skip != 0;
    }
    return v;
}

// The inline fold (InlineFold): the one-workgroup fold of at most 1024
// partials, reproduced by one wave.  Lane l stands for the fold's lanes l,
// l+64, l+128 and l+192; fold lane j adds the partials j, j+256, j+512, j+768
// (those below n) to 0.0 in that order, the four 64-lane butterflies are the
// fold's four waves, and their totals add in wave order, so the sum is bitwise
// the fold kernel's.  Every lane ends with the same value.  (Workgroups of 256
// lanes split it over their four waves instead, below.)
template <int T>
__device__ __forceinline__ double fold_small_t(const double* p, int n)
{
    // all 4T loads issued together (a slot past n loads p[0] and adds nothing)
    double x[4][T], w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int i = (int)(threadIdx.x & 63) + 64 * k + 256 * t;   // every wave sums them all
            x[k][t] = p[i < n ? i : 0];
        }
    }
    __builtin_amdgcn_sched_barrier(0);     // keep the loads ahead of every use
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        double s = 0.0;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int i = (int)(threadIdx.x & 63) + 64 * k + 256 * t;
            if (i < n) s += x[k][t];
        }
        w[k] = s;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = wave_sum(w[k]);
    return ((w[0] + w[1]) + w[2]) + w[3];
}

// The same fold with a 256-lane workgroup's four waves each taking one of the
// fold's waves: wave k loads and sums only the partials of fold wave k, and
// the four totals meet in LDS and add in wave order (the same bits, a quarter
// of the loads and butterflies per wave).  The kernels issue these loads
// before their own, so that the fold's arithmetic overlaps the wait for their
// data: lane l of wave k loads partials l + 64k and l + 64k + 256 (the second
// is added only when there are more than 256, as the fold kernel does; below
// that it loads partial 0 again).
struct FoldLoads {
    double x[4];
};

// T loads per lane: partials l + 64k + 256t, t < T (T = 2 up to 512
// partials, 4 up to 1024).
template <int T>
__device__ __forceinline__ FoldLoads fold_split_issue(const double* p, int n)
{
    FoldLoads fl;
    const int i = (int)(threadIdx.x & 63) + 64 * (int)(threadIdx.x >> 6);
#pragma unroll
    for (int t = 0; t < T; ++t) fl.x[t] = p[i + 256 * t < n ? i + 256 * t : 0];
    return fl;
}

template <int T>
__device__ __forceinline__ double fold_split_finish(const FoldLoads& fl, int n)
{
    __shared__ double sh_w[4];
    const int k = (int)(threadIdx.x >> 6);
    const int i = (int)(threadIdx.x & 63) + 64 * k;
    double s = 0.0;
#pragma unroll
    for (int t = 0; t < T; ++t)
        if (i + 256 * t < n) s += fl.x[t];
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) sh_w[k] = s;
    __syncthreads();
    return ((sh_w[0] + sh_w[1]) + sh_w[2]) + sh_w[3];
}

template <int B, int T>
__device__ __forceinline__ FoldLoads fold_issue(const InlineFold& f)
{
    if constexpr (B == 256) return fold_split_issue<T>(f.partial, f.n);
    else return FoldLoads{};
}

template <int B, int T>
__device__ __forceinline__ double fold_small(const double* p, int n, const FoldLoads& fl)
{
    if constexpr (B == 256) {
        (void)p;
        return fold_split_finish<T>(fl, n);
    } else {
        (void)fl;
        if constexpr (kInlineFoldMax > 512)
            if (n > 512) return fold_small_t<4>(p, n);
        return n <= 256 ? fold_small_t<1>(p, n) : fold_small_t<2>(p, n);
    }
}

// The step as the fold's last lane decides it, computed by every workgroup
// from the snapshot of the state the step started with.
struct InlineDecision {
    DevState next;
    double sumsq;
    float clip;
};

template <int B, int T>
__device__ __forceinline__ StepVals step_vals_inline(const InlineFold& f, const FoldLoads& fl,
                                                     InlineDecision& d)
{
    d.next = *f.snapshot;                  // loaded while the partials are in flight
    d.sumsq = fold_small<B, T>(f.partial, f.n, fl);
    prepare_step(&d.next, d.sumsq, f.pa);
    d.clip = clip_coef(d.sumsq, f.max_norm);
    return StepVals{d.next.upd_inv_scale, d.next.bc1, d.next.bc2, d.clip, d.next.skip != 0};
}

// Workgroup 0 writes the advanced state and the check result; no workgroup of
// the update reads either.
__device__ __forceinline__ void inline_commit(const InlineFold& f, const InlineDecision& d)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *f.dev = d.next;
        f.res->sumsq = d.sumsq;
        f.res->clip = d.clip;
        f.res->pad = 0.0f;
    }
}

// ----------------------------------------------------------------- Adam

// Textbook Adam on one element (Kingma & Ba 2015, Algorithm 1), in the order
// the public header states; p, m, v are updated in place.
template <int WD>
__device__ __forceinline__ void adam_e(float graw, float& p, float& m, float& v,
                                       const AdamLaunch& a, const StepVals& sv)
{
    float g = graw * sv.inv_scale;
    g = g * sv.clip;                       // exact when the coefficient is 1
    if constexpr (WD == kWdL2) g = g + a.wd * p;
    m = a.b1 * m + a.omb1 * g;
    v = a.b2 * v + a.omb2 * (g * g);
    const float mh = m / sv.bc1;
    const float vh = v / sv.bc2;
    float u = mh / (sqrtf(vh) + a.eps);
    if constexpr (WD == kWdDecoupled) u = u + a.wd * p;
    p = p - a.lr * u;
}

// Vector body: groups of 4 elements past `head` (fp32 pointers advanced by
// head are 16-byte aligned, 2-byte pointers 8-byte aligned).  Workgroup b
// covers groups [b*B*G, (b+1)*B*G) for B lanes and G groups per lane; lane l
// owns groups b*B*G + u*B + l, u < G, and issues all loads before any
// arithmetic.  With fp32 storage there is no 2-byte parameter to write.
// INL > 0: the step's values come from the inline fold (a.src.fold), whose
// partials each lane loads INL of (2 up to 512 partials, 4 up to 1024).  NT as
// for the reduce (plain loads and stores for small shards).
template <int LP, int WD, int INL, int B, int G, int NT>
__global__ __launch_bounds__(B) void adam_vec_kernel(AdamLaunch a)
{
    using V4 = typename Fmt<LP>::V4;
    const void* gb = adv<LP>(a.grad, a.head);
    float* pb = a.master + a.head;
    float* mb = a.m + a.head;
    float* vb = a.v + a.head;
    const int64_t q0 = (int64_t)blockIdx.x * (B * G) + threadIdx.x;
    FoldLoads fl{};
    if constexpr (INL) {
        fl = fold_issue<B, INL>(a.src.fold);
        __builtin_amdgcn_sched_barrier(0);
    }
    V4 g[G];
    f4 p[G], m[G], v[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const int64_t q = q0 + u * B;
        if (INL || q < a.ngroups) {
            // (an inline-fold launch has groups: lanes past them reload the
            // last one, so that no branch hides from the compiler how many
            // loads follow the fold's)
            const int64_t qc = q < a.ngroups ? q : a.ngroups - 1;
            g[u] = ld_v<V4, NT>(gb, qc);
            p[u] = ld_v<f4, NT>(pb, qc);
            m[u] = ld_v<f4, NT>(mb, qc);
            v[u] = ld_v<f4, NT>(vb, qc);
        }
    }
    if constexpr (INL) __builtin_amdgcn_sched_barrier(0);   // the fold's arithmetic after every load
    StepVals sv;
    InlineDecision dec;
    if constexpr (INL) {
        sv = step_vals_inline<B, INL>(a.src.fold, fl, dec);
    } else {
        sv = step_vals(a.src, a.inv_scale, a.bc1, a.bc2);
        if (sv.skip) return;
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const int64_t q = q0 + u * B;
        if (q < a.ngroups && !(INL && sv.skip)) {
            const f4 gf = __builtin_convertvector(g[u], f4);
            f4 pp = p[u], mm = m[u], vv = v[u];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float pk = pp[k], mk = mm[k], vk = vv[k];
                adam_e<WD>(gf[k], pk, mk, vk, a, sv);
                pp[k] = pk;
                mm[k] = mk;
                vv[k] = vk;
            }
            st_v<f4, NT>(pb, q, pp);
            st_v<f4, NT>(mb, q, mm);
            st_v<f4, NT>(vb, q, vv);
            if constexpr (LP != 3)
                st_v<V4, NT>(adv<LP>(a.param, a.head), q, __builtin_convertvector(pp, V4));
        }
    }
    if constexpr (INL) inline_commit(a.src.fold, dec);
}

template <int LP, int WD>
__global__ __launch_bounds__(kScalarBlock) void adam_elem_kernel(AdamLaunch a, Ranges rg)
{
    using T = typename Fmt<LP>::T;
    const StepVals sv = step_vals(a.src, a.inv_scale, a.bc1, a.bc2);
    if (sv.skip) return;
    const int64_t cnt = rg.count();
    for (int j = 0; j < (int)(kScalarElemsPerBlock / kScalarBlock); ++j) {
        const int64_t k = (int64_t)blockIdx.x * kScalarElemsPerBlock + j * kScalarBlock + threadIdx.x;
        if (k < cnt) {
            const int64_t e = rg.at(k);
            float p = a.master[e], m = a.m[e], v = a.v[e];
            adam_e<WD>(load_s<LP>(a.grad, e), p, m, v, a, sv);
            a.master[e] = p;
            a.m[e] = m;
            a.v[e] = v;
            if constexpr (LP != 3) static_cast<T*>(a.param)[e] = static_cast<T>(p);
        }
    }
}

// ----------------------------------------------------------------- SGD

// Heavy-ball SGD with L2 weight decay on one element, in the order the public
// header states; p and the momentum buffer b are updated in place.
template <int MOM, int WD>
__device__ __forceinline__ void sgd_e(float graw, float& p, float& b, const SgdLaunch& a,
                                      const StepVals& sv)
{
    float g = graw * sv.inv_scale;
    g = g * sv.clip;                       // exact when the coefficient is 1
    if constexpr (WD) g = g + a.wd * p;
    float d = g;
    if constexpr (MOM) {
        b = a.mu * b + g;
        d = b;
    }
    p = p - a.lr * d;
}

// Same layout and load-first order as adam_vec_kernel, with B lanes and G
// groups per lane; INL and NT as there.
template <int LP, int MOM, int WD, int G, int INL, int B, int NT>
__global__ __launch_bounds__(B) void sgd_vec_kernel(SgdLaunch a)
{
    using V4 = typename Fmt<LP>::V4;
    const void* gb = adv<LP>(a.grad, a.head);
    float* pb = a.master + a.head;
    float* bb = MOM ? a.mom + a.head : nullptr;
    const int64_t q0 = (int64_t)blockIdx.x * (B * G) + threadIdx.x;
    FoldLoads fl{};
    if constexpr (INL) {
        fl = fold_issue<B, INL>(a.src.fold);
        __builtin_amdgcn_sched_barrier(0);
    }
    V4 g[G];
    f4 p[G], b[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const int64_t q = q0 + u * B;
        if (INL || q < a.ngroups) {
            const int64_t qc = q < a.ngroups ? q : a.ngroups - 1;   // as in adam_vec_kernel
            g[u] = ld_v<V4, NT>(gb, qc);
            p[u] = ld_v<f4, NT>(pb, qc);
            if constexpr (MOM) b[u] = ld_v<f4, NT>(bb, qc);
        }
    }
    if constexpr (INL) __builtin_amdgcn_sched_barrier(0);
    StepVals sv;
    InlineDecision dec;
    if constexpr (INL) {
        sv = step_vals_inline<B, INL>(a.src.fold, fl, dec);
    } else {
        sv = step_vals(a.src, a.inv_scale, 1.0f, 1.0f);
        if (sv.skip) return;
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const int64_t q = q0 + u * B;
        if (q < a.ngroups && !(INL && sv.skip)) {
            const f4 gf = __builtin_convertvector(g[u], f4);
            f4 pp = p[u];
            f4 buf = (f4)(0.f);
            if constexpr (MOM) buf = b[u];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float pk = pp[k], bk = buf[k];
                sgd_e<MOM, WD>(gf[k], pk, bk, a, sv);
                pp[k] = pk;
                buf[k] = bk;
            }
            st_v<f4, NT>(pb, q, pp);
            if constexpr (MOM) st_v<f4, NT>(bb, q, buf);
            if constexpr (LP != 3)
                st_v<V4, NT>(adv<LP>(a.param, a.head), q, __builtin_convertvector(pp, V4));
        }
    }
    if constexpr (INL) inline_commit(a.src.fold, dec);
}

template <int LP, int MOM, int WD>
__global__ __launch_bounds__(kScalarBlock) void sgd_elem_kernel(SgdLaunch a, Ranges rg)
{
    using T = typename Fmt<LP>::T;
    const StepVals sv = step_vals(a.src, a.inv_scale, 1.0f, 1.0f);
    if (sv.skip) return;
    const int64_t cnt = rg.count();
    for (int j = 0; j < (int)(kScalarElemsPerBlock / kScalarBlock); ++j) {
        const int64_t k = (int64_t)blockIdx.x * kScalarElemsPerBlock + j * kScalarBlock + threadIdx.x;
        if (k < cnt) {
            const int64_t e = rg.at(k);
            float p = a.master[e];
            float b = 0.f;
            if constexpr (MOM) b = a.mom[e];
            sgd_e<MOM, WD>(load_s<LP>(a.grad, e), p, b, a, sv);
            a.master[e] = p;
            if constexpr (MOM) a.mom[e] = b;
            if constexpr (LP != 3) static_cast<T*>(a.param)[e] = static_cast<T>(p);
        }
    }
}

// ----------------------------------------------------------------- device-resident step

__global__ __launch_bounds__(64) void load_state_kernel(DevState* d, DevState init)
{
    if (threadIdx.x == 0) *d = init;
}

// ----------------------------------------------------------------- launches

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

// SNAP = 1 (a snapshot target is set) only for the small steps of the inline
// fold, so the reduce of every other step keeps the plain kernel.
template <int LP, int RT, int U, int BS, int NT = 1>
void reduce_vec_go(const ReduceLaunch& L, unsigned grid, hipStream_t s)
{
    if (L.snapshot != nullptr)
        reduce_vec_kernel<LP, RT, U, BS, 1, NT><<<grid, BS, L.lds_reserve, s>>>(L);
    else
        reduce_vec_kernel<LP, RT, U, BS, 0, NT><<<grid, BS, L.lds_reserve, s>>>(L);
}

// Below 8 contributions the workgroup has kRedBlock lanes and the runs per
// lane U is kRedRuns or kRedRunsSmall; from 8 on it has kRedBlockMany lanes
// and U is kRedRunsMany; a bucket of a small shard (shard_small) takes
// kSmallBlock lanes, one run each, plain loads and stores.  U and BS must be the ones the
// dispatch sized the grid with (red_runs / red_block of the whole bucket).
template <int LP, int RT>
void reduce_vec_few(const ReduceLaunch& L, unsigned grid, int U, hipStream_t s)
{
    if (U == kRedRunsSmall)
        reduce_vec_go<LP, RT, kRedRunsSmall, kRedBlock>(L, grid, s);
    else
        reduce_vec_go<LP, RT, kRedRuns, kRedBlock>(L, grid, s);
}

template <int LP, int RT>
void reduce_vec_small(const ReduceLaunch& L, unsigned grid, hipStream_t s)
{
    reduce_vec_go<LP, RT, 1, kSmallBlock, 0>(L, grid, s);
}

template <int LP>
hipError_t reduce_vec_launch(const ReduceLaunch& L, unsigned grid, int U, bool small,
                             hipStream_t s)
{
    constexpr int B = kRedRunsMany, BM = kRedBlockMany;
    if (small) {
        switch (L.R) {
        case 1: reduce_vec_small<LP, 1>(L, grid, s); break;
        case 2: reduce_vec_small<LP, 2>(L, grid, s); break;
        case 4: reduce_vec_small<LP, 4>(L, grid, s); break;
        case 8: reduce_vec_small<LP, 8>(L, grid, s); break;
        case 16: reduce_vec_small<LP, 16>(L, grid, s); break;
        default: reduce_vec_small<LP, 0>(L, grid, s); break;
        }
        return hipGetLastError();
    }
    switch (L.R) {
    case 1: reduce_vec_few<LP, 1>(L, grid, U, s); break;
    case 2: reduce_vec_few<LP, 2>(L, grid, U, s); break;
    case 4: reduce_vec_few<LP, 4>(L, grid, U, s); break;
    case 8: reduce_vec_go<LP, 8, B, BM>(L, grid, s); break;
    case 16: reduce_vec_go<LP, 16, B, BM>(L, grid, s); break;
    default:
        if (L.R >= kRedManyR)
            reduce_vec_go<LP, 0, B, BM>(L, grid, s);
        else
            reduce_vec_few<LP, 0>(L, grid, U, s);
        break;
    }
    return hipGetLastError();
}

// The shift kernel of a bucket (L.shift = 1): the vector kernel's workgroups,
// with kRedShiftRuns runs per lane below 8 contributions on large shards, and
// a compiled-in contribution count for R = 4, 8 and 16.
template <int LP, int RT, int U, int BS, int NT>
void reduce_shift_rt(const ReduceLaunch& L, unsigned grid, hipStream_t s)
{
    if (L.snapshot != nullptr)
        reduce_shift_kernel<LP, RT, U, BS, 1, NT><<<grid, BS, L.lds_reserve, s>>>(L);
    else
        reduce_shift_kernel<LP, RT, U, BS, 0, NT><<<grid, BS, L.lds_reserve, s>>>(L);
}

template <int LP, int U, int BS, int NT>
void reduce_shift_go(const ReduceLaunch& L, unsigned grid, hipStream_t s)
{
    switch (L.R) {
    case 4: reduce_shift_rt<LP, 4, U, BS, NT>(L, grid, s); break;
    case 8: reduce_shift_rt<LP, 8, U, BS, NT>(L, grid, s); break;
    case 16: reduce_shift_rt<LP, 16, U, BS, NT>(L, grid, s); break;
    default: reduce_shift_rt<LP, 0, U, BS, NT>(L, grid, s); break;
    }
}

template <int LP>
hipError_t reduce_shift_launch(const ReduceLaunch& L, unsigned grid, int U, bool small,
                               hipStream_t s)
{
    (void)U;
    if (small)
        reduce_shift_go<LP, 1, kSmallBlock, 0>(L, grid, s);
    else if (L.R >= kRedManyR)
        reduce_shift_go<LP, kRedRunsMany, kRedBlockMany, 1>(L, grid, s);
    else
        reduce_shift_go<LP, kRedShiftRuns, kRedBlock, 1>(L, grid, s);
    return hipGetLastError();
}

template <int LP>
hipError_t reduce_dispatch(const ReduceLaunch& L, hipStream_t s)
{
    constexpr int W = Fmt<LP>::W;
    const bool small = L.small != 0;
    const int U = red_runs(L.R, L.nvec, small, L.shift != 0);
    const int BS = red_block(L.R, small);
    const int64_t runs_per_block = (int64_t)BS * U;
    const int64_t vblocks = L.vec_ok ? ceil_div(L.nvec, runs_per_block) : 0;
    // consecutive launches of at most kMaxLaunchItems work-items; each starts
    // its runs and its partial slots where the previous one stopped
    const int64_t max_blocks = kMaxLaunchItems / BS;
    const Ranges rg = ranges_of(L.n, L.head, W * L.nvec, L.vec_ok);
    const bool inl = scalars_inline(vblocks, rg.a_len + rg.b_len, BS);
    for (int64_t b0 = 0; b0 < vblocks; b0 += max_blocks) {
        const int64_t nb = vblocks - b0 < max_blocks ? vblocks - b0 : max_blocks;
        ReduceLaunch part = L;
        part.head = L.head + W * runs_per_block * b0;
        part.nvec = L.nvec - runs_per_block * b0;
        part.slot_base = L.slot_base + b0;
        // the element-wise elements ride on the last workgroup of the last launch
        part.sc_inline = inl && b0 + nb == vblocks;
        part.sc_a_len = rg.a_len;
        part.sc_b_start = rg.b_start;
        part.sc_b_len = rg.b_len;
        hipError_t e = L.shift ? reduce_shift_launch<LP>(part, (unsigned)nb, U, small, s)
                                : reduce_vec_launch<LP>(part, (unsigned)nb, U, small, s);
        if (e != hipSuccess) return e;
    }
    const int64_t sblocks = inl ? 0 : ceil_div(rg.a_len + rg.b_len, kScalarElemsPerBlock);
    if (sblocks > 0)
        reduce_elem_kernel<LP><<<(unsigned)sblocks, kScalarBlock, 0, s>>>(L, rg, L.slot_base + vblocks);
    return hipGetLastError();
}

template <int LP>
hipError_t scan_dispatch(const ScanLaunch& L, hipStream_t s)
{
    constexpr int W = Fmt<LP>::W;
    const int64_t runs_per_block = (int64_t)kScanBlock * kScanRuns;
    const int64_t vblocks = L.vec_ok ? ceil_div(L.nvec, runs_per_block) : 0;
    const int64_t max_blocks = kMaxLaunchItems / kScanBlock;
    for (int64_t b0 = 0; b0 < vblocks; b0 += max_blocks) {
        const int64_t nb = vblocks - b0 < max_blocks ? vblocks - b0 : max_blocks;
        ScanLaunch part = L;
        part.head = L.head + W * runs_per_block * b0;
        part.nvec = L.nvec - runs_per_block * b0;
        part.slot_base = L.slot_base + b0;
        if (L.snapshot != nullptr)
            scan_vec_kernel<LP, 1><<<(unsigned)nb, kScanBlock, L.lds_reserve, s>>>(part);
        else
            scan_vec_kernel<LP, 0><<<(unsigned)nb, kScanBlock, L.lds_reserve, s>>>(part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const Ranges rg = ranges_of(L.n, L.head, W * L.nvec, L.vec_ok);
    const int64_t sblocks = ceil_div(rg.a_len + rg.b_len, kScalarElemsPerBlock);
    if (sblocks > 0)
        scan_elem_kernel<LP><<<(unsigned)sblocks, kScalarBlock, 0, s>>>(L, rg, L.slot_base + vblocks);
    return hipGetLastError();
}

// The vector launches of an update of B lanes and G groups per lane: the
// inline-fold launch (one over the whole array) or consecutive launches of at
// most kMaxLaunchItems work-items.
template <int LP, int WD, int B, int G, int NT>
hipError_t adam_vec_launches(const AdamLaunch& a, int64_t vblocks, hipStream_t s)
{
    constexpr int64_t groups_per_block = (int64_t)B * G;
    if (a.src.fold.partial != nullptr) {
        if (a.src.fold.n <= 512)
            adam_vec_kernel<LP, WD, 2, B, G, NT><<<(unsigned)vblocks, B, a.lds_reserve, s>>>(a);
        else
            adam_vec_kernel<LP, WD, 4, B, G, NT><<<(unsigned)vblocks, B, a.lds_reserve, s>>>(a);
        return hipGetLastError();
    }
    const int64_t max_blocks = kMaxLaunchItems / B;
    for (int64_t b0 = 0; b0 < vblocks; b0 += max_blocks) {
        const int64_t nb = vblocks - b0 < max_blocks ? vblocks - b0 : max_blocks;
        AdamLaunch part = a;
        part.head = a.head + 4 * groups_per_block * b0;
        part.ngroups = a.ngroups - groups_per_block * b0;
        adam_vec_kernel<LP, WD, 0, B, G, NT><<<(unsigned)nb, B, a.lds_reserve, s>>>(part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int LP, int WD>
hipError_t adam_dispatch(const AdamLaunch& a, hipStream_t s)
{
    const bool small = shard_small(a.n);
    const int lanes = adam_lanes(a.n), groups = adam_groups(a.n);
    const int64_t vblocks = a.vec_ok ? ceil_div(a.ngroups, (int64_t)lanes * groups) : 0;
    if (a.src.fold.partial != nullptr &&
        (!a.vec_ok || a.head != 0 || 4 * a.ngroups != a.n || vblocks < 1 ||
         !one_launch(a.ngroups, lanes, groups) || a.src.fold.n < 1 ||
         a.src.fold.n > kInlineFoldMax))
        return hipErrorInvalidValue;          // the inline fold needs one vector launch
    hipError_t e = small ? adam_vec_launches<LP, WD, kSmallUpdBlock, 1, 0>(a, vblocks, s)
                         : adam_vec_launches<LP, WD, kAdamBlock, kAdamGroups, 1>(a, vblocks, s);
    if (e != hipSuccess || a.src.fold.partial != nullptr) return e;
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

template <int LP, int MOM, int WD, int B, int G, int NT>
hipError_t sgd_vec_launches(const SgdLaunch& a, int64_t vblocks, hipStream_t s)
{
    constexpr int64_t groups_per_block = (int64_t)B * G;
    if (a.src.fold.partial != nullptr) {
        if (a.src.fold.n <= 512)
            sgd_vec_kernel<LP, MOM, WD, G, 2, B, NT><<<(unsigned)vblocks, B, a.lds_reserve, s>>>(a);
        else
            sgd_vec_kernel<LP, MOM, WD, G, 4, B, NT><<<(unsigned)vblocks, B, a.lds_reserve, s>>>(a);
        return hipGetLastError();
    }
    const int64_t max_blocks = kMaxLaunchItems / B;
    for (int64_t b0 = 0; b0 < vblocks; b0 += max_blocks) {
        const int64_t nb = vblocks - b0 < max_blocks ? vblocks - b0 : max_blocks;
        SgdLaunch part = a;
        part.head = a.head + 4 * groups_per_block * b0;
        part.ngroups = a.ngroups - groups_per_block * b0;
        sgd_vec_kernel<LP, MOM, WD, G, 0, B, NT><<<(unsigned)nb, B, a.lds_reserve, s>>>(part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int LP, int MOM, int WD>
hipError_t sgd_dispatch(const SgdLaunch& a, hipStream_t s)
{
    constexpr int G = MOM ? kSgdMomGroups : kSgdPlainGroups;
    const bool small = shard_small(a.n);
    const int lanes = sgd_lanes(a.n), groups = sgd_groups(a.n, MOM);
    const int64_t vblocks = a.vec_ok ? ceil_div(a.ngroups, (int64_t)lanes * groups) : 0;
    if (a.src.fold.partial != nullptr &&
        (!a.vec_ok || a.head != 0 || 4 * a.ngroups != a.n || vblocks < 1 ||
         !one_launch(a.ngroups, lanes, groups) || a.src.fold.n < 1 ||
         a.src.fold.n > kInlineFoldMax))
        return hipErrorInvalidValue;          // the inline fold needs one vector launch
    hipError_t e = small ? sgd_vec_launches<LP, MOM, WD, kSmallUpdBlock, 1, 0>(a, vblocks, s)
                         : sgd_vec_launches<LP, MOM, WD, kSgdBlock, G, 1>(a, vblocks, s);
    if (e != hipSuccess || a.src.fold.partial != nullptr) return e;
    const Ranges rg = ranges_of(a.n, a.head, 4 * a.ngroups, a.vec_ok);
    const int64_t sblocks = ceil_div(rg.a_len + rg.b_len, kScalarElemsPerBlock);
    if (sblocks > 0)
        sgd_elem_kernel<LP, MOM, WD><<<(unsigned)sblocks, kScalarBlock, 0, s>>>(a, rg);
    return hipGetLastError();
}

template <int LP>
hipError_t sgd_dispatch_kind(const SgdLaunch& a, hipStream_t s)
{
    if (a.mom != nullptr)
        return a.has_wd ? sgd_dispatch<LP, 1, 1>(a, s) : sgd_dispatch<LP, 1, 0>(a, s);
    return a.has_wd ? sgd_dispatch<LP, 0, 1>(a, s) : sgd_dispatch<LP, 0, 0>(a, s);
}

}  // namespace

int64_t reduce_blocks(int64_t n, int64_t head, int64_t nvec, int32_t vec_ok, int W, int U,
                      int BS, bool inline_scalars)
{
    (void)head;
    const int64_t vblocks = vec_ok ? ceil_div(nvec, (int64_t)BS * U) : 0;
    const int64_t scalars = vec_ok ? n - (int64_t)W * nvec : n;
    if (inline_scalars && scalars_inline(vblocks, scalars, BS)) return vblocks;
    return vblocks + ceil_div(scalars, kScalarElemsPerBlock);
}

hipError_t launch_reduce(const ReduceLaunch& L, hipStream_t s)
{
    switch (L.lp) {
    case 2: return reduce_dispatch<2>(L, s);
    case 3: return reduce_dispatch<3>(L, s);
    default: return reduce_dispatch<1>(L, s);
    }
}

hipError_t launch_scan(const ScanLaunch& L, hipStream_t s)
{
    switch (L.lp) {
    case 2: return scan_dispatch<2>(L, s);
    case 3: return scan_dispatch<3>(L, s);
    default: return scan_dispatch<1>(L, s);
    }
}

hipError_t launch_finalize(const double* partial, int64_t nslots, double* level1,
                           CheckResult* out, double max_norm, DevState* dev,
                           const PrepareArgs& pa, hipStream_t s)
{
    const PrepareArgs none{};
    if (nslots <= kFoldOneLevel) {
        // few partials: one workgroup sums them all (one launch less)
        fold_kernel<<<1, kFoldBlock, 0, s>>>(partial, nslots, nslots, nullptr, out, max_norm, dev,
                                             pa);
        return hipGetLastError();
    }
    int64_t g1 = ceil_div(nslots, 1024);
    if (g1 > kFoldMaxBlocks) g1 = kFoldMaxBlocks;
    const int64_t chunk = ceil_div(nslots, g1);
    fold_kernel<<<(unsigned)g1, kFoldBlock, 0, s>>>(partial, nslots, chunk, level1, nullptr, 0.0,
                                                    nullptr, none);
    fold_kernel<<<1, kFoldBlock, 0, s>>>(level1, g1, g1, nullptr, out, max_norm, dev, pa);
    return hipGetLastError();
}

hipError_t launch_load_state(DevState* d, const DevState& init, hipStream_t s)
{
    load_state_kernel<<<1, 64, 0, s>>>(d, init);
    return hipGetLastError();
}



hipError_t launch_adam(const AdamLaunch& a, hipStream_t s)
{
    switch (a.lp) {
    case 2: return adam_dispatch_wd<2>(a, s);
    case 3: return adam_dispatch_wd<3>(a, s);
    default: return adam_dispatch_wd<1>(a, s);
    }
}

hipError_t launch_sgd(const SgdLaunch& a, hipStream_t s)
{
    switch (a.lp) {
    case 2: return sgd_dispatch_kind<2>(a, s);
    case 3: return sgd_dispatch_kind<3>(a, s);
    default: return sgd_dispatch_kind<1>(a, s);
    }
}

}  // namespace zk
