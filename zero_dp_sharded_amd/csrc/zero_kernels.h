// Internal launch interface between the C ABI (zero_shard.cpp) and the gfx950
// kernels (zero_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zk {

constexpr int kMaxContrib = 64;

// Reduce / scan: each lane a few 16-byte runs (a run is 8 two-byte or 4 fp32
// elements; each load instruction of a wave covers 1 KiB contiguously).
// Workgroup size, runs per lane and resident workgroups per CU, as measured
// best on MI355X (roughly 80-144 KiB of loads in flight per CU):
//   reduce, R < 8:   64 lanes (one wave), 3 runs, 10 workgroups per CU (2 runs
//                    for buckets too small to fill the chip, where more
//                    workgroups finish sooner);
//   reduce, R >= 8:  64 lanes, 1 run, 12 workgroups per CU with 2-byte storage
//                    and 10 with fp32 (6 from R = 16); up to R = 8 the loads go
//                    out in groups of 4 contributions;
//   shift reduce (contributions off the output's 16-byte phase): 64 lanes,
//                    2 runs and 14 workgroups per CU below R = 8; 1 run and 16
//                    (2-byte storage) or 12 (fp32) workgroups per CU from R = 8;
//                    batches of 4 contributions;
//   scan (1 stream): 256 lanes, 4 runs, 8 workgroups per CU.
// (The ZK_* macros exist only to build tuning variants; the defaults are the
// measured optimum.)
#ifndef ZK_RED_BLOCK
#define ZK_RED_BLOCK 64
#endif
#ifndef ZK_RED_BLOCK_MANY
#define ZK_RED_BLOCK_MANY 64
#endif
#ifndef ZK_RED_RUNS
#define ZK_RED_RUNS 3
#endif
#ifndef ZK_RED_RUNS_SMALL
#define ZK_RED_RUNS_SMALL 2
#endif
#ifndef ZK_RED_RUNS_MANY
#define ZK_RED_RUNS_MANY 1
#endif
#ifndef ZK_RED_PER_CU
#define ZK_RED_PER_CU 10
#endif
#ifndef ZK_RED_PER_CU_MANY
#define ZK_RED_PER_CU_MANY 10
#endif
#ifndef ZK_RED_PER_CU_MANY_2B
#define ZK_RED_PER_CU_MANY_2B 12
#endif
#ifndef ZK_RED_PER_CU_WIDE
#define ZK_RED_PER_CU_WIDE 6
#endif
#ifndef ZK_RED_GROUP
#define ZK_RED_GROUP 4
#endif
#ifndef ZK_RED_SHIFT_K
#define ZK_RED_SHIFT_K 4
#endif
#ifndef ZK_RED_SHIFT_RUNS
#define ZK_RED_SHIFT_RUNS 2
#endif
#ifndef ZK_RED_SHIFT_PER_CU
#define ZK_RED_SHIFT_PER_CU 14
#endif
#ifndef ZK_RED_SHIFT_PER_CU_MANY
#define ZK_RED_SHIFT_PER_CU_MANY 12
#endif
#ifndef ZK_RED_SHIFT_PER_CU_MANY_2B
#define ZK_RED_SHIFT_PER_CU_MANY_2B 16
#endif
#ifndef ZK_RED_SHIFT_NX_EARLY_2B
#define ZK_RED_SHIFT_NX_EARLY_2B 1
#endif
#ifndef ZK_RED_SHIFT_NX_EARLY_F32
#define ZK_RED_SHIFT_NX_EARLY_F32 0
#endif
#ifndef ZK_RED_SHIFT_GROUP_RUNS
#define ZK_RED_SHIFT_GROUP_RUNS 64
#endif
#ifndef ZK_SCAN_BLOCK
#define ZK_SCAN_BLOCK 256
#endif
#ifndef ZK_SCAN_RUNS
#define ZK_SCAN_RUNS 4
#endif
#ifndef ZK_SCAN_PER_CU
#define ZK_SCAN_PER_CU 8
#endif
#ifndef ZK_ADAM_BLOCK
#define ZK_ADAM_BLOCK 64
#endif
#ifndef ZK_ADAM_GROUPS
#define ZK_ADAM_GROUPS 1
#endif
#ifndef ZK_ADAM_PER_CU
#define ZK_ADAM_PER_CU 10
#endif
#ifndef ZK_SGD_MOM_GROUPS
#define ZK_SGD_MOM_GROUPS 1
#endif
#ifndef ZK_SGD_MOM_PER_CU
#define ZK_SGD_MOM_PER_CU 16
#endif
#ifndef ZK_SGD_PLAIN_GROUPS
#define ZK_SGD_PLAIN_GROUPS 1
#endif
#ifndef ZK_SGD_PLAIN_PER_CU
#define ZK_SGD_PLAIN_PER_CU 24
#endif
constexpr int kRedBlock = ZK_RED_BLOCK;           // reduce, R < 8
constexpr int kRedBlockMany = ZK_RED_BLOCK_MANY;  // reduce, R >= 8
constexpr int kRedRuns = ZK_RED_RUNS;
constexpr int kRedRunsMany = ZK_RED_RUNS_MANY;   // runs per lane when R >= 8
constexpr int kRedManyR = 8;
constexpr int kRedRunsSmall = ZK_RED_RUNS_SMALL;   // R < 8, bucket below kRedSmallNvec runs
// contributions (of at most 8) whose loads a one-run-per-lane reduce issues
// together
constexpr int kRedGroup = ZK_RED_GROUP;
// contributions the shift kernel takes per batch of loads (measured with one
// run per lane: 4 beat 8 by 1-4 points)
constexpr int kRedShiftK = ZK_RED_SHIFT_K;
// runs per lane of the shift kernel below 8 contributions (its registers hold
// two words per run and contribution in flight)
constexpr int kRedShiftRuns = ZK_RED_SHIFT_RUNS;
// The shift kernel hands each XCD kRedShiftGroupRuns consecutive wave-runs
// (kRedShiftGroupRuns / U workgroups of U runs per lane) at a time, so that the
// word a wave's last lane reads past its runs is usually read by a wave of the
// same XCD (same L2) as well (0: plain order).  64 measured best for one and
// two runs per lane (32 or 128 lose up to 2.5 points with two).
constexpr int kRedShiftGroupRuns = ZK_RED_SHIFT_GROUP_RUNS;
// Lane 63's word past its last run: loaded before the contribution runs with
// the default cache policy (true), or after them, nontemporal (false).  Early
// and cached, for 2-byte data, the reduce reads x1.005-1.006 of its
// algorithmic bytes instead of x1.020 and runs 1-4 points faster; for fp32 it
// made every wave wait for those loads before issuing its runs (8 points
// slower), so fp32 keeps them last.
constexpr bool kRedShiftNxEarly2B = ZK_RED_SHIFT_NX_EARLY_2B != 0;
constexpr bool kRedShiftNxEarlyF32 = ZK_RED_SHIFT_NX_EARLY_F32 != 0;
// Resident shift-kernel workgroups per CU below 8 contributions, and from 8
// with fp32 and with 2-byte storage: more than the vector kernel's, whose
// loads it matches, to cover its extra exchange and shift instructions.
constexpr int kRedShiftPerCU = ZK_RED_SHIFT_PER_CU;
constexpr int kRedShiftPerCUMany = ZK_RED_SHIFT_PER_CU_MANY;
constexpr int kRedShiftPerCUMany2B = ZK_RED_SHIFT_PER_CU_MANY_2B;
// runs of one full residency of kRedRuns workgroups on 256 CUs
constexpr int64_t kRedSmallNvec = (int64_t)256 * ZK_RED_PER_CU * ZK_RED_BLOCK * ZK_RED_RUNS;
// The stand-alone scan reads a single stream, so it takes its own runs per
// lane and residency.
constexpr int kScanBlock = ZK_SCAN_BLOCK;
constexpr int kScanRuns = ZK_SCAN_RUNS;
constexpr int kScanPerCU = ZK_SCAN_PER_CU;
constexpr int kMin2(int a, int b) { return a < b ? a : b; }
// runs one vector reduce or scan workgroup covers at the least
constexpr int64_t kRunsPerBlockMin =
    kMin2(kMin2(kRedBlock * kMin2(kRedRuns, kRedRunsSmall), kRedBlockMany * kRedRunsMany),
          kScanBlock * kScanRuns);
constexpr int kRedPerCU = ZK_RED_PER_CU;
constexpr int kRedPerCUMany = ZK_RED_PER_CU_MANY;   // residency when 8 <= R < 16, fp32
constexpr int kRedPerCUMany2B = ZK_RED_PER_CU_MANY_2B;   // the same, 2-byte storage
constexpr int kRedPerCUWide = ZK_RED_PER_CU_WIDE;   // residency when R >= 16
constexpr int kRedWideR = 16;
// Adam: one wave (64 lanes) per workgroup, each lane one group of 4 elements;
// residency capped at 10 workgroups (10 waves) per CU.
constexpr int kAdamBlock = ZK_ADAM_BLOCK;
constexpr int kAdamGroups = ZK_ADAM_GROUPS;
constexpr int64_t kAdamElemsPerBlock = (int64_t)kAdamBlock * kAdamGroups * 4;  // 256
constexpr int kAdamPerCU = ZK_ADAM_PER_CU;
// SGD: one wave per workgroup, one group of 4 per lane like Adam, but it
// streams fewer arrays (3 with a momentum buffer, 2 without), so it keeps more
// waves resident to hold enough bytes in flight: 16 per CU with momentum, 24
// without (measured on MI355X; 10 per CU left plain SGD at 64% of peak).
constexpr int kSgdBlock = 64;
constexpr int kSgdMomGroups = ZK_SGD_MOM_GROUPS;
constexpr int kSgdMomPerCU = ZK_SGD_MOM_PER_CU;
constexpr int kSgdPlainGroups = ZK_SGD_PLAIN_GROUPS;
constexpr int kSgdPlainPerCU = ZK_SGD_PLAIN_PER_CU;
// Small shards (at most kSmallElems elements) keep their step's data in the
// caches (the 256 MiB Infinity Cache holds 8M elements' worth of an fp16 Adam
// step), and their steps are bound by launch and memory latency rather than by
// HBM bandwidth.  Every bucket reduce and the update of such a shard run
// 256-lane workgroups with one run or group per lane and plain (cached) loads
// and stores: the update then reads the gradient the reduce just stored from
// cache.  Measured on MI355X (device-resident fp16 Adam steps, R = 4, back to
// back): 7.45 -> 7.3 us at 262,144 elements, 13.4 -> 10.6 us at 1M, 33.4 ->
// 27.7 us at 4M, 59.1 -> 45.9 us at 8M; at 16M the streaming shapes below win.
#ifndef ZK_SMALL_ELEMS
#define ZK_SMALL_ELEMS (int64_t(1) << 23)
#endif
constexpr int64_t kSmallElems = ZK_SMALL_ELEMS;
#ifndef ZK_SMALL_BLOCK
#define ZK_SMALL_BLOCK 256
#endif
#ifndef ZK_SMALL_UPD_BLOCK
#define ZK_SMALL_UPD_BLOCK 256
#endif
constexpr int kSmallBlock = ZK_SMALL_BLOCK;         // reduce lanes per workgroup
constexpr int kSmallUpdBlock = ZK_SMALL_UPD_BLOCK;  // update lanes per workgroup
inline bool shard_small(int64_t S) { return S <= kSmallElems; }
// Lanes per workgroup and runs per lane of a bucket reduce (nvec runs, R
// contributions) of a small shard or not, in the vector or the shift kernel.
inline int red_block(int R, bool small)
{
    if (small) return kSmallBlock;
    return R >= kRedManyR ? kRedBlockMany : kRedBlock;
}
inline int red_runs(int R, int64_t nvec, bool small, bool shift = false)
{
    if (small) return 1;
    if (R >= kRedManyR) return kRedRunsMany;
    if (shift) return kRedShiftRuns;
    return nvec < kRedSmallNvec ? kRedRunsSmall : kRedRuns;
}
// The block of runs (and partial slot) workgroup b of n takes in the shift
// kernel, for groups of G workgroups.  Workgroups are dealt round-robin to the
// 8 XCDs; within each full set of 8 * G workgroups this hands XCD x
// (workgroups b = x mod 8) the G consecutive blocks x * G + (0 ..), so all XCDs
// still sweep one narrow front while neighbouring blocks mostly share an L2.
// A bijection on [0, n): the last, partial set keeps the plain order (as does
// G <= 1).
template <unsigned G>
__host__ __device__ inline unsigned shift_block(unsigned b, unsigned n)
{
    if constexpr (G <= 1) {
        (void)n;
        return b;
    } else {
        constexpr unsigned set = 8u * G;
        const unsigned s0 = b - b % set;
        if (s0 + set > n) return b;
        const unsigned j = b - s0;
        return s0 + (j % 8u) * G + j / 8u;
    }
}

// The shift kernel's group: kRedShiftGroupRuns wave-runs in workgroups of BS
// lanes with U runs per lane.
template <int BS, int U>
__host__ __device__ constexpr unsigned shift_group()
{
    return (unsigned)(kRedShiftGroupRuns / (U * (BS / 64)));
}

// Update of an S-element shard: lanes per workgroup and groups per lane.
inline int adam_lanes(int64_t S) { return shard_small(S) ? kSmallUpdBlock : kAdamBlock; }
inline int adam_groups(int64_t S) { return shard_small(S) ? 1 : kAdamGroups; }
inline int sgd_lanes(int64_t S) { return shard_small(S) ? kSmallUpdBlock : kSgdBlock; }
inline int sgd_groups(int64_t S, bool mom)
{
    return shard_small(S) ? 1 : (mom ? kSgdMomGroups : kSgdPlainGroups);
}
// Element-wise kernels (unaligned heads and tails, or arrays without a common
// alignment): 256 lanes, 8 elements per lane, lane-consecutive per step.
constexpr int kScalarBlock = 256;
constexpr int64_t kScalarElemsPerBlock = (int64_t)kScalarBlock * 8;
// Work-items per launch stay below 2^31; larger bodies are split into
// consecutive launches.
#ifndef ZK_MAX_LAUNCH_ITEMS
#define ZK_MAX_LAUNCH_ITEMS (int64_t(1) << 31)
#endif
constexpr int64_t kMaxLaunchItems = ZK_MAX_LAUNCH_ITEMS;
// Fixed-order fold of the per-workgroup partials.
constexpr int kFoldBlock = 256;
constexpr int kFoldMaxBlocks = 1024;
// At most this many partials are summed by one workgroup in one launch.
constexpr int64_t kFoldOneLevel = 4096;

struct ContribPtrs {
    const void* p[kMaxContrib];
};

// Result of a step's check, written by the last fold launch.
struct CheckResult {
    double sumsq;          // squared unscaled norm; NaN when an unscaled value was not finite
    float clip;            // global-norm clipping coefficient (1 when off or on overflow)
    float pad;
};

// Step state kept in device memory by the device-resident flow, so that a
// whole step (reduce, check, decision, update) runs without the host and can
// be captured in a graph.  The prepare kernel reads the check, decides, and
// advances the counters; the reduce reads inv_scale, the update upd_*.
struct DevState {
    double scale;          // loss scale the next step's gradients carry
    double pw1, pw2;       // products of the fp32-rounded betas over applied steps
    int64_t t;             // applied steps
    int64_t good;          // clean steps since the scale last changed
    int64_t steps_run;     // device steps prepared since the state was loaded
    double last_sumsq;     // the last step's check result (NaN: overflow)
    double last_scale;     // the loss scale the last step's gradients carried
    float inv_scale;       // fp32(1/scale) for the current step's check
    float upd_inv_scale;   // the same for the update of the step just decided
    float bc1, bc2;        // bias corrections of that update
    int32_t skip;          // 1: that update writes nothing
    int32_t pad;
};

// Constants of the prepare kernel (per handle).
struct PrepareArgs {
    double b1, b2;         // fp32-rounded betas, as fp64 factors
    double min_scale;
    int32_t bias_correction;
    int32_t dynamic;
    int64_t growth_interval;
};

// One bucket of the reduce.  Elements [0, n) of the bucket; the vector body
// starts at `head` and holds `nvec` 16-byte runs (8 two-byte or 4 fp32
// elements) that are 16-byte aligned in `out` and, with shift = 0, in every
// contribution.  shift = 1: each contribution keeps its own address phase
// modulo 16 bytes (the shift kernel cuts its runs out of aligned words), and
// head >= that phase in elements, with at least one whole run after the body.
// vec_ok = 0 selects the element-wise path.  Workgroup b writes
// partial[slot_base + b]: the fp64 sum of the squared unscaled stored values
// of its elements, or NaN if any unscaled value is not finite.  The unscale
// factor is inv_scale, or dev->inv_scale when dev is set.
struct ReduceLaunch {
    ContribPtrs c;
    void* out;
    int64_t n;
    int64_t head;
    int64_t nvec;
    int32_t R;
    int32_t lp;            // 1 fp16, 2 bf16, 3 fp32
    int32_t vec_ok;
    float inv_r;
    float inv_scale;
    double* partial;
    int64_t slot_base;
    uint32_t lds_reserve;  // dynamic LDS that caps workgroups per CU
    int32_t small;         // 1: a bucket of a small shard (see shard_small)
    int32_t shift;         // 1: contributions off the output's 16-byte phase (see above)
    // Element-wise part (the head [0, sc_a_len) and [sc_b_start, sc_b_start +
    // sc_b_len)) done by the last workgroup of the launch, one element per
    // lane, when sc_inline is set: the dispatch sets it on the last launch of
    // a vector body when the part fits one workgroup's lanes, and then runs no
    // element-wise kernel.
    int32_t sc_inline;
    int64_t sc_a_len, sc_b_start, sc_b_len;
    const DevState* dev;
    DevState* snapshot;    // set: workgroup 0 copies *dev there (see InlineFold)
};

// Stand-alone check of a stored gradient shard (no reduce this step).
struct ScanLaunch {
    const void* g;
    int64_t n;
    int64_t head;
    int64_t nvec;
    int32_t lp;
    int32_t vec_ok;
    float inv_scale;
    double* partial;
    int64_t slot_base;
    uint32_t lds_reserve;
    const DevState* dev;
    DevState* snapshot;
};

// The fold inside the update, for a device-resident step with few partials:
// every update workgroup sums the partials itself, in the fold kernel's order
// (so bitwise its sum), and takes the clipping coefficient and the decision
// from that sum and the step's starting state exactly as the fold's last lane
// would.  It reads that state from `snapshot`, the copy the step's reduce (or
// scan) launches made of `dev`, so workgroup 0 can write the advanced state to
// `dev` (and the check result) while the others still read: no counter, no
// atomics.  This saves the fold's launch on launch-bound shards.  The update
// must run as one vector launch with no element-wise part.
#ifndef ZK_INLINE_FOLD_MAX
#define ZK_INLINE_FOLD_MAX 1024
#endif
constexpr int kInlineFoldMax = ZK_INLINE_FOLD_MAX;   // 512 or 1024
static_assert(kInlineFoldMax == 512 || kInlineFoldMax == 1024, "fold of 2 or 4 loads per lane");
struct InlineFold {
    const double* partial;     // nullptr: off
    int32_t n;                 // partials, at most kInlineFoldMax
    int32_t pad;
    const DevState* snapshot;
    DevState* dev;
    CheckResult* res;
    double max_norm;
    PrepareArgs pa;
};

// Where an update takes its per-step values.  Host flows pass inv_scale (and
// the bias corrections) as arguments; res, when set, supplies the clipping
// coefficient (else `clip`), and with gate = 1 its NaN sum skips the update;
// dev, when set, supplies inv_scale, the bias corrections and the skip; fold,
// when set, replaces the fold kernel (see InlineFold).
struct StepSource {
    const CheckResult* res;
    const DevState* dev;
    int32_t gate;
    float clip;
    InlineFold fold;
};

enum WdKind { kWdNone = 0, kWdDecoupled = 1, kWdL2 = 2 };

// Adam over n elements: `head` scalar elements, then ngroups groups of 4
// elements aligned to 16 bytes in the fp32 arrays and 8 bytes in the 2-byte
// arrays, then a scalar tail.  vec_ok = 0 selects the element-wise path.
struct AdamLaunch {
    const void* grad;
    float* master;
    float* m;
    float* v;
    void* param;
    int64_t n;
    int64_t head;
    int64_t ngroups;
    int32_t lp;
    int32_t vec_ok;
    int32_t wd_kind;
    uint32_t lds_reserve;
    float b1, b2, omb1, omb2, bc1, bc2, lr, eps, wd, inv_scale;
    StepSource src;
};

// SGD over n elements, laid out like AdamLaunch.  mom == nullptr: plain SGD.
struct SgdLaunch {
    const void* grad;
    float* master;
    float* mom;
    void* param;
    int64_t n;
    int64_t head;
    int64_t ngroups;
    int32_t lp;
    int32_t vec_ok;
    int32_t has_wd;
    uint32_t lds_reserve;
    float lr, mu, wd, inv_scale;
    StepSource src;
};

// Elements per 16-byte run of a storage format: 8 two-byte or 4 fp32 values.
inline int run_width(int32_t lp) { return lp == 3 ? 4 : 8; }

// Partial slots a reduce / scan of this layout writes: one per workgroup of
// the vector kernel plus one per workgroup of the element-wise kernel, which a
// reduce (inline_scalars) does not launch when it has a vector body and at
// most BS element-wise elements (its last vector workgroup takes them).  W is
// the run width of the storage format, U the runs per lane and BS the lanes
// per workgroup (red_runs(R, nvec) and red_block(R) for a reduce, kScanRuns
// and kScanBlock for a scan).
int64_t reduce_blocks(int64_t n, int64_t head, int64_t nvec, int32_t vec_ok, int W, int U,
                      int BS, bool inline_scalars = false);

hipError_t launch_reduce(const ReduceLaunch& L, hipStream_t s);
hipError_t launch_scan(const ScanLaunch& L, hipStream_t s);
// Sum partial[0, nslots) in a fixed order into out->sumsq (one launch for up
// to kFoldOneLevel partials, else two) and set out->clip = min(1, max_norm /
// (sqrt(sumsq) + 1e-6)) in fp64, rounded to fp32 (1 when max_norm <= 0 or the
// sum is NaN).  dev set (device-resident flow): the same last lane then
// decides the step and advances the device state with pa.
hipError_t launch_finalize(const double* partial, int64_t nslots, double* level1,
                           CheckResult* out, double max_norm, DevState* dev,
                           const PrepareArgs& pa, hipStream_t s);
// Device-resident flow: write the state.
hipError_t launch_load_state(DevState* d, const DevState& init, hipStream_t s);
// Whether an update of ngroups groups of 4 with `lanes` lanes and `groups`
// groups per lane runs as one launch (the inline fold needs that).
inline bool one_launch(int64_t ngroups, int lanes, int groups)
{
    const int64_t blocks = (ngroups + (int64_t)lanes * groups - 1) / ((int64_t)lanes * groups);
    return blocks * lanes <= kMaxLaunchItems;
}
hipError_t launch_adam(const AdamLaunch& a, hipStream_t s);
hipError_t launch_sgd(const SgdLaunch& a, hipStream_t s);

}  // namespace zk
