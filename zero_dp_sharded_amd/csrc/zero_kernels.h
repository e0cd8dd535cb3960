// Internal launch interface between the C ABI (zero_shard.cpp) and the gfx950
// kernels (zero_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zk {

constexpr int kMaxContrib = 64;
constexpr int kBlock = 256;           // 4 wave64 per workgroup
constexpr int kSlots = 4096;          // per-block partial slots of the check

struct ContribPtrs {
    const void* p[kMaxContrib];
};

// One bucket of the reduce.  Elements [0, n) of the bucket; the vector body
// starts at `head` and holds `nvec` runs of 8 elements that are 16-byte aligned
// in every contribution and in `out`.  vec_ok = 0 selects the element-wise path.
struct ReduceLaunch {
    ContribPtrs c;
    void* out;
    int64_t n;
    int64_t head;
    int64_t nvec;
    int32_t R;
    int32_t lp;            // 1 fp16, 2 bf16
    int32_t vec_ok;
    int32_t first;         // first bucket of the step: slots are overwritten
    float inv_r;
    float inv_scale;
    double* part_sumsq;    // kSlots
    int32_t* part_flag;    // kSlots
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
    double* part_sumsq;
    int32_t* part_flag;
};

struct CheckResult {
    double sumsq;
    int32_t flag;
    int32_t pad;
};

enum WdKind { kWdNone = 0, kWdDecoupled = 1, kWdL2 = 2 };

struct AdamLaunch {
    const void* grad;
    float* master;
    float* m;
    float* v;
    void* param;
    int64_t n;
    int64_t head;
    int64_t nvec;
    int32_t lp;
    int32_t vec_ok;
    int32_t wd_kind;
    float b1, b2, omb1, omb2, bc1, bc2, lr, eps, wd, inv_scale;
};

hipError_t launch_reduce(const ReduceLaunch& L, hipStream_t s);
hipError_t launch_scan(const ScanLaunch& L, hipStream_t s);
hipError_t launch_finalize(const double* part_sumsq, const int32_t* part_flag,
                           CheckResult* out, hipStream_t s);
hipError_t launch_adam(const AdamLaunch& L, hipStream_t s);

}  // namespace zk
