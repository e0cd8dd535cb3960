// Plain device-to-device copy used by the benchmark as the achievable-HBM
// ceiling of this GPU for a stream that reads and writes equal bytes, and as
// the known-size reference that calibrates the rocprofv3 byte counters.  Not
// part of the owner-rank step.
//
// Shape: the fastest plain copy measured on MI355X (8e9 bytes of random bits,
// nontemporal loads and stores, interleaved sweeps on one box): one-wave
// workgroups, each lane one 16-byte vector, residency capped at 32 workgroups
// per CU by reserving dynamic LDS the kernel never touches.  It moved
// 6.66-6.70 TB/s, against 6.57-6.61 TB/s for four vectors per lane at 16 per
// CU, 6.45-6.53 TB/s at 24 per CU and 6.45 TB/s for 256-lane workgroups at 8
// per CU.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 64;
constexpr int kRuns = 1;
constexpr int kPerCU = 32;

__global__ __launch_bounds__(kBlock) void hbm_copy_kernel(const f4* __restrict__ src,
                                                          f4* __restrict__ dst, int64_t n16)
{
    const int64_t base = (int64_t)blockIdx.x * (kBlock * kRuns) + threadIdx.x;
    f4 x[kRuns];
#pragma unroll
    for (int u = 0; u < kRuns; ++u) {
        const int64_t i = base + u * kBlock;
        if (i < n16) x[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kRuns; ++u) {
        const int64_t i = base + u * kBlock;
        if (i < n16) __builtin_nontemporal_store(x[u], dst + i);
    }
}

}  // namespace

// Copy `bytes` bytes (a multiple of 16, both pointers 16-byte aligned, at most
// 2^34 bytes, so at most 2^30 work-items) from src to dst on `stream`, on the
// current device.  Returns 0 on success, 1 on a bad argument, 2 on a HIP error.
extern "C" int hbm_copy(void* dst, const void* src, int64_t bytes, void* stream)
{
    if (!dst || !src || bytes <= 0 || (bytes & 15) || ((uintptr_t)dst & 15) ||
        ((uintptr_t)src & 15) || bytes > (int64_t(1) << 34))
        return 1;
    int dev = 0, lds_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess)
        return 2;
    int64_t lds = (int64_t)lds_cu / kPerCU - 1024;
    if (lds < 0) lds = 0;
    lds &= ~(int64_t)511;
    const int64_t n16 = bytes / 16;
    const int64_t grid = (n16 + kBlock * kRuns - 1) / (kBlock * kRuns);
    hbm_copy_kernel<<<(unsigned)grid, kBlock, (unsigned)lds, static_cast<hipStream_t>(stream)>>>(
        static_cast<const f4*>(src), static_cast<f4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
