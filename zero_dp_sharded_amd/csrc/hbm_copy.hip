// Plain device-to-device copy used by the benchmark as the achievable-HBM
// ceiling of this GPU and as the known-size reference that calibrates the
// rocprofv3 byte counters.  Not part of the owner-rank step.
//
// Shape: the fastest plain copy measured on MI355X, one 16-byte vector per
// lane on an exact grid of 256-lane workgroups, nontemporal loads and stores.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void hbm_copy_kernel(const f4* __restrict__ src,
                                                       f4* __restrict__ dst, int64_t n16)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

// Copy `bytes` bytes (a multiple of 16, both pointers 16-byte aligned, at most
// 2^40 bytes) from src to dst on `stream`.  Returns 0 on success, 1 on a bad
// argument, 2 on a HIP launch error.
extern "C" int hbm_copy(void* dst, const void* src, int64_t bytes, void* stream)
{
    if (!dst || !src || bytes <= 0 || (bytes & 15) || ((uintptr_t)dst & 15) ||
        ((uintptr_t)src & 15) || bytes > (int64_t(1) << 40))
        return 1;
    const int64_t n16 = bytes / 16;
    const int64_t grid = (n16 + 255) / 256;
    hbm_copy_kernel<<<(unsigned)grid, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const f4*>(src), static_cast<f4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
