// Latency of the device-resident step through the C ABI, with no Python: a
// small fp16 Adam shard (4 contributions of zeros, so every step applies),
// stepped by
//   1. direct enqueue, one zero_step_device per step;
//   2. replays of a HIP graph holding one captured step;
//   3. replays of a HIP graph holding ten captured steps.
// Prints the microseconds per step of each, and the step count the device
// state reports at the end (every step counted once: 6150).
// Usage: step_latency [shard elements]   (default 262144)
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "zero_shard.h"

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            std::fprintf(stderr, "%s:%d HIP error %s\n", __FILE__, __LINE__,           \
                         hipGetErrorString(e_));                                      \
            std::exit(2);                                                             \
        }                                                                             \
    } while (0)
#define CHECK_Z(x)                                                                    \
    do {                                                                              \
        zero_status s_ = (x);                                                         \
        if (s_ != ZERO_OK) {                                                          \
            std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__,                 \
                         zero_status_str(s_), zero_last_error());                     \
            std::exit(3);                                                             \
        }                                                                             \
    } while (0)

namespace {

constexpr int R = 4;
constexpr int kSteps = 2000;   // timed steps per mode
constexpr int kWarm = 50;      // untimed steps before each mode

using Clock = std::chrono::steady_clock;

double us_per(Clock::time_point a, Clock::time_point b, int n)
{
    return std::chrono::duration<double, std::micro>(b - a).count() / n;
}

}  // namespace

int main(int argc, char** argv)
{
    const int64_t S = argc > 1 ? std::atoll(argv[1]) : 262144;
    if (S < 1 || S > (int64_t(1) << 30)) {
        std::fprintf(stderr, "shard elements must lie in [1, 2^30]\n");
        return 1;
    }
    CHECK_HIP(hipSetDevice(0));
    float *master, *m, *v;
    uint16_t *grad, *param;
    uint16_t* contrib[R];
    CHECK_HIP(hipMalloc(&master, S * 4));
    CHECK_HIP(hipMalloc(&m, S * 4));
    CHECK_HIP(hipMalloc(&v, S * 4));
    CHECK_HIP(hipMalloc(&grad, S * 2));
    CHECK_HIP(hipMalloc(&param, S * 2));
    for (int r = 0; r < R; ++r) {
        CHECK_HIP(hipMalloc(&contrib[r], S * 2));
        CHECK_HIP(hipMemset(contrib[r], 0, S * 2));
    }
    CHECK_HIP(hipMemset(master, 0, S * 4));
    CHECK_HIP(hipMemset(m, 0, S * 4));
    CHECK_HIP(hipMemset(v, 0, S * 4));
    CHECK_HIP(hipMemset(param, 0, S * 2));
    hipStream_t st;
    CHECK_HIP(hipStreamCreate(&st));

    zero_shard_desc d{S, 1, 0, S, ZERO_FP16, master, m, v, grad, param};
    zero_adam_hparams hp{1e-3, 0.9, 0.999, 1e-8, 0.0, 1, ZERO_WD_DECOUPLED, 0};
    zero_loss_scale_cfg ls{1024.0, 1, 1000, 1.0};
    zero_shard_t h = nullptr;
    CHECK_Z(zero_shard_init(&d, &hp, &ls, &h));
    const void* cp[R];
    for (int r = 0; r < R; ++r) cp[r] = contrib[r];
    CHECK_Z(zero_device_begin(h, st));

    // 1. direct enqueue
    for (int k = 0; k < kWarm; ++k) CHECK_Z(zero_step_device(h, cp, R, st));
    CHECK_HIP(hipStreamSynchronize(st));
    const auto t0 = Clock::now();
    for (int k = 0; k < kSteps; ++k) CHECK_Z(zero_step_device(h, cp, R, st));
    CHECK_HIP(hipStreamSynchronize(st));
    const auto t1 = Clock::now();

    // 2. a graph holding one step
    hipGraph_t g1;
    hipGraphExec_t e1;
    CHECK_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
    CHECK_Z(zero_step_device(h, cp, R, st));
    CHECK_HIP(hipStreamEndCapture(st, &g1));
    CHECK_HIP(hipGraphInstantiate(&e1, g1, nullptr, nullptr, 0));
    for (int k = 0; k < kWarm; ++k) CHECK_HIP(hipGraphLaunch(e1, st));
    CHECK_HIP(hipStreamSynchronize(st));
    const auto t2 = Clock::now();
    for (int k = 0; k < kSteps; ++k) CHECK_HIP(hipGraphLaunch(e1, st));
    CHECK_HIP(hipStreamSynchronize(st));
    const auto t3 = Clock::now();

    // 3. a graph holding ten steps
    hipGraph_t g10;
    hipGraphExec_t e10;
    CHECK_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
    for (int k = 0; k < 10; ++k) CHECK_Z(zero_step_device(h, cp, R, st));
    CHECK_HIP(hipStreamEndCapture(st, &g10));
    CHECK_HIP(hipGraphInstantiate(&e10, g10, nullptr, nullptr, 0));
    for (int k = 0; k < kWarm / 10; ++k) CHECK_HIP(hipGraphLaunch(e10, st));
    CHECK_HIP(hipStreamSynchronize(st));
    const auto t4 = Clock::now();
    for (int k = 0; k < kSteps / 10; ++k) CHECK_HIP(hipGraphLaunch(e10, st));
    CHECK_HIP(hipStreamSynchronize(st));
    const auto t5 = Clock::now();

    zero_step_info info;
    CHECK_Z(zero_device_end(h, st, &info));
    CHECK_HIP(hipGraphExecDestroy(e1));
    CHECK_HIP(hipGraphDestroy(g1));
    CHECK_HIP(hipGraphExecDestroy(e10));
    CHECK_HIP(hipGraphDestroy(g10));
    CHECK_Z(zero_shard_destroy(h));
    for (int r = 0; r < R; ++r) CHECK_HIP(hipFree(contrib[r]));
    CHECK_HIP(hipFree(master));
    CHECK_HIP(hipFree(m));
    CHECK_HIP(hipFree(v));
    CHECK_HIP(hipFree(grad));
    CHECK_HIP(hipFree(param));
    CHECK_HIP(hipStreamDestroy(st));
    std::printf("S=%lld direct_us=%.2f graph1_us=%.2f graph10_us=%.2f step_t=%lld overflow=%d\n",
                (long long)S, us_per(t0, t1, kSteps), us_per(t2, t3, kSteps),
                us_per(t4, t5, kSteps), (long long)info.step_t, info.overflow);
    return 0;
}
