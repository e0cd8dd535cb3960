// A native user of libzeroshard.so: plain HIP memory and streams, no torch,
// no Python.  Runs steps of an fp16 Adam shard through the C ABI in four
// ways and checks every one against the oracle (linked in from oracle/, test
// infrastructure), bitwise:
//   1. the synchronous check flow (bucket reduces, check, Adam);
//   2. the device-resident flow, one zero_step_device per step;
//   3. the device-resident step captured once with the HIP graph API
//      (hipStreamBeginCapture / hipGraphInstantiate) and replayed per step;
//   4. the allocation-free step (zero_adam_step_noalloc: no handle, the
//      counters carried by the caller), the form for callers that cannot
//      allocate device memory.
// Exit status 0 and a last line "abi_example ok" on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "zero_shard.h"

// the oracle's C entry points (oracle/zero_oracle.c)
extern "C" {
void oracle_bucket_reduce(int lp, int32_t n_contrib, const void* const* contribs, int64_t n,
                          void* out);
void oracle_flag_sumsq(int lp, const void* g, int64_t n, float inv_scale, int32_t* flag,
                       double* sumsq);
void oracle_adam_scalars(double beta1, double beta2, double lr, double eps, double weight_decay,
                         int32_t bias_correction, int64_t t, double loss_scale, float* out);
void oracle_adam_update(int lp, int64_t n, const void* grad, float* master, float* exp_avg,
                        float* exp_avg_sq, void* param, const float* sc, int32_t wd_mode);
uint16_t oracle_f32_to_f16(float x);
}

namespace {

constexpr int kFp16 = 1;
constexpr int64_t S = 100003;      // shard elements (ragged against every tile)
constexpr int R = 3;                // contributions
constexpr int64_t CB = 40000;       // bucket elements: 3 buckets, the last ragged
constexpr int kSteps = 3;
constexpr double kScale = 1024.0;

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

// deterministic pseudo-random fp32 in [-1, 1) (xorshift)
struct Rng {
    uint64_t s;
    float next()
    {
        s ^= s << 13;
        s ^= s >> 7;
        s ^= s << 17;
        return (float)((int64_t)(s >> 40) - (1 << 23)) / (float)(1 << 23);
    }
};

struct Host {
    std::vector<float> master, m, v;
    std::vector<uint16_t> param;
    int64_t t = 0;
};

// contributions of step `step`: fp16(N-ish(0, 1e-3) * scale)
std::vector<std::vector<uint16_t>> contributions(int step)
{
    std::vector<std::vector<uint16_t>> c(R, std::vector<uint16_t>(S));
    for (int r = 0; r < R; ++r) {
        Rng g{0x9e3779b97f4a7c15ull * (uint64_t)(step * 16 + r + 1)};
        for (int64_t i = 0; i < S; ++i) c[r][i] = oracle_f32_to_f16(g.next() * 1e-3f * (float)kScale);
    }
    return c;
}

// one oracle step on the host copy (no overflow in these inputs)
void oracle_step(Host& h, const std::vector<std::vector<uint16_t>>& c, const zero_adam_hparams& hp)
{
    std::vector<uint16_t> grad(S);
    for (int64_t off = 0; off < S; off += CB) {
        const int64_t len = S - off < CB ? S - off : CB;
        const void* p[R];
        for (int r = 0; r < R; ++r) p[r] = c[r].data() + off;
        oracle_bucket_reduce(kFp16, R, p, len, grad.data() + off);
    }
    int32_t flag = 0;
    double ss = 0.0;
    oracle_flag_sumsq(kFp16, grad.data(), S, (float)(1.0 / kScale), &flag, &ss);
    if (flag) {
        std::fprintf(stderr, "unexpected overflow in the oracle\n");
        std::exit(4);
    }
    h.t += 1;
    float sc[11];
    oracle_adam_scalars(hp.beta1, hp.beta2, hp.lr, hp.eps, hp.weight_decay, hp.bias_correction,
                        h.t, kScale, sc);
    sc[10] = 1.0f;
    oracle_adam_update(kFp16, S, grad.data(), h.master.data(), h.m.data(), h.v.data(),
                       h.param.data(), sc, hp.wd_mode);
}

int failures = 0;

void expect_equal(const char* what, const void* a, const void* b, size_t bytes)
{
    if (std::memcmp(a, b, bytes) != 0) {
        std::fprintf(stderr, "MISMATCH: %s\n", what);
        ++failures;
    }
}

}  // namespace

int main()
{
    int ndev = 0;
    CHECK_HIP(hipGetDeviceCount(&ndev));
    if (ndev < 1) {
        std::fprintf(stderr, "no GPU\n");
        return 2;
    }
    CHECK_HIP(hipSetDevice(0));
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));

    // initial state: master ~ U(-0.02, 0.02), m = v = 0
    Host init;
    init.master.resize(S);
    init.m.assign(S, 0.0f);
    init.v.assign(S, 0.0f);
    init.param.resize(S);
    Rng g{12345};
    for (int64_t i = 0; i < S; ++i) {
        init.master[i] = g.next() * 0.02f;
        init.param[i] = oracle_f32_to_f16(init.master[i]);
    }
    zero_adam_hparams hp;
    std::memset(&hp, 0, sizeof(hp));
    hp.lr = 1e-3;
    hp.beta1 = 0.9;
    hp.beta2 = 0.999;
    hp.eps = 1e-8;
    hp.weight_decay = 0.01;
    hp.bias_correction = 1;
    hp.wd_mode = ZERO_WD_DECOUPLED;
    zero_loss_scale_cfg ls{kScale, 1, 1000, 1.0};

    // the oracle's trajectory
    Host ref = init;
    std::vector<std::vector<std::vector<uint16_t>>> steps;
    for (int s = 0; s < kSteps; ++s) {
        steps.push_back(contributions(s));
        oracle_step(ref, steps.back(), hp);
    }

    // device arrays
    float *master, *m, *v;
    uint16_t *grad, *param;
    uint16_t* contrib[R];
    CHECK_HIP(hipMalloc(&master, S * 4));
    CHECK_HIP(hipMalloc(&m, S * 4));
    CHECK_HIP(hipMalloc(&v, S * 4));
    CHECK_HIP(hipMalloc(&grad, S * 2));
    CHECK_HIP(hipMalloc(&param, S * 2));
    for (int r = 0; r < R; ++r) CHECK_HIP(hipMalloc(&contrib[r], S * 2));

    for (int mode = 0; mode < 4; ++mode) {
        CHECK_HIP(hipMemcpy(master, init.master.data(), S * 4, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(m, init.m.data(), S * 4, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(v, init.v.data(), S * 4, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(param, init.param.data(), S * 2, hipMemcpyHostToDevice));
        zero_shard_desc d{S, 1, 0, CB, ZERO_FP16, master, m, v, grad, param};
        zero_shard_t h = nullptr;
        if (mode < 3) CHECK_Z(zero_shard_init(&d, &hp, &ls, &h));
        int64_t t = 0, good = 0;          // the counters the allocation-free step carries
        double scale = kScale;
        const void* cp[R];
        for (int r = 0; r < R; ++r) cp[r] = contrib[r];
        hipGraphExec_t exec = nullptr;
        hipGraph_t graph = nullptr;
        zero_step_info info;
        if (mode == 1 || mode == 2) CHECK_Z(zero_device_begin(h, stream));
        for (int s = 0; s < kSteps; ++s) {
            for (int r = 0; r < R; ++r)
                CHECK_HIP(hipMemcpyAsync(contrib[r], steps[s][r].data(), S * 2, hipMemcpyHostToDevice,
                                         stream));
            CHECK_HIP(hipStreamSynchronize(stream));
            if (mode == 0) {
                for (int64_t off = 0; off < S; off += CB) {
                    const int64_t len = S - off < CB ? S - off : CB;
                    const void* p[R];
                    for (int r = 0; r < R; ++r) p[r] = contrib[r] + off;
                    CHECK_Z(zero_bucket_reduce(h, p, R, off, len, stream));
                }
                CHECK_Z(zero_overflow_check(h, stream, &info));
                CHECK_Z(zero_adam_step(h, nullptr, stream, &info));
            } else if (mode == 1) {
                CHECK_Z(zero_step_device(h, cp, R, stream));
            } else if (mode == 3) {
                CHECK_Z(zero_adam_step_noalloc(&d, &hp, &ls, 0.0, cp, R, &t, &scale, &good, stream,
                                               &info));
            } else {
                if (exec == nullptr) {
                    // capture the whole step once; every replay is one step
                    CHECK_HIP(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
                    CHECK_Z(zero_step_device(h, cp, R, stream));
                    CHECK_HIP(hipStreamEndCapture(stream, &graph));
                    CHECK_HIP(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
                }
                CHECK_HIP(hipGraphLaunch(exec, stream));
            }
            CHECK_HIP(hipStreamSynchronize(stream));
        }
        if (mode == 1 || mode == 2) CHECK_Z(zero_device_end(h, stream, &info));
        if (mode == 3 && (t != kSteps || scale != kScale || good != kSteps)) {
            std::fprintf(stderr, "allocation-free step: counters %lld %g %lld\n", (long long)t,
                         scale, (long long)good);
            ++failures;
        }
        if (exec) CHECK_HIP(hipGraphExecDestroy(exec));
        if (graph) CHECK_HIP(hipGraphDestroy(graph));
        if (info.overflow != 0 || info.step_t != kSteps) {
            std::fprintf(stderr, "mode %d: overflow %d step_t %lld\n", mode, info.overflow,
                         (long long)info.step_t);
            ++failures;
        }
        Host got;
        got.master.resize(S);
        got.m.resize(S);
        got.v.resize(S);
        got.param.resize(S);
        CHECK_HIP(hipMemcpy(got.master.data(), master, S * 4, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(got.m.data(), m, S * 4, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(got.v.data(), v, S * 4, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(got.param.data(), param, S * 2, hipMemcpyDeviceToHost));
        const char* names[4] = {"synchronous flow", "device-resident flow", "graph replays",
                                "allocation-free step"};
        char what[96];
        std::snprintf(what, sizeof(what), "%s: master", names[mode]);
        expect_equal(what, got.master.data(), ref.master.data(), S * 4);
        std::snprintf(what, sizeof(what), "%s: m", names[mode]);
        expect_equal(what, got.m.data(), ref.m.data(), S * 4);
        std::snprintf(what, sizeof(what), "%s: v", names[mode]);
        expect_equal(what, got.v.data(), ref.v.data(), S * 4);
        std::snprintf(what, sizeof(what), "%s: param", names[mode]);
        expect_equal(what, got.param.data(), ref.param.data(), S * 2);
        if (h) CHECK_Z(zero_shard_destroy(h));
        std::printf("%s: %d steps, bitwise equal to the oracle: %s\n", names[mode], kSteps,
                    failures ? "no" : "yes");
    }
    for (int r = 0; r < R; ++r) CHECK_HIP(hipFree(contrib[r]));
    CHECK_HIP(hipFree(master));
    CHECK_HIP(hipFree(m));
    CHECK_HIP(hipFree(v));
    CHECK_HIP(hipFree(grad));
    CHECK_HIP(hipFree(param));
    CHECK_HIP(hipStreamDestroy(stream));
    if (failures) {
        std::printf("abi_example FAILED (%d)\n", failures);
        return 1;
    }
    std::printf("abi_example ok\n");
    return 0;
}
