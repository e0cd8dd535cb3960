// C ABI of the owner-rank ZeRO-DP step: argument validation, the per-step
// phase machine (reduce buckets -> check -> Adam), the host scalars of each
// Adam step, loss-scale bookkeeping, and the kernel launches.
//
// Method: "ZeRO：大模型训练的内存优化革命" 3.1.1 (each process updates its 1/Nd of
// the optimizer state, then parameters are all-gathered) and 3.1.2 (gradients
// reduced on the owner of the partition); 3.2.2 (constant-size buffers).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>

#include "../../include/zero_shard.h"
#include "zero_kernels.h"
#include "zero_layout.h"

namespace {

thread_local char g_last_error[512] = "";

zero_status fail(zero_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

zero_status hip_fail(hipError_t e, const char* what)
{
    return fail(ZERO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

enum Phase { kIdle = 0, kReducing = 1, kChecked = 2, kPending = 3 };
enum Opt { kOptAdam = 0, kOptSgd = 1 };

}  // namespace

struct zero_shard_s {
    int device = -1;
    zero_shard_desc d{};
    int64_t S = 0;
    Opt opt = kOptAdam;
    int esz = 2;                  // bytes per stored gradient / param element
    zero_adam_hparams hp{};       // Adam handles
    zero_sgd_hparams sgd{};       // SGD handles
    zero_loss_scale_cfg ls{};
    // step state
    int64_t t = 0;
    double scale = 1.0;
    int64_t good_steps = 0;
    // beta^t cache for the init betas: product of t fp32-rounded betas in fp64
    double pw1 = 1.0, pw2 = 1.0;
    int64_t pw_t = 0;
    Phase phase = kIdle;
    int64_t covered = 0;
    zero_step_info check{};
    int64_t slot_cursor = 0;      // partial slots written this step
    // device workspace: per-workgroup partials, the fold's first level and
    // the check result; pinned host copy of the result
    void* ws = nullptr;
    int64_t nslots = 0;
    double* partial = nullptr;
    double* level1 = nullptr;
    zk::CheckResult* result = nullptr;
    zk::CheckResult* host_result = nullptr;
    // dynamic LDS reserved per workgroup to cap residency per CU
    uint32_t lds_adam = 0;
    uint32_t lds_sgd_mom = 0;
    uint32_t lds_sgd_plain = 0;
    uint32_t lds_reduce = 0;
    uint32_t lds_reduce_many = 0;   // reduces of 8 <= R < 16 contributions
    uint32_t lds_reduce_wide = 0;   // reduces of R >= 16 contributions
    uint32_t lds_shift = 0;         // shift-kernel reduces of R < 8 contributions
    uint32_t lds_shift_many = 0;    // and of R >= 8
    uint32_t lds_scan = 0;
    // gated steps: event after the result copy, and the speculative update
    hipEvent_t result_ready = nullptr;
    double pend_pw1 = 1.0, pend_pw2 = 1.0;
    bool pend_same_betas = false;
    // global-norm clipping limit (0: off); a merged step's coefficient
    double max_norm = 0.0;
    bool merged = false;
    float merge_clip = 1.0f;
    // device-resident flow: the step state in device memory, its pinned copy
    zk::DevState* dev = nullptr;
    zk::DevState* host_dev = nullptr;
    bool device_mode = false;
    // the step's starting state as the reduce copies it for an inline-fold
    // update (device memory), and the device steps enqueued with that fold
    zk::DevState* dev_snapshot = nullptr;
    int64_t inline_folds = 0;
    // the contribution set zero_step_device last validated
    const void* dev_checked[ZERO_MAX_CONTRIB] = {};
    int32_t dev_checked_n = 0;
};

namespace {

std::mutex g_live_mu;
std::unordered_set<zero_shard_s*> g_live;

bool live(zero_shard_t h)
{
    std::lock_guard<std::mutex> lk(g_live_mu);
    return h != nullptr && g_live.count(h) != 0;
}

bool finite_pos(double x) { return std::isfinite(x) && x > 0.0; }

// A caller's enum field through its 32-bit representation: a value outside the
// enumerators is then an ordinary integer to refuse, not an out-of-range enum
// load (undefined in C++).  Fields are read this way until validated.
template <typename E>
int32_t enum_value(const E& e)
{
    static_assert(sizeof(E) == sizeof(int32_t), "32-bit enum");
    int32_t v;
    std::memcpy(&v, &e, sizeof(v));
    return v;
}

// A loss scale the kernels can unscale by: finite, positive, and with an fp32
// reciprocal that is neither 0 nor inf.
bool scale_ok(double s)
{
    if (!finite_pos(s)) return false;
    const float inv = (float)(1.0 / s);
    return std::isfinite(inv) && inv > 0.0f;
}

// Calls that launch work must run with the handle's device current and, for a
// non-default stream, on a stream of that device; otherwise the kernels would
// reach this device's arrays from another GPU.
zero_status check_device(const zero_shard_s* h, void* stream, const char* who)
{
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, who);
    if (cur != h->device)
        return fail(ZERO_ERR_STATE, "%s: the handle belongs to device %d but device %d is current",
                    who, h->device, cur);
    if (stream) {
        int sd = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd) != hipSuccess)
            (void)hipGetLastError();
        else if (sd != h->device)
            return fail(ZERO_ERR_INVALID_ARG, "%s: the stream belongs to device %d, the handle to %d",
                        who, sd, h->device);
    }
    return ZERO_OK;
}

zero_status check_hparams(const zero_adam_hparams* hp)
{
    if (!hp) return fail(ZERO_ERR_INVALID_ARG, "adam hparams: NULL");
    if (!(std::isfinite(hp->lr) && hp->lr >= 0.0))
        return fail(ZERO_ERR_INVALID_ARG, "adam hparams: lr must be finite and >= 0");
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
        return fail(ZERO_ERR_INVALID_ARG, "adam hparams: betas must lie in [0, 1)");
    // the kernels use the fp32 roundings; a beta within 3e-8 of 1 rounds to 1,
    // its bias correction 1 - beta^t to 0, and the update to NaN
    if (!((float)hp->beta1 < 1.0f) || !((float)hp->beta2 < 1.0f))
        return fail(ZERO_ERR_INVALID_ARG, "adam hparams: betas must stay below 1 in fp32");
    if (!finite_pos(hp->eps) || (float)hp->eps <= 0.0f)
        return fail(ZERO_ERR_INVALID_ARG, "adam hparams: eps must be > 0 in fp32");
    if (!(std::isfinite(hp->weight_decay) && hp->weight_decay >= 0.0))
        return fail(ZERO_ERR_INVALID_ARG, "adam hparams: weight_decay must be finite and >= 0");
    if (hp->bias_correction != 0 && hp->bias_correction != 1)
        return fail(ZERO_ERR_INVALID_ARG, "adam hparams: bias_correction must be 0 or 1");
    const int32_t wd_mode = enum_value(hp->wd_mode);
    if (wd_mode != ZERO_WD_DECOUPLED && wd_mode != ZERO_WD_L2)
        return fail(ZERO_ERR_INVALID_ARG, "adam hparams: unknown wd_mode %d", (int)wd_mode);
    if (hp->initial_step < 0)
        return fail(ZERO_ERR_INVALID_ARG, "adam hparams: initial_step must be >= 0");
    return ZERO_OK;
}

zero_status check_ls(const zero_loss_scale_cfg* ls)
{
    if (!ls) return fail(ZERO_ERR_INVALID_ARG, "loss scale: NULL");
    if (!scale_ok(ls->init_scale) || !scale_ok(ls->min_scale))
        return fail(ZERO_ERR_INVALID_ARG,
                    "loss scale: init_scale and min_scale must be finite and > 0 with a finite, "
                    "non-zero fp32 reciprocal");
    if (ls->dynamic != 0 && ls->dynamic != 1)
        return fail(ZERO_ERR_INVALID_ARG, "loss scale: dynamic must be 0 or 1");
    if (ls->growth_interval < 1)
        return fail(ZERO_ERR_INVALID_ARG, "loss scale: growth_interval must be >= 1");
    return ZERO_OK;
}

zero_status check_sgd_hparams(const zero_sgd_hparams* hp, bool has_buffer)
{
    if (!hp) return fail(ZERO_ERR_INVALID_ARG, "sgd hparams: NULL");
    if (!(std::isfinite(hp->lr) && hp->lr >= 0.0))
        return fail(ZERO_ERR_INVALID_ARG, "sgd hparams: lr must be finite and >= 0");
    if (!(hp->momentum >= 0.0 && hp->momentum < 1.0))
        return fail(ZERO_ERR_INVALID_ARG, "sgd hparams: momentum must lie in [0, 1)");
    if (hp->momentum != 0.0 && !has_buffer)
        return fail(ZERO_ERR_INVALID_ARG, "sgd hparams: momentum != 0 needs a momentum buffer (exp_avg)");
    if (!(std::isfinite(hp->weight_decay) && hp->weight_decay >= 0.0))
        return fail(ZERO_ERR_INVALID_ARG, "sgd hparams: weight_decay must be finite and >= 0");
    if (hp->initial_step < 0)
        return fail(ZERO_ERR_INVALID_ARG, "sgd hparams: initial_step must be >= 0");
    return ZERO_OK;
}

// Bytes per stored gradient / parameter element of a storage format.
int lp_bytes(zero_lp_dtype lp) { return lp == ZERO_FP32 ? 4 : 2; }

// Dynamic LDS that leaves room for `per_cu` workgroups of a kernel per CU.
uint32_t lds_reserve_for(int lds_per_cu, int lds_per_block_max, int per_cu)
{
    int64_t r = (int64_t)lds_per_cu / per_cu - 1024;   // room for static LDS
    if (r > lds_per_block_max) r = lds_per_block_max;
    if (r < 0) r = 0;
    return (uint32_t)(r & ~(int64_t)511);
}

// beta^t as a product of t copies of (double)(float)beta, as the header says.
double beta_pow(double beta, int64_t t)
{
    const double b = (double)(float)beta;
    double p = 1.0;
    for (int64_t k = 0; k < t; ++k) p = p * b;
    return p;
}

void next_scale(zero_shard_s* h, int overflow, double* scale, int64_t* good)
{
    double s = h->scale;
    int64_t g = h->good_steps;
    if (h->ls.dynamic) {
        if (overflow) {
            s = s / 2.0;
            if (s < h->ls.min_scale) s = h->ls.min_scale;
            g = 0;
        } else {
            g += 1;
            if (g == h->ls.growth_interval) {
                s = s * 2.0;
                g = 0;
            }
        }
    }
    *scale = s;
    *good = g;
}

bool overlaps(uintptr_t a, size_t na, uintptr_t b, size_t nb)
{
    return a < b + nb && b < a + na;
}

// Whether [p, p + nbytes) may be handed to the kernels of device `dev`: the
// runtime must not report it as unregistered host memory or as another
// device's memory, and where it knows the allocation's extent the range must
// end inside it.  Best effort: memory the runtime cannot classify (for
// example, ranges mapped through the virtual-memory API) is accepted.
bool device_range_ok(const void* p, size_t nbytes, int dev, char* why, size_t why_len)
{
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    if (a.type == hipMemoryTypeUnregistered) {
        snprintf(why, why_len, "is not device-accessible memory (pageable host memory?)");
        return false;
    }
    if (a.type == hipMemoryTypeDevice) {
        if (a.device != dev) {
            snprintf(why, why_len, "is memory of device %d, the handle's is %d", a.device, dev);
            return false;
        }
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) == hipSuccess) {
            if ((uintptr_t)p + nbytes > (uintptr_t)base + size) {
                snprintf(why, why_len, "runs %zu bytes past the end of its allocation",
                         (size_t)((uintptr_t)p + nbytes - ((uintptr_t)base + size)));
                return false;
            }
        } else {
            (void)hipGetLastError();
        }
    }
    return true;
}

}  // namespace

extern "C" {

int zero_abi_version(void) { return ZERO_SHARD_ABI_VERSION; }

const char* zero_last_error(void) { return g_last_error; }

const char* zero_status_str(zero_status s)
{
    switch (s) {
    case ZERO_OK: return "ZERO_OK";
    case ZERO_ERR_INVALID_ARG: return "ZERO_ERR_INVALID_ARG";
    case ZERO_ERR_STATE: return "ZERO_ERR_STATE";
    case ZERO_ERR_HIP: return "ZERO_ERR_HIP";
    case ZERO_ERR_OOM: return "ZERO_ERR_OOM";
    case ZERO_ERR_UNSUPPORTED: return "ZERO_ERR_UNSUPPORTED";
    }
    return "ZERO_ERR_UNKNOWN";
}

}  // extern "C"

// Host checks of a shard descriptor (no device access).  `need_m` /
// `need_v`: whether exp_avg / exp_avg_sq must be given (1), must be NULL (-1)
// or may be either (0).  Sets *S_out.
static zero_status check_desc(const zero_shard_desc& d, int need_m, int need_v, const char* who,
                              int64_t* S_out)
{
    if (d.psi < 1) return fail(ZERO_ERR_INVALID_ARG, "%s: psi must be >= 1", who);
    if (d.nd < 1) return fail(ZERO_ERR_INVALID_ARG, "%s: nd must be >= 1", who);
    if (d.rank < 0 || d.rank >= d.nd) return fail(ZERO_ERR_INVALID_ARG, "%s: rank outside [0, nd)", who);
    if (d.bucket_elems < 1) return fail(ZERO_ERR_INVALID_ARG, "%s: bucket_elems must be >= 1", who);
    const int32_t lp = enum_value(d.lp);
    if (lp != ZERO_FP16 && lp != ZERO_BF16 && lp != ZERO_FP32)
        return fail(ZERO_ERR_INVALID_ARG, "%s: unknown lp dtype %d", who, (int)lp);
    const bool fp32 = d.lp == ZERO_FP32;
    if (!d.master || !d.grad_shard) return fail(ZERO_ERR_INVALID_ARG, "%s: NULL master or grad_shard", who);
    if (fp32 && d.param_shard)
        return fail(ZERO_ERR_INVALID_ARG, "%s: param_shard must be NULL with fp32 storage", who);
    if (!fp32 && !d.param_shard) return fail(ZERO_ERR_INVALID_ARG, "%s: NULL param_shard", who);
    if ((need_m > 0 && !d.exp_avg) || (need_v > 0 && !d.exp_avg_sq))
        return fail(ZERO_ERR_INVALID_ARG, "%s: NULL optimizer state array", who);
    if ((need_m < 0 && d.exp_avg) || (need_v < 0 && d.exp_avg_sq))
        return fail(ZERO_ERR_INVALID_ARG, "%s: this optimizer takes no %s", who,
                    need_m < 0 && d.exp_avg ? "exp_avg" : "exp_avg_sq");
    const int esz = lp_bytes(d.lp);
    const int64_t S = (d.psi + d.nd - 1) / d.nd;
    // every given array: address, element size, bytes
    const void* arr[5] = {d.master, d.exp_avg, d.exp_avg_sq, d.grad_shard, d.param_shard};
    const int el[5] = {4, 4, 4, esz, esz};
    for (int i = 0; i < 5; ++i)
        if (arr[i] && ((uintptr_t)arr[i] % (uintptr_t)el[i]) != 0)
            return fail(ZERO_ERR_INVALID_ARG, "%s: shard array %d not %d-byte aligned", who, i, el[i]);
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (arr[i] && arr[j] &&
                overlaps((uintptr_t)arr[i], (size_t)S * el[i], (uintptr_t)arr[j], (size_t)S * el[j]))
                return fail(ZERO_ERR_INVALID_ARG, "%s: shard arrays %d and %d overlap", who, i, j);
    *S_out = S;
    return ZERO_OK;
}

// The runtime's view of the shard arrays (see device_range_ok).
static zero_status check_desc_ranges(const zero_shard_desc& d, int64_t S, int dev, const char* who)
{
    const int esz = lp_bytes(d.lp);
    const void* arr[5] = {d.master, d.exp_avg, d.exp_avg_sq, d.grad_shard, d.param_shard};
    const int el[5] = {4, 4, 4, esz, esz};
    for (int i = 0; i < 5; ++i) {
        char why[160];
        if (arr[i] && !device_range_ok(arr[i], (size_t)S * el[i], dev, why, sizeof(why)))
            return fail(ZERO_ERR_INVALID_ARG, "%s: shard array %d (%lld elements) %s", who, i,
                        (long long)S, why);
    }
    return ZERO_OK;
}

// LDS per CU and the largest dynamic LDS of one workgroup on device `dev`.
static void query_lds(int dev, int* lds_cu, int* lds_blk)
{
    if (hipDeviceGetAttribute(lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess || *lds_cu <= 0)
        *lds_cu = 160 * 1024;
    if (hipDeviceGetAttribute(lds_blk, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess || *lds_blk <= 0)
        *lds_blk = 64 * 1024;
    (void)hipGetLastError();
}

// The dynamic LDS each kernel reserves to cap its workgroups per CU.
static void set_lds_reserves(zero_shard_s* h, int lds_cu, int lds_blk)
{
    h->lds_adam = lds_reserve_for(lds_cu, lds_blk, zk::kAdamPerCU);
    h->lds_sgd_mom = lds_reserve_for(lds_cu, lds_blk, zk::kSgdMomPerCU);
    h->lds_sgd_plain = lds_reserve_for(lds_cu, lds_blk, zk::kSgdPlainPerCU);
    h->lds_reduce = lds_reserve_for(lds_cu, lds_blk, zk::kRedPerCU);
    h->lds_reduce_many = lds_reserve_for(
        lds_cu, lds_blk, h->d.lp == ZERO_FP32 ? zk::kRedPerCUMany : zk::kRedPerCUMany2B);
    h->lds_reduce_wide = lds_reserve_for(lds_cu, lds_blk, zk::kRedPerCUWide);
    h->lds_shift = lds_reserve_for(lds_cu, lds_blk, zk::kRedShiftPerCU);
    h->lds_shift_many = lds_reserve_for(
        lds_cu, lds_blk, h->d.lp == ZERO_FP32 ? zk::kRedShiftPerCUMany : zk::kRedShiftPerCUMany2B);
    h->lds_scan = lds_reserve_for(lds_cu, lds_blk, zk::kScanPerCU);
}

// Validation and creation shared by the Adam and the SGD handles (need_m /
// need_v as for check_desc).  On success the handle holds desc, S, opt and the
// loss scale; the caller stores its hyper-parameters and t.
static zero_status init_common(const zero_shard_desc* desc, Opt opt, int need_m, int need_v,
                               const zero_loss_scale_cfg* ls, const char* who,
                               zero_shard_s** out)
{
    const zero_shard_desc& d = *desc;
    int64_t S = 0;
    zero_status st = check_desc(d, need_m, need_v, who, &S);
    if (st != ZERO_OK) return st;
    st = check_ls(ls);
    if (st != ZERO_OK) return st;

    // One fp64 partial per reduce workgroup of a step.  A bucket of len
    // elements uses at most len/per + 2 workgroups, per being the smaller of
    // the element-wise and the vector kernels' elements per workgroup (plus a
    // ragged end), and the stand-alone scan needs no more.
    const int64_t vper = zk::kRunsPerBlockMin * zk::run_width(d.lp);
    const int64_t per = zk::kScalarElemsPerBlock < vper ? zk::kScalarElemsPerBlock : vper;
    const int64_t nbuckets = (S + d.bucket_elems - 1) / d.bucket_elems;
    const int64_t nslots = S / per + 2 * nbuckets + 4;
    if (nslots > (int64_t(1) << 25))
        return fail(ZERO_ERR_UNSUPPORTED,
                    "%s: %lld buckets of %lld elements need %lld partial slots (limit 2^25); "
                    "use a larger bucket_elems", who, (long long)nbuckets, (long long)d.bucket_elems,
                    (long long)nslots);

    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "init: hipGetDevice");
    st = check_desc_ranges(d, S, dev, who);
    if (st != ZERO_OK) return st;

    zero_shard_s* h = new (std::nothrow) zero_shard_s();
    if (!h) return fail(ZERO_ERR_OOM, "init: host allocation failed");
    h->device = dev;
    h->d = d;
    h->S = S;
    h->opt = opt;
    h->esz = lp_bytes(d.lp);
    h->ls = *ls;
    h->scale = ls->init_scale;
    h->good_steps = 0;
    h->nslots = nslots;

    const size_t ws_bytes = sizeof(double) * (size_t)(nslots + zk::kFoldMaxBlocks) +
                            sizeof(zk::CheckResult) + 2 * sizeof(zk::DevState);
    e = hipMalloc(&h->ws, ws_bytes);
    if (e != hipSuccess) {
        delete h;
        (void)hipGetLastError();
        return fail(e == hipErrorOutOfMemory ? ZERO_ERR_OOM : ZERO_ERR_HIP,
                    "init: hipMalloc of %zu bytes: %s", ws_bytes, hipGetErrorString(e));
    }
    h->partial = static_cast<double*>(h->ws);
    h->level1 = h->partial + nslots;
    h->result = reinterpret_cast<zk::CheckResult*>(h->level1 + zk::kFoldMaxBlocks);
    h->dev = reinterpret_cast<zk::DevState*>(h->result + 1);
    h->dev_snapshot = h->dev + 1;

    int lds_cu = 0, lds_blk = 0;
    query_lds(dev, &lds_cu, &lds_blk);
    set_lds_reserves(h, lds_cu, lds_blk);
    static_assert(sizeof(zk::CheckResult) <= 64 && sizeof(zk::DevState) <= 192, "pinned layout");
    e = hipHostMalloc(reinterpret_cast<void**>(&h->host_result), 256, hipHostMallocDefault);
    if (e != hipSuccess) {
        (void)hipFree(h->ws);
        delete h;
        (void)hipGetLastError();
        return fail(ZERO_ERR_OOM, "init: hipHostMalloc: %s", hipGetErrorString(e));
    }
    std::memset(h->host_result, 0, 256);
    h->host_dev = reinterpret_cast<zk::DevState*>(reinterpret_cast<char*>(h->host_result) + 64);
    e = hipEventCreateWithFlags(&h->result_ready, hipEventDisableTiming);
    if (e != hipSuccess) {
        (void)hipFree(h->ws);
        (void)hipHostFree(h->host_result);
        delete h;
        (void)hipGetLastError();
        return fail(ZERO_ERR_HIP, "init: hipEventCreate: %s", hipGetErrorString(e));
    }
    *out = h;
    return ZERO_OK;
}

// Validate R contribution pointers of a handle's storage format.
static zero_status check_contribs(const zero_shard_s* h, const void* const* contribs,
                                  int32_t n_contrib, const char* who)
{
    if (!contribs) return fail(ZERO_ERR_INVALID_ARG, "%s: NULL contribs", who);
    if (n_contrib < 1 || n_contrib > ZERO_MAX_CONTRIB)
        return fail(ZERO_ERR_INVALID_ARG, "%s: n_contrib %d outside [1, %d]", who, n_contrib,
                    ZERO_MAX_CONTRIB);
    for (int r = 0; r < n_contrib; ++r) {
        if (!contribs[r]) return fail(ZERO_ERR_INVALID_ARG, "%s: contribution %d is NULL", who, r);
        if ((uintptr_t)contribs[r] % (uintptr_t)h->esz != 0)
            return fail(ZERO_ERR_INVALID_ARG, "%s: contribution %d not %d-byte aligned", who, r,
                        h->esz);
    }
    return ZERO_OK;
}

// Contributions covering len elements for the shard elements [off, off + len)
// must be device-accessible memory of the handle's device (as far as the
// runtime can tell); they may be that very slice of grad_shard (an in-place
// reduce: each lane loads its elements before it stores them) but must not
// otherwise overlap grad_shard, and must not overlap master, exp_avg,
// exp_avg_sq or param_shard.
static zero_status check_contrib_overlap(const zero_shard_s* h, const void* const* contribs,
                                         int32_t n_contrib, int64_t off, int64_t len,
                                         const char* who)
{
    const size_t nb = (size_t)len * (size_t)h->esz;
    const uintptr_t own = (uintptr_t)h->d.grad_shard + (uintptr_t)off * (uintptr_t)h->esz;
    const void* state[4] = {h->d.master, h->d.exp_avg, h->d.exp_avg_sq, h->d.param_shard};
    const size_t state_bytes[4] = {(size_t)h->S * 4, (size_t)h->S * 4, (size_t)h->S * 4,
                                   (size_t)h->S * (size_t)h->esz};
    for (int r = 0; r < n_contrib; ++r) {
        const uintptr_t a = (uintptr_t)contribs[r];
        char why[160];
        if (!device_range_ok(contribs[r], nb, h->device, why, sizeof(why)))
            return fail(ZERO_ERR_INVALID_ARG, "%s: contribution %d (%lld elements) %s", who, r,
                        (long long)len, why);
        for (int k = 0; k < 4; ++k)
            if (state[k] && overlaps(a, nb, (uintptr_t)state[k], state_bytes[k]))
                return fail(ZERO_ERR_INVALID_ARG, "%s: contribution %d overlaps shard array %d",
                            who, r, k == 3 ? 4 : k);
        if (a != own &&
            overlaps(a, nb, (uintptr_t)h->d.grad_shard, (size_t)h->S * (size_t)h->esz))
            return fail(ZERO_ERR_INVALID_ARG,
                        "%s: contribution %d overlaps grad_shard other than as its own slice", who,
                        r);
    }
    return ZERO_OK;
}

// Launch the reduce of the bucket [off, off + len) of the shard from the
// contributions' bucket pointers, writing partial slots from slot_base on;
// dev set: the unscale factor comes from the device state; snapshot set: the
// launch also copies the device state there (inline-fold steps).  With
// launch = false only *blocks_out (the partial slots it would write) is set.
static zero_status enqueue_reduce(zero_shard_s* h, const void* const* ptrs, int32_t n_contrib,
                                  int64_t off, int64_t len, int64_t slot_base,
                                  const zk::DevState* dev, hipStream_t s, int64_t* blocks_out,
                                  const char* who, zk::DevState* snapshot = nullptr,
                                  bool launch = true)
{
    zk::ReduceLaunch L;
    std::memset(&L, 0, sizeof(L));
    uintptr_t addr[ZERO_MAX_CONTRIB + 1];
    for (int r = 0; r < n_contrib; ++r) {
        L.c.p[r] = ptrs[r];
        addr[r] = (uintptr_t)ptrs[r];
    }
    char* out = static_cast<char*>(h->d.grad_shard) + off * h->esz;
    addr[n_contrib] = (uintptr_t)out;
    L.out = out;
    L.n = len;
    const int W = zk::run_width(h->d.lp);
    // whole 16-byte runs when every array shares its address phase modulo 16;
    // else the shift kernel (each contribution read at its own phase), else
    // element by element
    const zl::ReduceLayout lay = zl::reduce_layout(addr, n_contrib, h->esz, len);
    L.shift = lay.shift;
    L.vec_ok = lay.vec_ok;
    L.head = lay.head;
    L.nvec = lay.nvec;
    L.R = n_contrib;
    L.lp = (int32_t)h->d.lp;
    L.inv_r = (float)(1.0 / (double)n_contrib);
    L.inv_scale = (float)(1.0 / h->scale);
    L.partial = h->partial;
    L.slot_base = slot_base;
    if (L.shift)
        L.lds_reserve = n_contrib >= zk::kRedManyR ? h->lds_shift_many : h->lds_shift;
    else
        L.lds_reserve = n_contrib >= zk::kRedWideR   ? h->lds_reduce_wide
                        : n_contrib >= zk::kRedManyR ? h->lds_reduce_many
                                                     : h->lds_reduce;
    L.dev = dev;
    L.snapshot = snapshot;
    L.small = zk::shard_small(h->S) ? 1 : 0;
    const int64_t blocks = zk::reduce_blocks(L.n, L.head, L.nvec, L.vec_ok, W,
                                             zk::red_runs(L.R, L.nvec, L.small != 0, L.shift != 0),
                                             zk::red_block(L.R, L.small != 0), true);
    if (L.slot_base + blocks > h->nslots)
        return fail(ZERO_ERR_UNSUPPORTED, "%s: partial slots exhausted", who);
    if (!launch) {
        *blocks_out = blocks;
        return ZERO_OK;
    }
    hipError_t e = zk::launch_reduce(L, s);
    if (e != hipSuccess) return hip_fail(e, who);
    *blocks_out = blocks;
    return ZERO_OK;
}

static void publish(zero_shard_s* h)
{
    std::lock_guard<std::mutex> lk(g_live_mu);
    g_live.insert(h);
}

extern "C" {

zero_status zero_shard_init(const zero_shard_desc* desc, const zero_adam_hparams* hp,
                            const zero_loss_scale_cfg* ls, zero_shard_t* out)
{
    if (!desc || !out) return fail(ZERO_ERR_INVALID_ARG, "init: NULL desc or out");
    zero_status st = check_hparams(hp);
    if (st != ZERO_OK) return st;
    zero_shard_s* h = nullptr;
    st = init_common(desc, kOptAdam, 1, 1, ls, "init", &h);
    if (st != ZERO_OK) return st;
    h->hp = *hp;
    h->t = hp->initial_step;
    publish(h);
    *out = h;
    return ZERO_OK;
}

zero_status zero_shard_init_sgd(const zero_shard_desc* desc, const zero_sgd_hparams* hp,
                                const zero_loss_scale_cfg* ls, zero_shard_t* out)
{
    if (!desc || !out) return fail(ZERO_ERR_INVALID_ARG, "init_sgd: NULL desc or out");
    zero_status st = check_sgd_hparams(hp, desc->exp_avg != nullptr);
    if (st != ZERO_OK) return st;
    zero_shard_s* h = nullptr;
    st = init_common(desc, kOptSgd, 0, -1, ls, "init_sgd", &h);
    if (st != ZERO_OK) return st;
    h->sgd = *hp;
    h->t = hp->initial_step;
    publish(h);
    *out = h;
    return ZERO_OK;
}

zero_status zero_shard_destroy(zero_shard_t h)
{
    {
        std::lock_guard<std::mutex> lk(g_live_mu);
        if (h == nullptr || g_live.erase(h) == 0)
            return fail(ZERO_ERR_STATE, "destroy: not a live handle");
    }
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != h->device) (void)hipSetDevice(h->device);
    (void)hipDeviceSynchronize();
    (void)hipFree(h->ws);
    (void)hipHostFree(h->host_result);
    if (h->result_ready) (void)hipEventDestroy(h->result_ready);
    if (cur != h->device && cur >= 0) (void)hipSetDevice(cur);
    delete h;
    return ZERO_OK;
}

zero_status zero_bucket_reduce(zero_shard_t h, const void* const* contribs, int32_t n_contrib,
                               int64_t bucket_off, int64_t bucket_len, void* stream)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "bucket_reduce: not a live handle");
    if (zero_status ds = check_device(h, stream, "bucket_reduce")) return ds;
    if (h->device_mode)
        return fail(ZERO_ERR_STATE, "bucket_reduce: device-resident flow active; call zero_device_end");
    zero_status cst = check_contribs(h, contribs, n_contrib, "bucket_reduce");
    if (cst != ZERO_OK) return cst;
    if (bucket_len < 1) return fail(ZERO_ERR_INVALID_ARG, "bucket_reduce: bucket_len must be >= 1");
    if (bucket_off < 0 || bucket_off >= h->S || bucket_len > h->S - bucket_off)
        return fail(ZERO_ERR_INVALID_ARG, "bucket_reduce: bucket [%lld, +%lld) outside [0, %lld)",
                    (long long)bucket_off, (long long)bucket_len, (long long)h->S);
    if (bucket_len > h->d.bucket_elems)
        return fail(ZERO_ERR_INVALID_ARG, "bucket_reduce: bucket_len %lld exceeds C_B %lld",
                    (long long)bucket_len, (long long)h->d.bucket_elems);
    cst = check_contrib_overlap(h, contribs, n_contrib, bucket_off, bucket_len, "bucket_reduce");
    if (cst != ZERO_OK) return cst;
    if (h->phase == kChecked)
        return fail(ZERO_ERR_STATE, "bucket_reduce: step already checked; call zero_adam_step");
    if (h->phase == kPending)
        return fail(ZERO_ERR_STATE, "bucket_reduce: a gated step is pending; call zero_step_resolve");
    const int64_t expect = h->phase == kIdle ? 0 : h->covered;
    if (bucket_off != expect)
        return fail(ZERO_ERR_STATE, "bucket_reduce: expected bucket at %lld, got %lld",
                    (long long)expect, (long long)bucket_off);
    if (bucket_off + bucket_len < h->S && bucket_len != h->d.bucket_elems)
        return fail(ZERO_ERR_STATE, "bucket_reduce: only the last bucket may be shorter than C_B");

    int64_t blocks = 0;
    const int64_t slot_base = h->phase == kIdle ? 0 : h->slot_cursor;
    zero_status st = enqueue_reduce(h, contribs, n_contrib, bucket_off, bucket_len, slot_base, nullptr,
                                    static_cast<hipStream_t>(stream), &blocks, "bucket_reduce");
    if (st != ZERO_OK) return st;
    h->covered = bucket_off + bucket_len;
    h->slot_cursor = slot_base + blocks;
    h->phase = kReducing;
    return ZERO_OK;
}

}  // extern "C"

// Launch the stand-alone scan of the stored grad_shard (no bucket reduced this
// step) into partial slots from 0; returns the slots written.  snapshot and
// launch as for enqueue_reduce.
static zero_status enqueue_scan(zero_shard_s* h, const zk::DevState* dev, hipStream_t s,
                                int64_t* slots, const char* who,
                                zk::DevState* snapshot = nullptr, bool launch = true)
{
    zk::ScanLaunch L;
    std::memset(&L, 0, sizeof(L));
    const uintptr_t a = (uintptr_t)h->d.grad_shard;
    const int el = h->esz, al = 16;
    const int W = zk::run_width(h->d.lp);
    L.g = h->d.grad_shard;
    L.n = h->S;
    zl::split(h->S, zl::common_head(&a, &el, &al, 1), W, &L.head, &L.nvec, &L.vec_ok);
    L.lp = (int32_t)h->d.lp;
    L.inv_scale = (float)(1.0 / h->scale);
    L.partial = h->partial;
    L.slot_base = 0;
    L.lds_reserve = h->lds_scan;
    L.dev = dev;
    L.snapshot = snapshot;
    *slots = zk::reduce_blocks(L.n, L.head, L.nvec, L.vec_ok, W, zk::kScanRuns, zk::kScanBlock);
    if (!launch) return ZERO_OK;
    hipError_t e = zk::launch_scan(L, s);
    if (e != hipSuccess) return hip_fail(e, who);
    return ZERO_OK;
}

// Launch the check of the step on `s`: the stand-alone scan when no bucket was
// reduced, the fixed-order fold of the partials (with the clipping
// coefficient), and the copy of the result to pinned host memory.  Call only
// in phase kIdle or kReducing with full coverage.
static zero_status launch_check(zero_shard_s* h, hipStream_t s, const char* who)
{
    if (h->phase == kIdle) {
        zero_status st = enqueue_scan(h, nullptr, s, &h->slot_cursor, who);
        if (st != ZERO_OK) return st;
    }
    const zk::PrepareArgs none{};
    hipError_t e = zk::launch_finalize(h->partial, h->slot_cursor, h->level1, h->result, h->max_norm,
                                       nullptr, none, s);
    if (e != hipSuccess) return hip_fail(e, who);
    e = hipMemcpyAsync(h->host_result, h->result, sizeof(zk::CheckResult), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, who);
    return ZERO_OK;
}

// The step's result from the pinned copy: overflow when the total is not
// finite (a non-finite unscaled gradient makes its workgroup partial NaN; the
// fp64 squares of finite fp32 values cannot sum to inf).
static zero_step_info read_check(zero_shard_s* h)
{
    zero_step_info info;
    std::memset(&info, 0, sizeof(info));
    const double total = h->host_result->sumsq;
    info.overflow = std::isfinite(total) ? 0 : 1;
    info.skipped = info.overflow;
    info.step_t = h->t;
    info.grad_norm = std::sqrt(total);
    info.scale_used = h->scale;
    int64_t g;
    next_scale(h, info.overflow, &info.scale_next, &g);
    return info;
}

// Where the update of each flow takes its per-step values.  Synchronous check:
// the clipping coefficient from the device result (the host-computed one after
// a merge); gated: also skip on the result's NaN; device-resident: everything
// from the device state.
static zk::StepSource source_sync(const zero_shard_s* h)
{
    zk::StepSource src{};
    src.res = h->merged ? nullptr : h->result;
    src.clip = h->merged ? h->merge_clip : 1.0f;
    return src;
}

static zk::StepSource source_gated(const zero_shard_s* h)
{
    zk::StepSource src{};
    src.res = h->result;
    src.gate = 1;
    src.clip = 1.0f;
    return src;
}

static zk::StepSource source_device(const zero_shard_s* h)
{
    zk::StepSource src{};
    src.res = h->result;
    src.dev = h->dev;
    src.clip = 1.0f;
    return src;
}

// Layout of the update over the shard: groups of 4 elements, 16-byte aligned
// in the fp32 arrays and 4*esz in the stored ones, after a common scalar head
// (see split); the arrays present are those of the handle's optimizer.
static void update_layout(const zero_shard_s* h, int64_t* head, int64_t* ngroups, int32_t* vec_ok)
{
    uintptr_t addr[5];
    int elt[5], align[5], cnt = 0;
    const void* arr[5] = {h->d.master, h->d.exp_avg, h->opt == kOptAdam ? h->d.exp_avg_sq : nullptr,
                          h->d.grad_shard, h->d.param_shard};
    const int el[5] = {4, 4, 4, h->esz, h->esz};
    for (int k = 0; k < 5; ++k) {
        if (!arr[k]) continue;
        addr[cnt] = (uintptr_t)arr[k];
        elt[cnt] = el[k];
        align[cnt] = 4 * el[k];
        ++cnt;
    }
    zl::split(h->S, zl::common_head(addr, elt, align, cnt), 4, head, ngroups, vec_ok);
}

// Whether a device-resident step with `slots` partials folds them inside the
// update: few enough partials, and an update that is one vector launch over
// the whole shard (no element-wise head or tail).
static bool inline_fold_ok(const zero_shard_s* h, int64_t slots)
{
    if (slots < 1 || slots > zk::kInlineFoldMax) return false;
    int64_t head, ngroups;
    int32_t vec_ok;
    update_layout(h, &head, &ngroups, &vec_ok);
    if (!vec_ok || head != 0 || 4 * ngroups != h->S) return false;
    if (h->opt == kOptAdam)
        return zk::one_launch(ngroups, zk::adam_lanes(h->S), zk::adam_groups(h->S));
    return zk::one_launch(ngroups, zk::sgd_lanes(h->S), zk::sgd_groups(h->S, h->d.exp_avg != nullptr));
}

// Launch Adam for applied step t = h->t + 1 with hyper-parameters hp; src says
// where the kernels take the per-step values (see source_*).
// Returns the fp64 powers beta^t it used and whether they extend the cache.
static zero_status launch_adam_step(zero_shard_s* h, const zero_adam_hparams& hp, hipStream_t s,
                                    const zk::StepSource& src, double* pw1_out,
                                    double* pw2_out, bool* same_betas_out, const char* who)
{
    const int64_t t = h->t + 1;
    double pw1 = 1.0, pw2 = 1.0;
    const bool same_betas = hp.beta1 == h->hp.beta1 && hp.beta2 == h->hp.beta2;
    if (src.dev != nullptr) {
        // the device-resident flow takes t and the bias corrections from the
        // device state; the host copies are stale and unused
    } else if (same_betas && h->pw_t == t - 1) {
        pw1 = h->pw1 * (double)(float)hp.beta1;
        pw2 = h->pw2 * (double)(float)hp.beta2;
    } else {
        pw1 = beta_pow(hp.beta1, t);
        pw2 = beta_pow(hp.beta2, t);
    }
    zk::AdamLaunch a;
    std::memset(&a, 0, sizeof(a));
    a.grad = h->d.grad_shard;
    a.master = h->d.master;
    a.m = h->d.exp_avg;
    a.v = h->d.exp_avg_sq;
    a.param = h->d.param_shard;
    a.n = h->S;
    update_layout(h, &a.head, &a.ngroups, &a.vec_ok);
    a.lds_reserve = h->lds_adam;
    a.lp = (int32_t)h->d.lp;
    a.b1 = (float)hp.beta1;
    a.b2 = (float)hp.beta2;
    a.omb1 = 1.0f - a.b1;
    a.omb2 = 1.0f - a.b2;
    a.bc1 = hp.bias_correction ? (float)(1.0 - pw1) : 1.0f;
    a.bc2 = hp.bias_correction ? (float)(1.0 - pw2) : 1.0f;
    a.lr = (float)hp.lr;
    a.eps = (float)hp.eps;
    a.wd = (float)hp.weight_decay;
    a.inv_scale = (float)(1.0 / h->scale);
    a.wd_kind = a.wd == 0.0f ? zk::kWdNone
              : (hp.wd_mode == ZERO_WD_L2 ? zk::kWdL2 : zk::kWdDecoupled);
    a.src = src;
    hipError_t e = zk::launch_adam(a, s);
    if (e != hipSuccess) return hip_fail(e, who);
    *pw1_out = pw1;
    *pw2_out = pw2;
    *same_betas_out = same_betas;
    return ZERO_OK;
}

// Launch SGD for applied step t + 1 with hyper-parameters hp; src as in
// launch_adam_step.
static zero_status launch_sgd_step(zero_shard_s* h, const zero_sgd_hparams& hp, hipStream_t s,
                                   const zk::StepSource& src, const char* who)
{
    zk::SgdLaunch a;
    std::memset(&a, 0, sizeof(a));
    a.grad = h->d.grad_shard;
    a.master = h->d.master;
    a.mom = h->d.exp_avg;
    a.param = h->d.param_shard;
    a.n = h->S;
    update_layout(h, &a.head, &a.ngroups, &a.vec_ok);
    a.lds_reserve = a.mom ? h->lds_sgd_mom : h->lds_sgd_plain;
    a.lp = (int32_t)h->d.lp;
    a.lr = (float)hp.lr;
    a.mu = (float)hp.momentum;
    a.wd = (float)hp.weight_decay;
    a.has_wd = a.wd != 0.0f;
    a.inv_scale = (float)(1.0 / h->scale);
    a.src = src;
    hipError_t e = zk::launch_sgd(a, s);
    if (e != hipSuccess) return hip_fail(e, who);
    return ZERO_OK;
}

// Commit the outcome of a step: on success t advances (and the beta^t cache);
// the loss scale follows the overflow flag; the handle returns to idle.
static void commit_step(zero_shard_s* h, zero_step_info* info, double pw1, double pw2,
                        bool same_betas)
{
    double scale_next;
    int64_t good_next;
    next_scale(h, info->overflow, &scale_next, &good_next);
    if (!info->overflow) {
        h->t += 1;
        if (same_betas) {
            h->pw1 = pw1;
            h->pw2 = pw2;
            h->pw_t = h->t;
        }
    }
    info->step_t = h->t;
    info->scale_next = scale_next;
    h->scale = scale_next;
    h->good_steps = good_next;
    h->phase = kIdle;
    h->covered = 0;
    h->slot_cursor = 0;
    h->merged = false;
}

// Checks shared by the gated step calls of both optimizers.
static zero_status gated_preconditions(zero_shard_s* h, Opt opt, const char* who)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "%s: not a live handle", who);
    if (h->device_mode)
        return fail(ZERO_ERR_STATE, "%s: device-resident flow active; call zero_device_end", who);
    if (h->opt != opt)
        return fail(ZERO_ERR_STATE, "%s: handle was created for %s", who,
                    h->opt == kOptAdam ? "Adam" : "SGD");
    if (h->phase == kChecked || h->phase == kPending)
        return fail(ZERO_ERR_STATE, "%s: step already checked or pending", who);
    if (h->phase == kReducing && h->covered != h->S)
        return fail(ZERO_ERR_STATE, "%s: buckets cover [0, %lld) of [0, %lld)", who,
                    (long long)h->covered, (long long)h->S);
    return ZERO_OK;
}

// Enqueue a gated step: the check, its result copy and the event the resolve
// waits on, then the update (launch_update), which skips itself on overflow.
// On an error the handle returns to the phase it was in.
template <typename F>
static zero_status enqueue_gated(zero_shard_s* h, hipStream_t s, const char* who, F launch_update)
{
    const Phase before = h->phase;
    const int64_t cursor_before = h->slot_cursor;
    zero_status st = launch_check(h, s, who);
    if (st == ZERO_OK) {
        hipError_t e = hipEventRecord(h->result_ready, s);
        if (e != hipSuccess) st = hip_fail(e, who);
    }
    if (st == ZERO_OK) st = launch_update(s);
    if (st != ZERO_OK) {
        h->phase = before;
        h->slot_cursor = cursor_before;
        return st;
    }
    h->phase = kPending;
    return ZERO_OK;
}

extern "C" {

zero_status zero_overflow_check(zero_shard_t h, void* stream, zero_step_info* out)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "overflow_check: not a live handle");
    if (zero_status ds = check_device(h, stream, "overflow_check")) return ds;
    if (h->device_mode)
        return fail(ZERO_ERR_STATE, "%s: device-resident flow active; call zero_device_end", "overflow_check");
    if (!out) return fail(ZERO_ERR_INVALID_ARG, "overflow_check: NULL out");
    if (h->phase == kPending)
        return fail(ZERO_ERR_STATE, "overflow_check: a gated step is pending; call zero_step_resolve");
    if (h->phase == kChecked) {
        *out = h->check;
        return ZERO_OK;
    }
    if (h->phase == kReducing && h->covered != h->S)
        return fail(ZERO_ERR_STATE, "overflow_check: buckets cover [0, %lld) of [0, %lld)",
                    (long long)h->covered, (long long)h->S);
    hipStream_t s = static_cast<hipStream_t>(stream);
    zero_status st = launch_check(h, s, "overflow_check");
    if (st != ZERO_OK) return st;
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "overflow_check: synchronize");
    h->check = read_check(h);
    h->phase = kChecked;
    *out = h->check;
    return ZERO_OK;
}

zero_status zero_adam_step(zero_shard_t h, const zero_adam_hparams* hp_in, void* stream,
                           zero_step_info* out)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "adam_step: not a live handle");
    if (zero_status ds = check_device(h, stream, "adam_step")) return ds;
    if (h->opt != kOptAdam) return fail(ZERO_ERR_STATE, "adam_step: handle was created for SGD");
    if (h->phase != kChecked)
        return fail(ZERO_ERR_STATE, "adam_step: zero_overflow_check has not completed this step");
    if (hp_in) {
        zero_status st = check_hparams(hp_in);
        if (st != ZERO_OK) return st;
    }
    const zero_adam_hparams& hp = hp_in ? *hp_in : h->hp;
    zero_step_info info = h->check;
    double pw1 = 1.0, pw2 = 1.0;
    bool same = false;
    if (!info.overflow) {
        zero_status st = launch_adam_step(h, hp, static_cast<hipStream_t>(stream), source_sync(h),
                                          &pw1, &pw2, &same, "adam_step: launch");
        if (st != ZERO_OK) return st;
    }
    commit_step(h, &info, pw1, pw2, same);
    if (out) *out = info;
    return ZERO_OK;
}

zero_status zero_overflow_merge(zero_shard_t h, int32_t global_overflow, double global_grad_norm,
                                zero_step_info* out)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "overflow_merge: not a live handle");
    if (h->phase != kChecked)
        return fail(ZERO_ERR_STATE, "overflow_merge: zero_overflow_check has not completed this step");
    if (global_overflow != 0 && global_overflow != 1)
        return fail(ZERO_ERR_INVALID_ARG, "overflow_merge: global_overflow must be 0 or 1");
    if (global_overflow < h->check.overflow)
        return fail(ZERO_ERR_INVALID_ARG,
                    "overflow_merge: this rank overflowed; the global flag cannot be 0");
    // an applied step takes its clipping coefficient from the global norm,
    // which sums this rank's squares with the others': finite, >= 0 and not
    // below this rank's own norm (to a relative 1e-9, the rounding of the sum)
    if (!global_overflow &&
        !(std::isfinite(global_grad_norm) && global_grad_norm >= 0.0 &&
          global_grad_norm >= h->check.grad_norm * (1.0 - 1e-9)))
        return fail(ZERO_ERR_INVALID_ARG,
                    "overflow_merge: global_grad_norm %g must be finite and not below this "
                    "rank's norm %g", global_grad_norm, h->check.grad_norm);
    h->check.overflow = global_overflow;
    h->check.skipped = global_overflow;
    h->check.grad_norm = global_grad_norm;
    // the clipping coefficient of the global norm, by the rule the fold applies
    h->merged = true;
    h->merge_clip = 1.0f;
    if (h->max_norm > 0.0 && !global_overflow) {
        const double c = h->max_norm / (global_grad_norm + 1e-6);
        if (c < 1.0) h->merge_clip = (float)c;
    }
    int64_t g;
    next_scale(h, global_overflow, &h->check.scale_next, &g);
    if (out) *out = h->check;
    return ZERO_OK;
}

zero_status zero_adam_step_gated(zero_shard_t h, const zero_adam_hparams* hp_in, void* stream)
{
    const char* who = "adam_step_gated";
    zero_status st = gated_preconditions(h, kOptAdam, who);
    if (st == ZERO_OK) st = check_device(h, stream, who);
    if (st != ZERO_OK) return st;
    if (hp_in && (st = check_hparams(hp_in)) != ZERO_OK) return st;
    const zero_adam_hparams& hp = hp_in ? *hp_in : h->hp;
    return enqueue_gated(h, static_cast<hipStream_t>(stream), who, [&](hipStream_t s) {
        return launch_adam_step(h, hp, s, source_gated(h), &h->pend_pw1, &h->pend_pw2,
                                &h->pend_same_betas, "adam_step_gated: launch");
    });
}

zero_status zero_sgd_step(zero_shard_t h, const zero_sgd_hparams* hp_in, void* stream,
                          zero_step_info* out)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "sgd_step: not a live handle");
    if (zero_status ds = check_device(h, stream, "sgd_step")) return ds;
    if (h->opt != kOptSgd) return fail(ZERO_ERR_STATE, "sgd_step: handle was created for Adam");
    if (h->phase != kChecked)
        return fail(ZERO_ERR_STATE, "sgd_step: zero_overflow_check has not completed this step");
    if (hp_in) {
        zero_status st = check_sgd_hparams(hp_in, h->d.exp_avg != nullptr);
        if (st != ZERO_OK) return st;
    }
    const zero_sgd_hparams& hp = hp_in ? *hp_in : h->sgd;
    zero_step_info info = h->check;
    if (!info.overflow) {
        zero_status st = launch_sgd_step(h, hp, static_cast<hipStream_t>(stream), source_sync(h),
                                         "sgd_step: launch");
        if (st != ZERO_OK) return st;
    }
    commit_step(h, &info, 1.0, 1.0, false);
    if (out) *out = info;
    return ZERO_OK;
}

zero_status zero_sgd_step_gated(zero_shard_t h, const zero_sgd_hparams* hp_in, void* stream)
{
    const char* who = "sgd_step_gated";
    zero_status st = gated_preconditions(h, kOptSgd, who);
    if (st == ZERO_OK) st = check_device(h, stream, who);
    if (st != ZERO_OK) return st;
    if (hp_in && (st = check_sgd_hparams(hp_in, h->d.exp_avg != nullptr)) != ZERO_OK) return st;
    const zero_sgd_hparams& hp = hp_in ? *hp_in : h->sgd;
    return enqueue_gated(h, static_cast<hipStream_t>(stream), who, [&](hipStream_t s) {
        h->pend_pw1 = h->pend_pw2 = 1.0;
        h->pend_same_betas = false;
        return launch_sgd_step(h, hp, s, source_gated(h), "sgd_step_gated: launch");
    });
}

zero_status zero_step_resolve(zero_shard_t h, zero_step_info* out)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "step_resolve: not a live handle");
    if (h->phase != kPending) return fail(ZERO_ERR_STATE, "step_resolve: no gated step pending");
    hipError_t e = hipEventSynchronize(h->result_ready);
    if (e != hipSuccess) return hip_fail(e, "step_resolve: event");
    zero_step_info info = read_check(h);
    commit_step(h, &info, h->pend_pw1, h->pend_pw2, h->pend_same_betas);
    if (out) *out = info;
    return ZERO_OK;
}

zero_status zero_shard_get_counters(zero_shard_t h, int64_t* step_t, double* scale,
                                    int64_t* good_steps)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "get_counters: not a live handle");
    if (h->device_mode)
        return fail(ZERO_ERR_STATE, "%s: device-resident flow active; call zero_device_end", "get_counters");
    if (!step_t || !scale || !good_steps) return fail(ZERO_ERR_INVALID_ARG, "get_counters: NULL");
    *step_t = h->t;
    *scale = h->scale;
    *good_steps = h->good_steps;
    return ZERO_OK;
}

zero_status zero_shard_set_counters(zero_shard_t h, int64_t step_t, double scale,
                                    int64_t good_steps)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "set_counters: not a live handle");
    if (h->device_mode)
        return fail(ZERO_ERR_STATE, "%s: device-resident flow active; call zero_device_end", "set_counters");
    if (step_t < 0 || !scale_ok(scale) || good_steps < 0)
        return fail(ZERO_ERR_INVALID_ARG, "set_counters: values out of range");
    if (h->phase != kIdle) return fail(ZERO_ERR_STATE, "set_counters: a step is in progress");
    h->t = step_t;
    h->scale = scale;
    h->good_steps = good_steps;
    h->pw_t = -1;
    return ZERO_OK;
}

zero_status zero_shard_set_clip(zero_shard_t h, double max_grad_norm)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "set_clip: not a live handle");
    if (h->device_mode)
        return fail(ZERO_ERR_STATE, "set_clip: device-resident flow active; call zero_device_end");
    if (h->phase != kIdle) return fail(ZERO_ERR_STATE, "set_clip: a step is in progress");
    if (!(std::isfinite(max_grad_norm) && max_grad_norm >= 0.0))
        return fail(ZERO_ERR_INVALID_ARG, "set_clip: max_grad_norm must be finite and >= 0");
    h->max_norm = max_grad_norm;
    return ZERO_OK;
}

zero_status zero_device_begin(zero_shard_t h, void* stream)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "device_begin: not a live handle");
    if (zero_status ds = check_device(h, stream, "device_begin")) return ds;
    if (h->device_mode) return fail(ZERO_ERR_STATE, "device_begin: already active");
    if (h->phase != kIdle) return fail(ZERO_ERR_STATE, "device_begin: a step is in progress");
    zk::DevState init;
    std::memset(&init, 0, sizeof(init));
    init.scale = h->scale;
    init.pw1 = h->opt == kOptAdam ? beta_pow(h->hp.beta1, h->t) : 1.0;
    init.pw2 = h->opt == kOptAdam ? beta_pow(h->hp.beta2, h->t) : 1.0;
    init.t = h->t;
    init.good = h->good_steps;
    init.inv_scale = (float)(1.0 / h->scale);
    init.upd_inv_scale = init.inv_scale;
    init.bc1 = init.bc2 = 1.0f;
    hipError_t e = zk::launch_load_state(h->dev, init, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "device_begin: launch");
    h->dev_checked_n = 0;
    h->device_mode = true;
    return ZERO_OK;
}

zero_status zero_step_device(zero_shard_t h, const void* const* contribs, int32_t n_contrib,
                             void* stream)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "step_device: not a live handle");
    if (zero_status ds = check_device(h, stream, "step_device")) return ds;
    if (!h->device_mode) return fail(ZERO_ERR_STATE, "step_device: call zero_device_begin first");
    const bool scan = n_contrib == 0 && contribs == nullptr;
    if (!scan) {
        zero_status st = check_contribs(h, contribs, n_contrib, "step_device");
        if (st != ZERO_OK) return st;
        // a launch-bound step repeats the same pointers: validate a new set once
        bool same = n_contrib == h->dev_checked_n;
        for (int r = 0; same && r < n_contrib; ++r) same = contribs[r] == h->dev_checked[r];
        if (!same) {
            st = check_contrib_overlap(h, contribs, n_contrib, 0, h->S, "step_device");
            if (st != ZERO_OK) return st;
            for (int r = 0; r < n_contrib; ++r) h->dev_checked[r] = contribs[r];
            h->dev_checked_n = n_contrib;
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the reduce (or scan) launches: first counted, so that a step with few
    // partials can snapshot the state for an update that folds them itself
    auto enqueue_check = [&](bool launch, zk::DevState* snapshot, int64_t* slots) -> zero_status {
        *slots = 0;
        if (scan) return enqueue_scan(h, h->dev, s, slots, "step_device: scan", snapshot, launch);
        const void* ptrs[ZERO_MAX_CONTRIB];
        for (int64_t off = 0; off < h->S; off += h->d.bucket_elems) {
            const int64_t len = h->S - off < h->d.bucket_elems ? h->S - off : h->d.bucket_elems;
            for (int r = 0; r < n_contrib; ++r)
                ptrs[r] = static_cast<const char*>(contribs[r]) + off * h->esz;
            int64_t blocks = 0;
            zero_status st = enqueue_reduce(h, ptrs, n_contrib, off, len, *slots, h->dev, s,
                                            &blocks, "step_device: reduce", snapshot, launch);
            if (st != ZERO_OK) return st;
            *slots += blocks;
        }
        return ZERO_OK;
    };
    int64_t slots = 0;
    zero_status cst = enqueue_check(false, nullptr, &slots);
    if (cst != ZERO_OK) return cst;
    const bool fold_inline = inline_fold_ok(h, slots);
    cst = enqueue_check(true, fold_inline ? h->dev_snapshot : nullptr, &slots);
    if (cst != ZERO_OK) return cst;
    zk::PrepareArgs pa;
    std::memset(&pa, 0, sizeof(pa));
    if (h->opt == kOptAdam) {
        pa.b1 = (double)(float)h->hp.beta1;
        pa.b2 = (double)(float)h->hp.beta2;
        pa.bias_correction = h->hp.bias_correction;
    }
    pa.min_scale = h->ls.min_scale;
    pa.dynamic = h->ls.dynamic;
    pa.growth_interval = h->ls.growth_interval;
    zk::StepSource src = source_device(h);
    if (fold_inline) {
        // the update folds the partials and decides the step itself
        src.fold.partial = h->partial;
        src.fold.n = (int32_t)slots;
        src.fold.snapshot = h->dev_snapshot;
        src.fold.dev = h->dev;
        src.fold.res = h->result;
        src.fold.max_norm = h->max_norm;
        src.fold.pa = pa;
    } else {
        hipError_t e = zk::launch_finalize(h->partial, slots, h->level1, h->result, h->max_norm,
                                           h->dev, pa, s);
        if (e != hipSuccess) return hip_fail(e, "step_device: fold");
    }
    double pw1, pw2;
    bool same;
    zero_status st = h->opt == kOptAdam
        ? launch_adam_step(h, h->hp, s, src, &pw1, &pw2, &same, "step_device: update")
        : launch_sgd_step(h, h->sgd, s, src, "step_device: update");
    if (st == ZERO_OK && src.fold.partial != nullptr) h->inline_folds += 1;
    return st;
}

zero_status zero_shard_inline_folds(zero_shard_t h, int64_t* count)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "inline_folds: not a live handle");
    if (!count) return fail(ZERO_ERR_INVALID_ARG, "inline_folds: count is NULL");
    *count = h->inline_folds;
    return ZERO_OK;
}

zero_status zero_device_end(zero_shard_t h, void* stream, zero_step_info* out)
{
    if (!live(h)) return fail(ZERO_ERR_STATE, "device_end: not a live handle");
    if (zero_status ds = check_device(h, stream, "device_end")) return ds;
    if (!h->device_mode) return fail(ZERO_ERR_STATE, "device_end: the device flow is not active");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(h->host_dev, h->dev, sizeof(zk::DevState), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "device_end: state copy");
    const zk::DevState st = *h->host_dev;
    h->t = st.t;
    h->scale = st.scale;
    h->good_steps = st.good;
    if (h->opt == kOptAdam) {
        h->pw1 = st.pw1;
        h->pw2 = st.pw2;
        h->pw_t = st.t;
    }
    h->device_mode = false;
    zero_step_info info;
    std::memset(&info, 0, sizeof(info));
    info.step_t = h->t;
    info.scale_next = h->scale;
    info.scale_used = h->scale;
    if (st.steps_run > 0) {
        info.overflow = std::isfinite(st.last_sumsq) ? 0 : 1;
        info.skipped = info.overflow;
        info.grad_norm = std::sqrt(st.last_sumsq);
        info.scale_used = st.last_scale;
    }
    if (out) *out = info;
    return ZERO_OK;
}

}  // extern "C"

// ----------------------------------------------------------------- no allocation

// Scratch of zero_adam_step_noalloc: the check result (first 256 bytes), the
// fold's first level, then the per-workgroup partials.  Every GPU the library
// runs on holds one copy until the process ends.  Nothing in it must start at
// zero: each launch writes every slot it later reads.
constexpr size_t kNoallocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) double scratch[kNoallocScratchBytes / sizeof(double)];

namespace {

constexpr int kNoallocMaxDevices = 64;
constexpr int64_t kNoallocHead = 256 / sizeof(double);
constexpr int64_t kNoallocMaxSlots =
    (int64_t)(kNoallocScratchBytes / sizeof(double)) - kNoallocHead - zk::kFoldMaxBlocks;
static_assert(sizeof(zk::CheckResult) <= 256, "check result fits the scratch head");

struct NoallocDevice {
    double* ptr = nullptr;   // device address of this device's scratch
    int lds_cu = 0, lds_blk = 0;
};
std::mutex g_noalloc_mu;
NoallocDevice g_noalloc[kNoallocMaxDevices];

// Once per device, with that device current: the device address of its copy
// of `scratch` (host code must never pass the array's own name to a kernel:
// on the host it names a host-side stand-in) and its LDS limits.
zero_status noalloc_device(int dev, NoallocDevice* out, const char* who)
{
    if (dev < 0 || dev >= kNoallocMaxDevices)
        return fail(ZERO_ERR_UNSUPPORTED, "%s: device %d beyond the %d this entry point serves",
                    who, dev, kNoallocMaxDevices);
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    NoallocDevice& d = g_noalloc[dev];
    if (d.ptr == nullptr) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                            "adam_step_noalloc: hipGetSymbolAddress of the scratch");
        }
        query_lds(dev, &d.lds_cu, &d.lds_blk);
        d.ptr = static_cast<double*>(p);
    }
    *out = d;
    return ZERO_OK;
}

}  // namespace

extern "C" {

zero_status zero_adam_step_noalloc(const zero_shard_desc* desc, const zero_adam_hparams* hp,
                                   const zero_loss_scale_cfg* ls, double max_grad_norm,
                                   const void* const* contribs, int32_t n_contrib,
                                   int64_t* step_t, double* scale, int64_t* good_steps,
                                   void* stream, zero_step_info* out)
{
    const char* who = "adam_step_noalloc";
    if (!desc || !step_t || !scale || !good_steps)
        return fail(ZERO_ERR_INVALID_ARG, "%s: NULL desc or counter", who);
    zero_status st = check_hparams(hp);
    if (st != ZERO_OK) return st;
    int64_t S = 0;
    if ((st = check_desc(*desc, 1, 1, who, &S)) != ZERO_OK) return st;
    if ((st = check_ls(ls)) != ZERO_OK) return st;
    if (*step_t < 0 || !scale_ok(*scale) || *good_steps < 0)
        return fail(ZERO_ERR_INVALID_ARG, "%s: counters out of range", who);
    if (!(std::isfinite(max_grad_norm) && max_grad_norm >= 0.0))
        return fail(ZERO_ERR_INVALID_ARG, "%s: max_grad_norm must be finite and >= 0", who);
    const bool scan = contribs == nullptr && n_contrib == 0;

    // the step's state lives on this stack frame: no handle, no allocation
    zero_shard_s h;
    h.d = *desc;
    h.S = S;
    h.opt = kOptAdam;
    h.esz = lp_bytes(desc->lp);
    h.hp = *hp;
    h.ls = *ls;
    h.t = *step_t;
    h.scale = *scale;
    h.good_steps = *good_steps;
    h.pw_t = -1;
    h.max_norm = max_grad_norm;
    if (!scan && (st = check_contribs(&h, contribs, n_contrib, who)) != ZERO_OK) return st;
    hipError_t e = hipGetDevice(&h.device);
    if (e != hipSuccess) return hip_fail(e, who);
    if ((st = check_device(&h, stream, who)) != ZERO_OK) return st;

    // the partial slots of the step's reduce (or scan) launches, counted
    // before anything is launched, against what the scratch holds
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto enqueue_check = [&](bool launch, int64_t* slots) -> zero_status {
        *slots = 0;
        if (scan) return enqueue_scan(&h, nullptr, s, slots, who, nullptr, launch);
        const void* ptrs[ZERO_MAX_CONTRIB];
        for (int64_t off = 0; off < S; off += desc->bucket_elems) {
            const int64_t len = S - off < desc->bucket_elems ? S - off : desc->bucket_elems;
            for (int r = 0; r < n_contrib; ++r)
                ptrs[r] = static_cast<const char*>(contribs[r]) + off * h.esz;
            int64_t blocks = 0;
            zero_status rs = enqueue_reduce(&h, ptrs, n_contrib, off, len, *slots, nullptr, s,
                                            &blocks, who, nullptr, launch);
            if (rs != ZERO_OK) return rs;
            *slots += blocks;
        }
        return ZERO_OK;
    };
    int64_t slots = 0;
    h.nslots = INT64_MAX;
    if ((st = enqueue_check(false, &slots)) != ZERO_OK) return st;
    if (slots > kNoallocMaxSlots)
        return fail(ZERO_ERR_INVALID_ARG,
                    "%s: this shard's check needs %lld partial slots, the %zu-byte static "
                    "scratch holds %lld; use a handle (zero_shard_init) for larger shards",
                    who, (long long)slots, kNoallocScratchBytes, (long long)kNoallocMaxSlots);
    if ((st = check_desc_ranges(*desc, S, h.device, who)) != ZERO_OK) return st;
    if (!scan && (st = check_contrib_overlap(&h, contribs, n_contrib, 0, S, who)) != ZERO_OK)
        return st;

    NoallocDevice nd;
    if ((st = noalloc_device(h.device, &nd, who)) != ZERO_OK) return st;
    set_lds_reserves(&h, nd.lds_cu, nd.lds_blk);
    h.result = reinterpret_cast<zk::CheckResult*>(nd.ptr);
    h.level1 = nd.ptr + kNoallocHead;
    h.partial = h.level1 + zk::kFoldMaxBlocks;
    h.nslots = kNoallocMaxSlots;

    if ((st = enqueue_check(true, &slots)) != ZERO_OK) return st;
    const zk::PrepareArgs none{};
    e = zk::launch_finalize(h.partial, slots, h.level1, h.result, h.max_norm, nullptr, none, s);
    if (e != hipSuccess) return hip_fail(e, who);
    zk::CheckResult res;
    e = hipMemcpyAsync(&res, h.result, sizeof(res), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, who);
    h.host_result = &res;
    zero_step_info info = read_check(&h);
    double pw1 = 1.0, pw2 = 1.0;
    bool same = false;
    if (!info.overflow) {
        st = launch_adam_step(&h, *hp, s, source_sync(&h), &pw1, &pw2, &same, who);
        if (st != ZERO_OK) return st;
    }
    commit_step(&h, &info, pw1, pw2, same);
    *step_t = h.t;
    *scale = h.scale;
    *good_steps = h.good_steps;
    if (out) *out = info;
    return ZERO_OK;
}

}  // extern "C"
