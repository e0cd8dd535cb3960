// Per-rank model-state ledger (pure host arithmetic).
//
// Byte model from "AI论文陪读·ZeRO" section 01 and the blog.vllbc.top
// ZeRO/DeepSpeed page (ledger, stage formulas, Table 1, worked examples A/B,
// extension group C): with b bytes per parameter and per gradient and K bytes
// of optimizer state per parameter, a data-parallel rank holds
//   stage 0 (plain DP):               (2b + K) Psi
//   stage 1 (optimizer partitioned):  2b Psi + K Psi / Nd
//   stage 2 (+ gradients):            b Psi + (b + K) Psi / Nd
//   stage 3 (+ parameters):           (2b + K) Psi / Nd
// and the communication ledger of the same page moves 2 Psi elements per step
// for stages 0-2 and 3 Psi for stage 3 (stage 1 counts 3 Psi when the
// step-end parameter gather is included).

#include <cstring>

#include "../../include/zero_shard.h"

namespace {

// The caller's enum argument through its 32-bit representation: a value
// outside the enumerators is then an ordinary integer to refuse, not an
// out-of-range enum load (undefined in C++).
int32_t enum_value(const zero_lp_dtype& e)
{
    static_assert(sizeof(zero_lp_dtype) == sizeof(int32_t), "32-bit enum");
    int32_t v;
    std::memcpy(&v, &e, sizeof(v));
    return v;
}

zero_status ledger(int64_t psi, int32_t nd, int32_t n_contrib, int64_t bucket_elems,
                   int32_t lp, int32_t b_bytes, int32_t k_optim, zero_state_bytes_t* out)
{
    if (!out || psi < 1 || nd < 1 || n_contrib < 1 || n_contrib > ZERO_MAX_CONTRIB ||
        bucket_elems < 1 || (lp != ZERO_FP16 && lp != ZERO_BF16 && lp != ZERO_FP32) ||
        (b_bytes != 2 && b_bytes != 4) || k_optim < 0)
        return ZERO_ERR_INVALID_ARG;
    const int64_t shard = psi / nd + (psi % nd != 0 ? 1 : 0);
    zero_state_bytes_t r;
    std::memset(&r, 0, sizeof(r));
    r.shard_elems = shard;
    // The shard a handle allocates: the fp32 master (with 4-byte storage it is
    // the parameter itself, and no 2-byte copy exists), the optimizer's fp32
    // arrays, the stored gradient and the 2-byte parameter.  K counts the
    // master copy with 2-byte storage (12 = 4 + 8 Adam) and only the
    // optimizer's arrays with 4-byte storage (8 Adam, 4 SGD momentum, 0 SGD).
    const int64_t esz = lp == ZERO_FP32 ? 4 : 2;
    const int64_t opt = lp == ZERO_FP32 ? k_optim : k_optim - 4;
    r.bytes_master = shard * 4;
    r.bytes_m = opt >= 4 ? shard * 4 : 0;
    r.bytes_v = opt >= 8 ? shard * 4 : 0;
    r.bytes_grad = shard * esz;
    r.bytes_param = lp == ZERO_FP32 ? 0 : shard * 2;
    r.bytes_shard_total = r.bytes_master + r.bytes_m + r.bytes_v + r.bytes_grad + r.bytes_param;
    r.bytes_staging = (int64_t)n_contrib * bucket_elems * esz;

    const double P = (double)psi;
    const double N = (double)nd;
    const double b = (double)b_bytes;
    const double K = (double)k_optim;
    const double params_full = b * P, grads_full = b * P, optim_full = K * P;
    const double params_part = params_full / N, grads_part = grads_full / N,
                 optim_part = optim_full / N;
    // stage: 0 nothing partitioned, 1 optimizer, 2 + gradients, 3 + parameters
    for (int st = 0; st < 4; ++st) {
        r.comp_optim[st] = st >= 1 ? optim_part : optim_full;
        r.comp_grads[st] = st >= 2 ? grads_part : grads_full;
        r.comp_params[st] = st >= 3 ? params_part : params_full;
    }
    r.per_rank_stage[0] = (2.0 * b + K) * P;
    r.per_rank_stage[1] = 2.0 * b * P + K * P / N;
    r.per_rank_stage[2] = b * P + (b + K) * P / N;
    r.per_rank_stage[3] = (2.0 * b + K) * P / N;
    r.comm_bytes_stage[0] = r.comm_bytes_stage[1] = r.comm_bytes_stage[2] = 2.0 * P * b;
    r.comm_bytes_stage[3] = 3.0 * P * b;
    r.comm_bytes_stage1_with_gather = 3.0 * P * b;
    *out = r;
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_state_bytes(int64_t psi, int32_t nd, int32_t n_contrib,
                                        int64_t bucket_elems, zero_lp_dtype lp,
                                        zero_state_bytes_t* out)
{
    return ledger(psi, nd, n_contrib, bucket_elems, enum_value(lp), 2, 12, out);
}

extern "C" zero_status zero_state_bytes_ex(int64_t psi, int32_t nd, int32_t n_contrib,
                                           int64_t bucket_elems, zero_lp_dtype lp,
                                           int32_t param_bytes, int32_t k_optim,
                                           zero_state_bytes_t* out)
{
    return ledger(psi, nd, n_contrib, bucket_elems, enum_value(lp), param_bytes, k_optim, out);
}
