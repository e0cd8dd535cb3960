/*
 * zero_oracle.c -- plain, slow, scalar CPU oracle for the owner-rank step of
 * ZeRO-DP (optimizer-state partitioning P_os and gradient partitioning P_os+g).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the GPU library: it has its own half-precision converters, its own scalar
 * set-up and its own byte ledger.
 *
 * Sources (the pages this follows):
 *  [P1] "AI论文陪读·ZeRO：分布式训练的第一篇论文（中英双语）", section 01
 *       (memory breakdown: fp16 params 2 bytes, fp16 grads 2 bytes, Adam
 *       K = 12 bytes of fp32 master/momentum/variance per parameter).
 *  [P2] "ZeRO：大模型训练的内存优化革命", sections 3.1.1 (P_os: each DP
 *       process stores and updates 1/Nd of the optimizer state, then the
 *       updated parameters are all-gathered), 3.1.2 (P_os+g: gradients are
 *       reduced only on the process owning that partition), 3.2.2 (C_B:
 *       constant-size fused buffers).
 *  [P3] blog.vllbc.top "ZeRO / DeepSpeed" visual reading: the 16-byte ledger,
 *       the stage formulas (Stage 0 = (2b+K)Psi, Stage 1, 2, 3), the worked
 *       examples A (7.5B, Nd=64), B (128B, Nd=64), C1 and C2, Table 1, Table 2,
 *       the display rule, and the statement that ZeRO-DP changes neither the
 *       optimizer nor the math of a step, only where the states live.
 *  [P4] "SC-2020 ZeRO: Memory Optimizations Toward Training Trillion Parameter
 *       Models" notes, "Where Did All the Memory Go?": updates run on fp32
 *       weights, which are then cast back to fp16.
 *
 * The pages give no Adam formula, no loss scaling and no summation order.
 * Where they are silent this file takes these readings:
 *  - Adam is the textbook algorithm (Kingma & Ba 2015, Algorithm 1): bias-
 *    corrected first and second moments, epsilon added outside the square root.
 *  - The reduce is the mean over the R contributions actually reduced, summed
 *    in fp32 in ascending contribution order starting from +0.0f.
 *  - The reduced gradient shard is stored in the 2-byte format (16 Psi/Nd
 *    ledger); overflow is any non-finite stored or unscaled value; a step
 *    with overflow is skipped and, with dynamic scaling, halves the loss
 *    scale.
 *  - Weight decay is decoupled (AdamW form, scaled by lr) unless L2 mode is set.
 *  - Floating point: fp32 arithmetic as the pages fix for the optimizer state
 *    ("fp32 momentum, variance and parameter copy"); every operation rounds to
 *    nearest-even with no contraction (built with -ffp-contract=off); the
 *    gradient norm is accumulated in fp64.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_FP16 1
#define ORACLE_BF16 2
#define ORACLE_FP32 3   /* 4-byte storage of grads and params (the pages' b = 4) */

/* ------------------------------------------------------------------------ */
/* 2-byte formats.  IEEE binary16 and bfloat16, round to nearest, ties to    */
/* even.  [P1] section 01 and [P3] ledger: params and grads are 2-byte       */
/* values; [P4] "Where Did All the Memory Go?": fp32 results are cast back.  */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* binary16 -> binary32, exact. */
float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu;
    uint32_t f = h & 0x3ffu;
    if (e == 0) {
        /* zero or subnormal: value = f * 2^-24, exact in fp32 */
        float mag = (float)f * 5.9604644775390625e-8f;
        return sign ? -mag : mag;
    }
    if (e == 31)                       /* inf or NaN, payload kept */
        return bits_f32(sign | 0x7f800000u | (f << 13));
    return bits_f32(sign | ((e + 112u) << 23) | (f << 13));
}

/* binary32 -> binary16, round to nearest even; |x| >= 65520 becomes inf. */
uint16_t oracle_f32_to_f16(float x)
{
    uint32_t u = f32_bits(x);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t e8 = (u >> 23) & 0xffu;
    uint32_t f = u & 0x7fffffu;
    if (e8 == 0xffu)                   /* inf stays inf; NaN stays a quiet NaN */
        return (uint16_t)(sign | 0x7c00u | (f ? (0x200u | (f >> 13)) : 0u));
    int e = (int)e8 - 127 + 15;        /* binary16 biased exponent */
    if (e >= 31)
        return (uint16_t)(sign | 0x7c00u);
    if (e <= 0) {
        /* result is a binary16 subnormal (or rounds up to the smallest normal);
         * unit 2^-24; |x| = sig * 2^(e8-150) with a 24-bit significand */
        if (e < -10)
            return (uint16_t)sign;     /* below half of 2^-24 */
        uint32_t sig = f | 0x800000u;
        int drop = 14 - e;             /* 14 .. 24 bits dropped */
        uint32_t q = sig >> drop;
        uint32_t rem = sig & ((1u << drop) - 1u);
        uint32_t half = 1u << (drop - 1);
        if (rem > half || (rem == half && (q & 1u)))
            q++;
        return (uint16_t)(sign | q);
    }
    uint32_t q = ((uint32_t)e << 10) | (f >> 13);
    uint32_t rem = f & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u)))
        q++;                           /* a carry may reach the inf encoding */
    return (uint16_t)(sign | q);
}

/* bfloat16 -> binary32, exact (the top half of the fp32 encoding). */
float oracle_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* binary32 -> bfloat16, round to nearest even; NaN stays a quiet NaN. */
uint16_t oracle_f32_to_bf16(float x)
{
    uint32_t u = f32_bits(x);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu))
        return (uint16_t)((u >> 16) | 0x40u);
    uint32_t keep = u >> 16;
    uint32_t rem = u & 0xffffu;
    if (rem > 0x8000u || (rem == 0x8000u && (keep & 1u)))
        keep++;                        /* may carry into the exponent, up to inf */
    return (uint16_t)keep;
}

static float lp_to_f32(int lp, uint16_t v)
{
    return lp == ORACLE_BF16 ? oracle_bf16_to_f32(v) : oracle_f16_to_f32(v);
}

static uint16_t f32_to_lp(int lp, float x)
{
    return lp == ORACLE_BF16 ? oracle_f32_to_bf16(x) : oracle_f32_to_f16(x);
}

/* Gradients, contributions and 2-byte params live as uint16 bit patterns;
 * with 4-byte storage they are plain fp32 values. */
static float load_g(int lp, const void* a, int64_t i)
{
    if (lp == ORACLE_FP32) return ((const float*)a)[i];
    return lp_to_f32(lp, ((const uint16_t*)a)[i]);
}

static void store_g(int lp, void* a, int64_t i, float x)
{
    if (lp == ORACLE_FP32)
        ((float*)a)[i] = x;
    else
        ((uint16_t*)a)[i] = f32_to_lp(lp, x);
}

void oracle_lp_to_f32_array(int lp, const uint16_t* in, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = lp_to_f32(lp, in[i]);
}

void oracle_f32_to_lp_array(int lp, const float* in, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_lp(lp, in[i]);
}

/* ------------------------------------------------------------------------ */
/* Flat partition.  [P2] 3.1.1 / 3.1.2 and [P3] stage descriptions: each of  */
/* the Nd data-parallel ranks owns 1/Nd of the flattened state.  Rank r owns */
/* elements [r*S, (r+1)*S) with S = ceil(Psi/Nd); the last shard is padded   */
/* with zeros when Nd does not divide Psi.  Tensor boundaries play no part.  */
/* ------------------------------------------------------------------------ */

void oracle_partition(int64_t psi, int32_t nd, int32_t rank,
                      int64_t* shard_elems, int64_t* begin, int64_t* valid)
{
    int64_t s = (psi + nd - 1) / nd;
    int64_t b = (int64_t)rank * s;
    int64_t v = psi - b;
    if (v > s) v = s;
    if (v < 0) v = 0;
    *shard_elems = s;
    *begin = b;
    *valid = v;
}

/* Copy the owner's shard out of a flat 2-byte buffer, zero-padding the tail. */
void oracle_take_shard_u16(const uint16_t* flat, int64_t psi, int32_t nd,
                           int32_t rank, uint16_t* shard)
{
    int64_t s, b, v;
    oracle_partition(psi, nd, rank, &s, &b, &v);
    for (int64_t i = 0; i < s; ++i) shard[i] = i < v ? flat[b + i] : 0;
}

void oracle_take_shard_f32(const float* flat, int64_t psi, int32_t nd,
                           int32_t rank, float* shard)
{
    int64_t s, b, v;
    oracle_partition(psi, nd, rank, &s, &b, &v);
    for (int64_t i = 0; i < s; ++i) shard[i] = i < v ? flat[b + i] : 0.0f;
}

/* ------------------------------------------------------------------------ */
/* Gradient reduce to the owner, one bucket.  [P2] 3.1.2: gradients are      */
/* reduced only on the owner of the partition; [P3] communication ledger:    */
/* the all-reduce splits into a reduce-scatter plus an all-gather; [P2]      */
/* 3.2.2 and [P4] "C_B": a constant-size buffer carries one bucket.          */
/* Per element: acc = +0, then acc += f32(c_r) for r = 0..R-1 in order;      */
/* g = rne_lp(acc * (1/R)).                                                   */
/* ------------------------------------------------------------------------ */

void oracle_bucket_reduce(int lp, int32_t n_contrib, const void* const* contribs,
                          int64_t n, void* out)
{
    float inv_r = (float)(1.0 / (double)n_contrib);
    for (int64_t i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (int32_t r = 0; r < n_contrib; ++r)
            acc = acc + load_g(lp, contribs[r], i);
        store_g(lp, out, i, acc * inv_r);
    }
}

/* ------------------------------------------------------------------------ */
/* Unscale, overflow check and squared gradient norm over a stored shard.    */
/* The pages are silent on loss scaling; reading: the step unscales first and */
/* then checks for inf/nan, so the flag is set when an unscaled fp32 value    */
/* u = x * (1/scale) is not finite.  That covers every non-finite stored x    */
/* (inf or NaN times any factor is inf or NaN) and also a finite x that       */
/* unscales to inf under a scale below 1.  sumsq adds u*u in fp64.            */
/* Accumulates into *flag and *sumsq.                                         */
/* ------------------------------------------------------------------------ */

void oracle_flag_sumsq(int lp, const void* g, int64_t n, float inv_scale,
                       int32_t* flag, double* sumsq)
{
    int32_t f = *flag;
    double s = *sumsq;
    for (int64_t i = 0; i < n; ++i) {
        float x = load_g(lp, g, i);
        float u = x * inv_scale;
        if (!isfinite(u)) f = 1;
        s += (double)u * (double)u;
    }
    *flag = f;
    *sumsq = s;
}

/* ------------------------------------------------------------------------ */
/* Global-norm clipping coefficient (the pages are silent; the textbook rule, */
/* as in PyTorch's clip_grad_norm_): with norm = sqrt(sumsq) of the unscaled  */
/* gradient and a limit max_norm > 0, coef = min(1, max_norm/(norm + 1e-6)),  */
/* computed in fp64 and rounded to fp32; max_norm <= 0 disables clipping      */
/* (coef = 1).  The update multiplies the unscaled gradient by coef.          */
/* ------------------------------------------------------------------------ */

float oracle_clip_coef(double sumsq, double max_norm)
{
    if (!(max_norm > 0.0)) return 1.0f;
    double norm = sqrt(sumsq);
    double c = max_norm / (norm + 1e-6);
    return c < 1.0 ? (float)c : 1.0f;
}

/* ------------------------------------------------------------------------ */
/* Host scalars of one applied Adam step (t counts applied steps, t >= 1).   */
/* out: [0] beta1 [1] beta2 [2] 1-beta1 [3] 1-beta2 [4] bias corr. 1          */
/*      [5] bias corr. 2 [6] lr [7] eps [8] weight decay [9] 1/scale          */
/*      [10] clipping coefficient (set to 1 here; the caller may replace it)  */
/* beta^t is the product of t copies of the fp32-rounded beta, in fp64.       */
/* ------------------------------------------------------------------------ */

void oracle_adam_scalars(double beta1, double beta2, double lr, double eps,
                         double weight_decay, int32_t bias_correction,
                         int64_t t, double loss_scale, float* out)
{
    float b1 = (float)beta1, b2 = (float)beta2;
    double pw1 = 1.0, pw2 = 1.0;
    for (int64_t k = 0; k < t; ++k) {
        pw1 = pw1 * (double)b1;
        pw2 = pw2 * (double)b2;
    }
    out[0] = b1;
    out[1] = b2;
    out[2] = 1.0f - b1;
    out[3] = 1.0f - b2;
    out[4] = bias_correction ? (float)(1.0 - pw1) : 1.0f;
    out[5] = bias_correction ? (float)(1.0 - pw2) : 1.0f;
    out[6] = (float)lr;
    out[7] = (float)eps;
    out[8] = (float)weight_decay;
    out[9] = (float)(1.0 / loss_scale);
    out[10] = 1.0f;
}

/* ------------------------------------------------------------------------ */
/* Adam on the owner's fp32 shard and the cast into the 2-byte all-gather     */
/* slice.  [P2] 3.1.1: the rank updates only its 1/Nd of the states, then the */
/* parameters are all-gathered; [P3] Stage 3 section: the step updates only   */
/* the local fp32 parameter shard and optimizer state; [P4] "Where Did All    */
/* the Memory Go?": the update runs on fp32 weights, then casts to fp16.      */
/* Textbook Adam (Kingma & Ba 2015, Algorithm 1) per element:                 */
/*   g  = f32(grad) * (1/scale) ; g = g * coef  [clipping]                   */
/*                                        [L2 mode: g += wd * p]              */
/*   m  = b1*m + (1-b1)*g                                                     */
/*   v  = b2*v + (1-b2)*(g*g)                                                 */
/*   u  = (m/bc1) / (sqrt(v/bc2) + eps)  [decoupled mode: u += wd * p]        */
/*   p  = p - lr*u;   param = rne_lp(p)                                       */
/* wd_mode: 0 decoupled, 1 L2.  A zero weight decay adds no term.             */
/* ------------------------------------------------------------------------ */

void oracle_adam_update(int lp, int64_t n, const void* grad, float* master,
                        float* exp_avg, float* exp_avg_sq, void* param,
                        const float* sc, int32_t wd_mode)
{
    float b1 = sc[0], b2 = sc[1], omb1 = sc[2], omb2 = sc[3];
    float bc1 = sc[4], bc2 = sc[5], lr = sc[6], eps = sc[7], wd = sc[8];
    float inv_scale = sc[9], coef = sc[10];
    for (int64_t i = 0; i < n; ++i) {
        float p = master[i];
        float g = load_g(lp, grad, i) * inv_scale;
        if (coef != 1.0f)
            g = g * coef;
        if (wd_mode == 1 && wd != 0.0f)
            g = g + wd * p;
        float m = b1 * exp_avg[i] + omb1 * g;
        float v = b2 * exp_avg_sq[i] + omb2 * (g * g);
        float m_hat = m / bc1;
        float v_hat = v / bc2;
        float u = m_hat / (sqrtf(v_hat) + eps);
        if (wd_mode == 0 && wd != 0.0f)
            u = u + wd * p;
        p = p - lr * u;
        master[i] = p;
        exp_avg[i] = m;
        exp_avg_sq[i] = v;
        if (param) store_g(lp, param, i, p);
    }
}

/* ------------------------------------------------------------------------ */
/* SGD on the owner's shard (the optimizers of the blog.vllbc.top page's      */
/* extension group C: SGD with momentum, K = 4 bytes of state, and plain SGD, */
/* K = 0).  The pages give no formula; textbook heavy-ball SGD, with the      */
/* classic L2 weight decay folded into the gradient:                          */
/*   g = f32(grad) * (1/scale) ; g = g * coef   [clipping]                   */
/*                                        [wd != 0: g = g + wd * p]           */
/*   with momentum:  buf = mu*buf + g ;  d = buf                              */
/*   plain SGD:      d = g                                                    */
/*   p = p - lr*d ;  2-byte storage: param = rne_lp(p)                        */
/* sc: [0] lr [1] mu [2] wd [3] 1/scale [4] clipping coefficient.            */
/* momentum == NULL: plain SGD.                                               */
/* ------------------------------------------------------------------------ */

void oracle_sgd_update(int lp, int64_t n, const void* grad, float* master, float* momentum,
                       void* param, const float* sc)
{
    float lr = sc[0], mu = sc[1], wd = sc[2], inv_scale = sc[3], coef = sc[4];
    for (int64_t i = 0; i < n; ++i) {
        float p = master[i];
        float g = load_g(lp, grad, i) * inv_scale;
        if (coef != 1.0f)
            g = g * coef;
        if (wd != 0.0f)
            g = g + wd * p;
        float d = g;
        if (momentum) {
            float b = mu * momentum[i] + g;
            momentum[i] = b;
            d = b;
        }
        p = p - lr * d;
        master[i] = p;
        if (param) store_g(lp, param, i, p);
    }
}

/* ------------------------------------------------------------------------ */
/* Loss-scale bookkeeping after the skip decision (pages silent; reading:     */
/* halve on overflow down to min_scale, double after growth_interval clean    */
/* steps; a static scale never changes).                                      */
/* ------------------------------------------------------------------------ */

void oracle_loss_scale_next(int32_t overflow, int32_t dynamic, int32_t growth_interval,
                            double min_scale, double* scale, int64_t* good_steps)
{
    if (!dynamic) return;
    if (overflow) {
        double s = *scale / 2.0;
        *scale = s < min_scale ? min_scale : s;
        *good_steps = 0;
    } else {
        *good_steps += 1;
        if (*good_steps == growth_interval) {
            *scale = *scale * 2.0;
            *good_steps = 0;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Per-rank model-state ledger.  [P1] 01 and [P3] ledger: b bytes per param   */
/* for params and for grads (2 in mixed precision, 4 in fp32), K bytes of     */
/* optimizer state (12 for mixed-precision Adam).  [P3] stage formulas:       */
/*   Stage 0 = (2b+K) Psi                                                     */
/*   Stage 1 = 2b Psi + K Psi/Nd           (optimizer state partitioned)      */
/*   Stage 2 = b Psi + (b+K) Psi/Nd        (+ gradients partitioned)          */
/*   Stage 3 = (2b+K) Psi/Nd               (+ parameters partitioned)         */
/* [P3] communication ledger: 2 Psi elements per rank per step for stages     */
/* 0-2, 3 Psi for stage 3 (b bytes each); stage 1 with the step-end gather    */
/* counts 3 Psi.  Allocated bytes of the library's shard: master, m, v in fp32 */
/* and grad, param in the 2-byte format = (12 + 2*lp) * S.                    */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t shard_elems;
    int64_t bytes_master, bytes_m, bytes_v, bytes_grad, bytes_param;
    int64_t bytes_shard_total, bytes_staging;
    double per_rank_stage[4];
    double comm_bytes_stage[4];
    double comm_bytes_stage1_with_gather;
    double comp_params[4], comp_grads[4], comp_optim[4];
} oracle_bytes;

void oracle_state_bytes(int64_t psi, int32_t nd, int32_t n_contrib, int64_t bucket_elems,
                        int32_t lp_bytes, int32_t param_bytes, int32_t k_optim,
                        oracle_bytes* out)
{
    int64_t s = (psi + nd - 1) / nd;
    double P = (double)psi, N = (double)nd, b = (double)param_bytes, K = (double)k_optim;
    memset(out, 0, sizeof(*out));
    out->shard_elems = s;
    /* The shard the library allocates for storage lp_bytes and optimizer
       state K.  With 2-byte storage K counts the fp32 master copy (12 = 4
       master + 8 Adam moments); with 4-byte storage the fp32 master is the
       parameter and K counts only the optimizer's own arrays (8 Adam, 4 SGD
       momentum, 0 plain SGD; the page's extension group C).  The optimizer's
       arrays are fp32: a first one when they take 4 bytes, a second at 8. */
    int64_t opt = lp_bytes == 4 ? k_optim : k_optim - 4;
    out->bytes_master = 4 * s;
    out->bytes_m = opt >= 4 ? 4 * s : 0;
    out->bytes_v = opt >= 8 ? 4 * s : 0;
    out->bytes_grad = (int64_t)lp_bytes * s;
    out->bytes_param = lp_bytes == 4 ? 0 : (int64_t)lp_bytes * s;
    out->bytes_shard_total = out->bytes_master + out->bytes_m + out->bytes_v
                           + out->bytes_grad + out->bytes_param;
    out->bytes_staging = (int64_t)n_contrib * bucket_elems * lp_bytes;

    /* components per stage: params, grads, optimizer state */
    for (int st = 0; st < 4; ++st) {
        out->comp_params[st] = st < 3 ? b * P : (b * P) / N;
        out->comp_grads[st] = st < 2 ? b * P : (b * P) / N;
        out->comp_optim[st] = st < 1 ? K * P : (K * P) / N;
    }
    out->per_rank_stage[0] = (2.0 * b + K) * P;
    out->per_rank_stage[1] = 2.0 * b * P + (K * P) / N;
    out->per_rank_stage[2] = b * P + ((b + K) * P) / N;
    out->per_rank_stage[3] = ((2.0 * b + K) * P) / N;
    for (int st = 0; st < 3; ++st) out->comm_bytes_stage[st] = 2.0 * P * b;
    out->comm_bytes_stage[3] = 3.0 * P * b;
    out->comm_bytes_stage1_with_gather = 3.0 * P * b;
}

int oracle_abi(void) { return 1; }
