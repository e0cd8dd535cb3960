"""The oracle's pins catch plausible mistakes: each mutation below plants one
(a dropped term, a wrong sign, index, operand or constant) in a copy of
oracle/zero_oracle.c, the copy is built with the oracle's own flags, and the
pin suite (ledger, formats, step) must fail against it."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "oracle", "zero_oracle.c")
PINS = ["tests/test_oracle_ledger.py", "tests/test_oracle_formats.py", "tests/test_oracle_step.py",
        "tests/test_oracle_sgd.py", "tests/test_oracle_clip.py"]

# (name, exact text in zero_oracle.c, replacement); each text occurs once
MUTATIONS = [
    ("reduce starts from -0", "float acc = 0.0f;", "float acc = -0.0f;"),
    ("reduce divides by R+1", "float inv_r = (float)(1.0 / (double)n_contrib);",
     "float inv_r = (float)(1.0 / (double)(n_contrib + 1));"),
    ("reduce drops the last contribution", "for (int32_t r = 0; r < n_contrib; ++r)",
     "for (int32_t r = 0; r < n_contrib - 1; ++r)"),
    ("fp16 ties away from zero", "if (rem > 0x1000u || (rem == 0x1000u && (q & 1u)))",
     "if (rem >= 0x1000u)"),
    ("fp16 overflow threshold", "    if (e >= 31)\n        return (uint16_t)(sign | 0x7c00u);",
     "    if (e > 31)\n        return (uint16_t)(sign | 0x7c00u);"),
    ("fp16 subnormal shift", "int drop = 14 - e;", "int drop = 13 - e;"),
    ("bf16 rounding", "if (rem > 0x8000u || (rem == 0x8000u && (keep & 1u)))",
     "if (rem >= 0x8000u)"),
    ("fp16 subnormal decode", "float mag = (float)f * 5.9604644775390625e-8f;",
     "float mag = (float)f * 1.1920928955078125e-7f;"),
    ("momentum uses beta2", "float m = b1 * exp_avg[i] + omb1 * g;",
     "float m = b2 * exp_avg[i] + omb1 * g;"),
    ("variance uses g not g^2", "float v = b2 * exp_avg_sq[i] + omb2 * (g * g);",
     "float v = b2 * exp_avg_sq[i] + omb2 * g;"),
    ("eps inside the square root", "float u = m_hat / (sqrtf(v_hat) + eps);",
     "float u = m_hat / sqrtf(v_hat + eps);"),
    ("bias corrections swapped", "float m_hat = m / bc1;", "float m_hat = m / bc2;"),
    ("update sign", "p = p - lr * u;", "p = p + lr * u;"),
    ("decoupled decay sign", "u = u + wd * p;", "u = u - wd * p;"),
    ("Adam L2 decay sign", "if (wd_mode == 1 && wd != 0.0f)\n            g = g + wd * p;",
     "if (wd_mode == 1 && wd != 0.0f)\n            g = g - wd * p;"),
    ("Adam ignores the loss scale",
     "float g = load_g(lp, grad, i) * inv_scale;\n        if (coef != 1.0f)\n            g = g * coef;\n        if (wd_mode == 1",
     "float g = load_g(lp, grad, i);\n        if (coef != 1.0f)\n            g = g * coef;\n        if (wd_mode == 1"),
    ("bias correction of step t-1", "for (int64_t k = 0; k < t; ++k) {",
     "for (int64_t k = 1; k < t; ++k) {"),
    ("1-beta1 from beta2", "out[2] = 1.0f - b1;", "out[2] = 1.0f - b2;"),
    ("flag misses inf", "if (!isfinite(u)) f = 1;", "if (isnan(u)) f = 1;"),
    ("norm not unscaled", "float u = x * inv_scale;", "float u = x;"),
    ("flag tests the stored value, not the unscaled one",
     "float u = x * inv_scale;\n        if (!isfinite(u)) f = 1;",
     "float u = x * inv_scale;\n        if (!isfinite(x)) f = 1;"),
    ("scale not halved", "double s = *scale / 2.0;", "double s = *scale;"),
    ("reduce divides by R", "store_g(lp, out, i, acc * inv_r);",
     "store_g(lp, out, i, acc / (float)n_contrib);"),
    ("fp16 NaN narrowed to inf", "(f ? (0x200u | (f >> 13)) : 0u)", "0u"),
    ("bf16 NaN rounded like a number",
     "    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu))\n        return (uint16_t)((u >> 16) | 0x40u);\n",
     ""),
    ("fp16 subnormal loses its sign", "return sign ? -mag : mag;", "return mag;"),
    ("fp16 exponent rebias off by one", "((e + 112u) << 23)", "((e + 111u) << 23)"),
    ("SGD stores the gradient as the buffer", "momentum[i] = b;", "momentum[i] = g;"),
    ("SGD momentum scales the gradient too", "float b = mu * momentum[i] + g;",
     "float b = mu * (momentum[i] + g);"),
    ("stage 0 counts one 2-byte copy", "out->per_rank_stage[0] = (2.0 * b + K) * P;",
     "out->per_rank_stage[0] = (b + K) * P;"),
    ("gradients partitioned from stage 1", "out->comp_grads[st] = st < 2 ? b * P : (b * P) / N;",
     "out->comp_grads[st] = st < 1 ? b * P : (b * P) / N;"),
    ("staging ignores the contribution count",
     "out->bytes_staging = (int64_t)n_contrib * bucket_elems * lp_bytes;",
     "out->bytes_staging = bucket_elems * lp_bytes;"),
    ("norm summed in fp32", "s += (double)u * (double)u;", "s = (double)((float)s + u * u);"),
    ("L2 decay before clipping",
     "if (coef != 1.0f)\n            g = g * coef;\n        if (wd_mode == 1 && wd != 0.0f)\n            g = g + wd * p;",
     "if (wd_mode == 1 && wd != 0.0f)\n            g = g + wd * p;\n        if (coef != 1.0f)\n            g = g * coef;"),
    ("bias correction applied when off", "out[4] = bias_correction ? (float)(1.0 - pw1) : 1.0f;",
     "out[4] = (float)(1.0 - pw1);"),
    ("variance corrected by bc1", "float v_hat = v / bc2;", "float v_hat = v / bc1;"),
    ("scale not floored at min_scale", "*scale = s < min_scale ? min_scale : s;", "*scale = s;"),
    ("scale grows one clean step late", "if (*good_steps == growth_interval)",
     "if (*good_steps > growth_interval)"),
    ("clean count kept after growth", "*scale = *scale * 2.0;\n            *good_steps = 0;",
     "*scale = *scale * 2.0;"),
    ("clean count kept after overflow", "        *good_steps = 0;\n    } else {",
     "    } else {"),
    ("static scale still halves", "    if (!dynamic) return;\n", ""),
    ("partition floors", "    int64_t s = (psi + nd - 1) / nd;\n    int64_t b = (int64_t)rank * s;",
     "    int64_t s = psi / nd;\n    int64_t b = (int64_t)rank * s;"),
    ("stage 2 drops b/Nd", "out->per_rank_stage[2] = b * P + ((b + K) * P) / N;",
     "out->per_rank_stage[2] = b * P + (K * P) / N;"),
    ("stage 1 keeps b not 2b", "out->per_rank_stage[1] = 2.0 * b * P + (K * P) / N;",
     "out->per_rank_stage[1] = b * P + (K * P) / N;"),
    ("stage-3 communication 2 Psi", "out->comm_bytes_stage[3] = 3.0 * P * b;",
     "out->comm_bytes_stage[3] = 2.0 * P * b;"),
    ("bf16 decoded as fp16", "return lp == ORACLE_BF16 ? oracle_bf16_to_f32(v) : oracle_f16_to_f32(v);",
     "return lp == ORACLE_BF16 ? oracle_f16_to_f32(v) : oracle_f16_to_f32(v);"),
    ("param cast from the momentum", "exp_avg_sq[i] = v;\n        if (param) store_g(lp, param, i, p);",
     "exp_avg_sq[i] = v;\n        if (param) store_g(lp, param, i, m);"),
    ("SGD momentum ignores mu", "float b = mu * momentum[i] + g;", "float b = momentum[i] + g;"),
    ("SGD steps along g, not the buffer", "d = b;", "d = g;"),
    ("SGD decay sign", "if (wd != 0.0f)\n            g = g + wd * p;",
     "if (wd != 0.0f)\n            g = g - wd * p;"),
    ("SGD step sign", "p = p - lr * d;", "p = p + lr * d;"),
    ("SGD ignores the loss scale",
     "float g = load_g(lp, grad, i) * inv_scale;\n        if (coef != 1.0f)\n            g = g * coef;\n        if (wd != 0.0f)",
     "float g = load_g(lp, grad, i);\n        if (coef != 1.0f)\n            g = g * coef;\n        if (wd != 0.0f)"),
    ("clip not clamped at 1", "return c < 1.0 ? (float)c : 1.0f;", "return (float)c;"),
    ("clip norm without the root", "double norm = sqrt(sumsq);", "double norm = sumsq;"),
    ("clip drops the 1e-6", "double c = max_norm / (norm + 1e-6);", "double c = max_norm / norm;"),
    ("Adam ignores the clip", "g = g * coef;\n        if (wd_mode == 1", "g = g * 1.0f;\n        if (wd_mode == 1"),
    ("SGD clips twice", "g = g * coef;\n        if (wd != 0.0f)", "g = g * coef * coef;\n        if (wd != 0.0f)"),
    ("fp32 storage read as 2-byte", "if (lp == ORACLE_FP32) return ((const float*)a)[i];",
     "if (lp == 99) return ((const float*)a)[i];"),
    ("fp32 storage written rounded to fp16", "    if (lp == ORACLE_FP32)\n        ((float*)a)[i] = x;",
     "    if (lp == ORACLE_FP32)\n        ((float*)a)[i] = oracle_f16_to_f32(oracle_f32_to_f16(x));"),
]


def _build_and_run(tmp, name, old, new):
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, (name, src.count(old))
    d = os.path.join(tmp, name.replace(" ", "_").replace("/", "_"))
    os.makedirs(d, exist_ok=True)
    c = os.path.join(d, "zero_oracle.c")
    with open(c, "w", encoding="utf-8") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(d, "liboracle.so")
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    from build import CFLAGS  # the oracle's own flags
    subprocess.run(["gcc", *CFLAGS, "-o", lib, c, "-lm"], check=True)
    env = dict(os.environ, ZERO_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    return name, r.returncode


def test_every_mutation_is_caught(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda m: _build_and_run(str(tmp_path), *m), MUTATIONS))
    survivors = [name for name, rc in results if rc == 0]
    assert not survivors, f"mutations not caught by any pin: {survivors}"
    assert all(rc == 1 for _, rc in results), results   # failures, not errors
