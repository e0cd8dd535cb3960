"""Pins of the oracle's own 2-byte converters against library routines:
numpy's IEEE binary16 conversion and torch's CPU bfloat16 conversion, both
round-to-nearest-even.  fp16 params/grads are the pages' 2-byte formats
("AI论文陪读·ZeRO" section 01 memory breakdown)."""
import numpy as np
import pytest
import torch

FP16, BF16 = 1, 2


def _same_bits_or_both_nan(a_bits, b_bits, nan_mask_a, nan_mask_b):
    assert np.array_equal(nan_mask_a, nan_mask_b)
    keep = ~nan_mask_a
    bad = np.nonzero(a_bits[keep] != b_bits[keep])[0]
    assert bad.size == 0, (a_bits[keep][bad[:5]], b_bits[keep][bad[:5]])


def test_f16_to_f32_exhaustive(oracle):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.lp_to_f32(FP16, h)
    ref = h.view(np.float16).astype(np.float32)
    _same_bits_or_both_nan(got.view(np.uint32), ref.view(np.uint32), np.isnan(got), np.isnan(ref))


def test_bf16_to_f32_exhaustive(oracle):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.lp_to_f32(BF16, b)
    ref = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    _same_bits_or_both_nan(got.view(np.uint32), ref.view(np.uint32), np.isnan(got), np.isnan(ref))


def _probe_floats(rng, lp):
    """Every finite 2-byte value, its neighbours in fp32 and the exact midpoints
    between consecutive 2-byte values (the ties), their fp32 neighbours, plus
    random fp32 bit patterns and the special values."""
    all16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if lp == FP16:
        vals = all16.view(np.float16).astype(np.float64)
    else:
        with np.errstate(invalid="ignore"):       # signalling-NaN patterns widen quietly
            vals = (all16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    vals = vals[np.isfinite(vals)]
    vals = np.unique(vals)
    mids = (vals[:-1] + vals[1:]) / 2.0        # exact in float64
    base = np.concatenate([vals, mids]).astype(np.float32)
    bits = base.view(np.uint32)
    near = np.concatenate([bits, bits + 1, bits - 1]).view(np.float32)
    rnd = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65519.996, 65520.0,
                        -65520.0, 2.0**-24, 2.0**-25, -(2.0**-25), 2.0**-25 * 1.5,
                        2.0**-14, 2.0**-14 - 2.0**-25, 3.3895314e38, 3.4028235e38],
                       dtype=np.float32)
    return np.concatenate([near, rnd, special])


def test_f32_to_f16_against_numpy(oracle):
    x = _probe_floats(np.random.default_rng(1), FP16)
    got = oracle.f32_to_lp(FP16, x)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    _same_bits_or_both_nan(got, ref, np.isnan(x), np.isnan(x))
    # NaN in, NaN out
    g = got[np.isnan(x)]
    assert np.all((g & 0x7C00) == 0x7C00) and np.all((g & 0x3FF) != 0)


def test_f32_to_bf16_against_torch(oracle):
    x = _probe_floats(np.random.default_rng(2), BF16)
    got = oracle.f32_to_lp(BF16, x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _same_bits_or_both_nan(got, ref, np.isnan(x), np.isnan(x))
    g = got[np.isnan(x)]
    assert np.all((g & 0x7F80) == 0x7F80) and np.all((g & 0x7F) != 0)


@pytest.mark.parametrize("v,expect", [(65519.0, 0x7BFF), (65520.0, 0x7C00), (-65520.0, 0xFC00),
                                      (65504.0, 0x7BFF), (1.0, 0x3C00), (-0.0, 0x8000)])
def test_f16_overflow_threshold(oracle, v, expect):
    assert int(oracle.f32_to_lp(FP16, np.array([v], np.float32))[0]) == expect
