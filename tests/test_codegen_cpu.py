"""What the compiler emits for the gfx950 kernels, checked on the CPU.

The method rounds each reduced gradient to fp32 and then to the storage
format (two roundings).  AMDGPU has mixed-precision fused instructions
(v_fma_mix*, v_mad_mix*) that take a multiply straight to fp16 with one
rounding; a product that lands on an fp16 rounding tie then differs in the
last bit.  hipcc emitted such a fusion for the element-wise reduce until the
kernels pinned the fp32 value, so this test keeps every mixed-precision fused
instruction out of the kernels, and likewise the packed-fp32 arithmetic the
build disables."""
import re

from zero_dp_sharded_amd import build


def test_kernels_have_no_fused_narrowing_or_packed_fp32():
    asm = build.device_asm("zero_kernels.hip")
    body = [ln for ln in asm.splitlines() if ln.startswith("\t") and not ln.startswith("\t.")]
    assert len(body) > 1000
    bad = [ln.strip() for ln in body
           if re.match(r"\s*v_(fma|mad)_mix", ln) or re.match(r"\s*v_pk_(add|mul|fma)_f32", ln)]
    assert bad == [], bad[:8]
    # the fp16 narrowing is a plain conversion
    assert any(re.match(r"\s*v_cvt_(pk_)?f16_f32", ln) for ln in body)
