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

import pytest

from zero_dp_sharded_amd import build


@pytest.fixture(scope="module")
def asm():
    return build.device_asm("zero_kernels.hip")


def test_kernels_have_no_fused_narrowing_or_packed_fp32(asm):
    body = [ln for ln in asm.splitlines() if ln.startswith("\t") and not ln.startswith("\t.")]
    assert len(body) > 1000
    bad = [ln.strip() for ln in body
           if re.match(r"\s*v_(fma|mad)_mix", ln) or re.match(r"\s*v_pk_(add|mul|fma)_f32", ln)]
    assert bad == [], bad[:8]
    # the fp16 narrowing is a plain conversion
    assert any(re.match(r"\s*v_cvt_(pk_)?f16_f32", ln) for ln in body)


def test_shift_reduce_loads_the_word_past_its_runs_as_measured(asm):
    """In every streaming (nontemporal) shift reduce, lane 63's word past its
    runs goes out, for 2-byte data, before that batch's contribution runs and
    without the nontemporal hint (the next workgroup of the XCD then finds the
    line in L2), and for fp32 after them, nontemporal (issued first it made
    every wave wait for it).  The sequence of 16-byte loads shows it: plain
    loads (c) then nontemporal ones (N) per batch for 2-byte data, all N for
    fp32.  (Kernels that also copy the step's state snapshot, with plain
    16-byte loads at their end, are left out.)"""
    names = re.findall(r"^(_Z\S*reduce_shift_kernelILi(\d)ELi(\d+)ELi(\d)ELi(\d+)ELi0ELi1E\S*):",
                       asm, re.M)
    assert len(names) >= 8
    for name, lp, rt, u, bs in names:
        body = asm[asm.index(name + ":"):]
        body = body[:body.index(".Lfunc_end")]
        seq = "".join("N" if " nt" in ln else "c" for ln in body.splitlines()
                      if "global_load_dwordx4" in ln)
        if lp == "3":
            assert re.fullmatch(r"N+", seq), (name, seq)
        else:
            assert re.fullmatch(r"(c{1,4}N+)+", seq), (name, seq)
