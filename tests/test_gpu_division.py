"""Exhaustive checks of the short division sequences the quantizer kernels use
instead of the IEEE division ([Review] §2.2: the quantizer divides by the step;
[Review] §5.1 eq. (3): the activation is divided by s).  Bit-exact codes rest
on these sequences returning the correctly rounded quotient:

  rcp_rn(b)            v_rcp_f32 + one Newton step, claimed = RN(1/b) for
                       2^-126 <= b < 2^126 (the library divides elsewhere)
  div_rn_narrow(a,b,r) three operations, claimed = RN(a/b) when a has at most
                       8 significant bits (bf16 activations)
  div_rn(a,b,r)        five operations, RN(a/b) by Markstein's theorem
  chunk_codes          the int8 codes rne(RN(v/d)) of eight values from the
                       exact product v * RN(1/d), deferring to div_rn near
                       half-integers

The check kernels (libsqprobe.so, compiled from the same device functions)
decide correct rounding exactly from the fp64 residual a - b q, with no
division instruction; each check also runs a deliberately short form (the
bare estimate or product) that must fail, which shows the checker catches
wrong roundings.  Every kernel is a bounded loop over computed values."""
import numpy as np
import pytest
import torch

from w8a8_int8_gemm_colwise_amd import probes
from sqcase import dev, say

pytestmark = pytest.mark.gpu

LO, HI = 0x00800000, 0x7E800000  # [2^-126, 2^126): where rcp_rn takes the short form


def test_rcp_rn_every_float_in_range():
    d = dev()
    say(f"[case] rcp_rn over every float in [2^-126, 2^126): {HI - LO} values")
    bad, ieee, first = probes.check_rcp(d, LO, HI)
    assert (bad, ieee, first) == (0, 0, None)
    # negative control: the bare hardware estimate is not always RN(1/b)
    bad, ieee, first = probes.check_rcp(d, 0x3F800000, 0x40000000, raw=True)
    say(f"  bare v_rcp_f32 on [1, 2): {bad} not correctly rounded")
    assert bad > 0 and ieee == bad and first is not None


def test_div_rn_narrow_every_bf16_by_fp32_significand():
    d = dev()
    say("[case] div_rn_narrow: 128 bf16 x 2^23 fp32 significands")
    assert probes.check_div_narrow(d) == (0, 0, None)
    bad, ieee, first = probes.check_div_narrow(d, raw=True)
    say(f"  bare product RN(a * RN(1/b)): {bad} of 2^30 not correctly rounded")
    assert bad > 0 and ieee == bad and first is not None


def test_div_rn_fp32_dividends():
    d = dev()
    say("[case] div_rn: 2^30 hashed fp32 significand pairs (every b significand 128 times)")
    assert probes.check_div(d, seed=20251203, count=1 << 30) == (0, 0, None)
    bad, _, _ = probes.check_div(d, seed=20251203, count=1 << 24, raw=True)
    assert bad > 0


@pytest.mark.parametrize("clamp", [False, True], ids=["row-step", "static"])
def test_chunk_codes_match_the_division(clamp):
    """The quantizers' code step (chunk_codes) takes rne of the exact product
    with RN(1/step) and defers to the division only where a half-integer lies
    within that product's error bound; its codes must equal those of the IEEE
    quotient on 2^27 values, half of them exact ties or within 4 ulps of one."""
    d = dev()
    say(f"[case] chunk_codes clamp={clamp}: 2^24 hashed chunks of 8 values")
    assert probes.check_codes(d, seed=20251204, count=1 << 24, clamp=clamp) == (0, 0, None)
    bad, _, first = probes.check_codes(d, seed=20251204, count=1 << 20, clamp=clamp, raw=True)
    say(f"  short form without the fallback: {bad} of 2^23 codes wrong")
    assert bad > 0 and first is not None


def test_compiler_division_is_the_ieee_division():
    """The reference the kernels' divisions fall back to (and the checks above
    compare with) is the correctly rounded fp32 quotient: the GPU's a / b equals
    numpy's IEEE division on 4M random pairs spanning the exponent range, plus
    the quantizer's own operand shapes (steps RN(m/127), the factors' range)."""
    d = dev()
    rng = np.random.default_rng(5)
    n = 1 << 22
    bits_a = rng.integers(0x00800000, 0x7F000000, n, dtype=np.int64).astype(np.uint32)
    bits_b = rng.integers(0x00800000, 0x7F000000, n, dtype=np.int64).astype(np.uint32)
    a = bits_a.view(np.float32) * np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32)
    b = bits_b.view(np.float32)
    steps = (rng.uniform(1e-3, 200, 4096).astype(np.float32) / np.float32(127)).astype(np.float32)
    a = np.concatenate([a, rng.normal(0, 60, 4096).astype(np.float32)])
    b = np.concatenate([b, steps])
    with np.errstate(over="ignore", under="ignore"):
        want = a / b
    got = probes.div_ref(d, torch.from_numpy(a).to(d), torch.from_numpy(b).to(d)).cpu().numpy()
    ok = np.isfinite(want) & (np.abs(want) >= np.float32(2.0 ** -126))
    assert np.array_equal(got[ok].view(np.uint32), want[ok].view(np.uint32))
