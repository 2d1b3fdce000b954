"""The error bound of the split bf16 products in the row kernels (CPU).

The kernels that multiply bf16 block rows on the bf16 matrix-core
instruction split every fp32 input x into hi = bf16(x) and lo = bf16(x - hi),
both rounded to nearest even, and take C x as C hi + C lo.  These checks pin
the two facts the kernels rely on, with torch's bf16 rounding (nearest even)
standing in for the device conversion: x - hi is exact in fp32, and
|x - hi - lo| <= 2^-16 |x| (bf16 keeps 8 significant bits, so each rounding
is within 2^-8 relative).  A truncating split, or a lo rounded from the
wrong difference, breaks the bound.
"""
import numpy as np
import torch


def _split(x: torch.Tensor):
    hi = x.to(torch.bfloat16).float()
    r = x - hi
    lo = r.to(torch.bfloat16).float()
    return hi, r, lo


def test_residual_is_exact_and_split_within_2_pow_minus_16():
    gen = np.random.default_rng(7)
    # every exponent the rows can reach, both signs, plus exact bf16 values
    mant = gen.uniform(1.0, 2.0, 200000)
    expo = gen.integers(-60, 60, mant.size)
    sign = gen.choice([-1.0, 1.0], mant.size)
    v = np.concatenate([sign * np.ldexp(mant, expo), [0.0, 1.0, -3.0, 1.0 + 2.0 ** -8, 1.0 + 2.0 ** -9]])
    x = torch.from_numpy(v.astype(np.float32))
    hi, r, lo = _split(x)
    x64, hi64 = x.double(), hi.double()
    assert torch.equal(r.double(), x64 - hi64)                      # exact residual
    err = (x64 - hi64 - lo.double()).abs()
    assert bool((err <= 2.0 ** -16 * x64.abs()).all())
    # the bound is reached within a factor of two, so it is not loose
    assert float((err / x64.abs().clamp_min(1e-300)).max()) > 2.0 ** -18


def test_bf16_inputs_have_zero_lo():
    # the first forward stage reads bf16 rows (times +-1): lo is 0 there
    x = torch.randn(4096).to(torch.bfloat16).float()
    hi, r, lo = _split(x)
    assert torch.equal(hi, x) and bool((lo == 0).all())


def test_truncating_split_breaks_the_bound():
    # a plausible mistake: hi by truncation and lo by truncation of the residual
    gen = np.random.default_rng(3)
    x = torch.from_numpy(gen.standard_normal(100000).astype(np.float32))
    hi = (x.view(torch.int32) & ~0xFFFF).view(torch.float32)
    lo = ((x - hi).view(torch.int32) & ~0xFFFF).view(torch.float32)
    err = (x.double() - hi.double() - lo.double()).abs()
    assert not bool((err <= 2.0 ** -16 * x.double().abs()).all())
