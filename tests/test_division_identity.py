"""The normalisation kernel divides every bf16 value of X and of the Gram by one fp32 divisor per
matrix (d, and d*d).  It forms each quotient from the correctly rounded reciprocal r = 1/d as
q = x*r, then q + (x - q*d)*r with both steps fused multiply-adds, and keeps a plain division for
values outside [2^-100, 2^100] (of x or of q).  This checks on the CPU, with exactly rounded
emulation of each fp32 operation, that the guarded formula equals the correctly rounded quotient
x/d for every finite bf16 x and a spread of divisors, so the kernel's result is the division the
page writes (X / d, A / d**2), not an approximation of it."""
import numpy as np

from oracle.anvil_oracle import fma32

F32 = np.float32
LO, HI = F32(2.0 ** -100), F32(2.0 ** 100)


def _bf16_values():
    x = (np.arange(65536, dtype=np.uint32) << np.uint32(16)).view(F32)
    return x[np.isfinite(x)]


def _guarded_quotient(x, d):
    r = F32(1.0 / np.float64(d))                       # correctly rounded reciprocal
    with np.errstate(over="ignore"):
        q = (x * r).astype(F32)
    fast = (np.abs(x) >= LO) & (np.abs(x) <= HI) & (np.abs(q) >= LO) & (np.abs(q) <= HI)
    rem = fma32(-q, d, x)
    q2 = fma32(rem, r, q)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        slow = (x / d).astype(F32)
    return np.where(fast, q2, slow), fast


def test_guarded_reciprocal_division_is_correctly_rounded():
    x = _bf16_values()
    rng = np.random.default_rng(12)
    divisors = np.concatenate([
        (rng.random(150) * 10.0 ** rng.integers(-6, 7, 150)).astype(F32),
        np.array([1e-6, 1.0, 1.05, 2.0, 3.0, 0.7, 12345.678, 1e6], dtype=F32)])
    for d in divisors:
        for div in (F32(d), F32(F32(d) * F32(d))):
            with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
                want = (x.astype(np.float64) / np.float64(div)).astype(F32)   # innocuous double rounding
            got, fast = _guarded_quotient(x, div)
            same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
            assert same.all(), (float(div), x[~same][:4])
            assert fast.mean() > 0.5          # the fused path is the common one


def test_unguarded_formula_would_fail_near_the_normal_range_edge():
    """Without the guard the formula is wrong for tiny x (the remainder drops below the normal
    range): the guard is what makes it exact."""
    x = _bf16_values()
    d = F32(0.48999998)
    r = F32(1.0 / np.float64(d))
    with np.errstate(over="ignore"):
        q = (x * r).astype(F32)
    q2 = fma32(fma32(-q, d, x), r, q)
    with np.errstate(over="ignore"):
        want = (x.astype(np.float64) / np.float64(d)).astype(F32)
    tiny = (np.abs(x) > 0) & (np.abs(x) < F32(2.0 ** -120))
    assert np.any(q2[tiny].view(np.uint32) != want[tiny].view(np.uint32))
