"""Pins for the oracle's lerp and blend (modded-nanogpt anvil.py, `anvil_cascade` momentum block:
both rails and the Nesterov lookahead are in-place `lerp_` calls of torch; the blend of the rails
is a weighted sum of two tensor products; `_rail_equalizer` updates the lane energies with
`lerp_` too).

Witnesses: torch's own CPU lerp (the library routine the page calls) for the lerp, bit for bit,
with the weights the page uses as Python floats and as 0-D fp32 tensors; exact rational
arithmetic for the fused multiply-add underneath; torch's eager tensor expression for the blend.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import anvil_oracle as O

F32 = np.float32

# the weights the page hands to lerp_: 1 - 0.85f (fast rail), 1 - 0.98 (slow rail, a host
# double), the momentum 0.95 (Nesterov), 1 - beta2 for beta2 = 0.95 (lane energies); and the
# boundary values of the library's two branches
WEIGHTS = [float(F32(1.0) - F32(0.85)), 1.0 - 0.98, 0.95, 1.0 - 0.95, 0.5, 0.49999997, 0.0, 1.0,
           0.4385]


def _inputs(n, seed):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal(n).astype(F32)
    e = (rng.standard_normal(n) * np.exp(rng.standard_normal(n))).astype(F32)
    # edge values: zeros of both signs, equal ends, subnormals, large magnitudes
    edge = np.array([0.0, -0.0, 1.0, -1.0, 1e-40, -1e-40, 3e38, -3e38, 1e-30, 65504.0],
                    dtype=F32)
    s[:edge.size] = edge
    e[:edge.size] = edge[::-1]
    s[edge.size:2 * edge.size] = edge
    e[edge.size:2 * edge.size] = edge
    return s, e


@pytest.mark.parametrize("w", WEIGHTS)
@pytest.mark.parametrize("as_tensor", [False, True])
def test_lerp_equals_torch_cpu(w, as_tensor):
    torch = pytest.importorskip("torch")
    s, e = _inputs(300_007, seed=int(w * 1e6) + 3)   # not a multiple of any vector width
    weight = torch.tensor(F32(w)) if as_tensor else float(F32(w))
    with np.errstate(over="ignore", invalid="ignore"):
        want = torch.from_numpy(s).lerp(torch.from_numpy(e), weight).numpy()
        got = O.lerp(s, e, F32(w))
    same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
    assert same.all(), f"weight {w}: {np.count_nonzero(~same)} of {s.size} values differ"


def test_lerp_differs_from_unfused_form():
    """The lerp is not the separately rounded start + w*(end - start): at the Nesterov weight the
    two differ in a large share of fp32 values, so a plausible simplification fails the pin."""
    s, e = _inputs(100_000, seed=5)
    w = F32(0.95)
    unfused = s + w * (e - s)
    assert np.mean(O.lerp(s, e, w) != unfused) > 0.2


def _fma_exact(a, b, c):
    """fp32 value of a*b + c, rounded once from the exact rational value (ties to even)."""
    x = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    lo = F32(float(x))                      # a neighbour of x (double rounding is only a guess)
    cands = {lo, np.nextafter(lo, F32(np.inf)), np.nextafter(lo, F32(-np.inf))}
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - x),
                                     int(np.asarray(v, F32).view(np.uint32)) & 1))
    return best


def test_fma32_equals_exact_rational():
    rng = np.random.default_rng(7)
    a = rng.standard_normal(3000).astype(F32)
    b = rng.standard_normal(3000).astype(F32)
    c = (rng.standard_normal(3000) * 10.0 ** rng.integers(-8, 8, 3000)).astype(F32)
    # engineered near-midpoint cases: c large, a*b a tiny nudge around half an ulp of c
    c[:500] = F32(1.0) + np.arange(500, dtype=F32) * F32(2.0 ** -23)
    a[:500] = F32(2.0 ** -24)
    b[:500] = (F32(1.0) + rng.integers(-3, 4, 500).astype(F32) * F32(2.0 ** -23))
    # exact sums one 2^-70 off a midpoint: the fp64 sum lands on the midpoint and only the
    # two-sum error says which way to round (below for 1 - 2^-23, above for 1 + 2^-23)
    c[500:700] = F32(1.0) + np.arange(200, dtype=F32) * F32(2.0 ** -23)
    a[500:700] = F32(2.0 ** -24) * F32(1.0 + 2.0 ** -23)
    b[500:600] = F32(1.0 - 2.0 ** -23)
    b[600:700] = F32(1.0 + 2.0 ** -23)
    c[700:800] = -c[500:600]
    a[700:800] = a[500:600]
    b[700:800] = -b[500:600]
    got = O.fma32(a, b, c)
    naive = (a.astype(np.float64) * b + c).astype(F32)
    assert np.count_nonzero(got[500:800] != naive[500:800]) >= 100   # the careful path matters
    for i in range(a.size):
        want = _fma_exact(a[i], b[i], c[i])
        assert got[i].view(np.uint32) == F32(want).view(np.uint32), (i, a[i], b[i], c[i])


def test_blend_equals_torch_eager():
    """blend = w * v0 + (1 - w) * v1 with w a 0-D fp32 tensor: three separately rounded fp32
    tensor operations in torch's eager semantics."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    g = rng.standard_normal((1, 64, 48)).astype(F32)
    v = rng.standard_normal((2, 1, 64, 48)).astype(F32)
    w = torch.tensor(F32(0.4385))
    v_t = torch.from_numpy(v.copy())
    g_t = torch.from_numpy(g)
    v_t[0].lerp_(g_t, 1 - torch.tensor(F32(0.85)))
    v_t[1].lerp_(g_t, 1 - 0.98)
    blend = w * v_t[0] + (1 - w) * v_t[1]
    y = g_t.clone().lerp_(blend, torch.tensor(F32(0.95)))
    v_or, y_or = O.momentum_step(g, v, 0.95, 0.85, 0.4385)
    assert np.array_equal(v_or.view(np.uint32), v_t.numpy().view(np.uint32))
    assert np.array_equal(y_or.view(np.uint32), y.numpy().view(np.uint32))
