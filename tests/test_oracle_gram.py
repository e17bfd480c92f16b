"""Pins for the Gram step and the trace normalisation (modded-nanogpt anvil.py, `anvil_cascade`:
the first Gram on the unnormalised X and its trace)."""
from fractions import Fraction

import numpy as np
import torch

from oracle import anvil_oracle as O


def _bf16_values(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


def _torch_round(x64: float) -> float:
    """Exact value -> fp32 (nearest) -> bf16 (nearest), with numpy/torch as the rounding witness."""
    return float(torch.tensor(np.float32(x64)).to(torch.bfloat16).to(torch.float32))


def test_gram_against_exact_rationals():
    rng = np.random.default_rng(3)
    for (m, n) in [(5, 3), (3, 5), (4, 4), (7, 2), (2, 9)]:
        X = _bf16_values(rng, (m, n))
        tall = m > n
        A = O.gram(X[None], tall)[0]
        s = n if tall else m
        for i in range(s):
            for j in range(s):
                if tall:
                    exact = sum(Fraction(float(X[k, i])) * Fraction(float(X[k, j])) for k in range(m))
                else:
                    exact = sum(Fraction(float(X[i, k])) * Fraction(float(X[j, k])) for k in range(n))
                # bf16 products and short sums are exact in fp64, so float(exact) is exact too
                assert A[i, j] == _torch_round(float(exact)), (m, n, i, j)


def test_gram_is_symmetric_and_matches_fp32_library_product():
    rng = np.random.default_rng(4)
    X = _bf16_values(rng, (3, 96, 40))
    for tall, Xi in ((True, X), (False, np.swapaxes(X, 1, 2).copy())):
        A = O.gram(Xi, tall)
        assert np.array_equal(A, np.swapaxes(A, 1, 2))
        t = torch.from_numpy(Xi)
        ref = (t.mT @ t if tall else t @ t.mT).to(torch.bfloat16).to(torch.float32).numpy()
        ulp = np.abs(A - ref) / np.maximum(np.abs(ref), 1e-30)
        assert np.all(ulp <= 2 ** -7 + 1e-9)           # at most one bf16 ulp apart
        assert np.mean(A == ref) > 0.97


def test_trace_identity():
    """trace(R(G(X))) = ||X||_F^2 up to one bf16 rounding per diagonal entry (relative 2^-9) and
    the fp32 summation."""
    rng = np.random.default_rng(5)
    for shape in [(4, 64, 24), (4, 24, 64), (2, 50, 50)]:
        X = _bf16_values(rng, shape, 3.0)
        tall = shape[1] > shape[2]
        A = O.gram(X, tall)
        tr, d = O.trace_scale(A)
        fro2 = np.sum(X.astype(np.float64) ** 2, axis=(1, 2))
        assert np.all(np.abs(tr[:, 0, 0] - fro2) <= (2 ** -9 + 1e-6) * fro2)
        want_d = np.sqrt(fro2) * 1.05 + 1e-6
        np.testing.assert_allclose(d[:, 0, 0], want_d, rtol=2e-3)


def test_normalised_spectrum_below_one():
    """After dividing by d, every singular value is below 1/1.05 (the margin's purpose)."""
    rng = np.random.default_rng(6)
    X = _bf16_values(rng, (3, 40, 24))
    A = O.gram(X, True)
    _, d = O.trace_scale(A)
    Xn, An = O.normalize(X, A, d)
    s = np.linalg.svd(Xn.astype(np.float64), compute_uv=False)
    assert s.max() <= 1 / 1.05 * (1 + 2 ** -7)
    # A / d^2 is (up to bf16 rounding) the Gram of X / d
    G2 = np.matmul(np.swapaxes(Xn, 1, 2).astype(np.float64), Xn)
    assert np.max(np.abs(An - G2)) <= 0.02 * np.max(np.abs(G2))


def test_zero_input_gives_eps_scale():
    X = np.zeros((1, 16, 8), np.float32)
    A = O.gram(X, True)
    tr, d = O.trace_scale(A)
    assert tr[0, 0, 0] == 0.0
    assert d[0, 0, 0] == np.float32(1e-6)
