"""Per-stage parity of the HIP kernels against the oracle, through the C ABI stage entry points.

Shapes span several 128-wide tiles with ragged edges, both orientations, the square case and the
split threshold; the last two are stacks of small wide matrices whose 32x32 Gram and polynomial
tiles would outnumber the CUs, so they take 64x64 tiles (the Gram with its 256-k groups on
separate sets of waves: two groups with a ragged last slab, and three).  The 44-matrix stack's
Gram (264 tiles, 132 diagonal) gives the CU-sharing workgroup slots to its diagonal tiles."""
import numpy as np
import pytest

from oracle import anvil_oracle as O
from tests.helpers import (assert_gemm_close, bf16_bits_of, from_gpu, oracle_normalised_pair,
                           to_gpu_bf16, to_gpu_f32)

pytestmark = pytest.mark.gpu

SHAPES = [(3, 200, 328), (3, 392, 136), (2, 264, 264), (2, 1096, 136), (2, 136, 1096),
          (1, 8, 8), (2, 8, 72), (2, 72, 8), (1, 256, 768), (1, 768, 256), (10, 200, 328),
          (12, 256, 768), (44, 392, 264)]


@pytest.mark.parametrize("g,m,n", SHAPES)
@pytest.mark.parametrize("fast_weight", [1.0, 0.4385])
def test_momentum_bit_exact(gpu_lib, g, m, n, fast_weight):
    rng = np.random.default_rng(g * 1000 + m + n)
    G = rng.standard_normal((g, m, n)).astype(np.float32)
    V = rng.standard_normal((2, g, m, n)).astype(np.float32)
    v_want, y = O.momentum_step(G, V, 0.95, 0.85, fast_weight)
    x_want = O.bf16_bits(y)
    Gd, Vd = to_gpu_f32(G), to_gpu_f32(V)
    x = gpu_lib.anvil_momentum(Gd, Vd, 0.95, 0.85, fast_weight)
    assert np.array_equal(from_gpu(Vd).view(np.uint32), v_want.view(np.uint32))
    assert np.array_equal(bf16_bits_of(x), x_want)
    assert np.array_equal(from_gpu(Gd), G)      # grad is read only


@pytest.mark.parametrize("g,m,n", SHAPES)
def test_gram_and_trace(gpu_lib, g, m, n):
    rng = np.random.default_rng(7 + m * n)
    X = O.R(rng.standard_normal((g, m, n)).astype(np.float32) * 2.0)
    tall = m > n
    want = O.gram(X, tall)
    a, parts = gpu_lib.anvil_gram(to_gpu_bf16(X), want_trace=True)
    got = from_gpu(a)
    assert np.array_equal(got, np.swapaxes(got, 1, 2)), "Gram must be stored exactly symmetric"
    assert_gemm_close(got, want, "gram")
    # the partials add up to the trace of the stored bf16 diagonal
    p = from_gpu(parts).astype(np.float64)
    diag = np.diagonal(got, axis1=1, axis2=2).astype(np.float64)
    np.testing.assert_allclose(p.sum(axis=1), diag.sum(axis=1), rtol=2e-5)
    tr_want, _ = O.trace_scale(want)
    np.testing.assert_allclose(p.sum(axis=1), tr_want[:, 0, 0], rtol=1e-4)


@pytest.mark.parametrize("g,m,n", SHAPES)
def test_normalize_bit_exact(gpu_lib, g, m, n):
    rng = np.random.default_rng(11 + m + 3 * n)
    X = O.R(rng.standard_normal((g, m, n)).astype(np.float32))
    Xd = to_gpu_bf16(X)
    a, parts = gpu_lib.anvil_gram(Xd, want_trace=True)
    A = from_gpu(a)
    P = from_gpu(parts)
    d = from_gpu(gpu_lib.anvil_normalize(Xd, a, parts))
    # d from the same partials, summed in slot order in fp32
    tr = np.zeros(g, np.float32)
    for j in range(P.shape[1]):
        tr = (tr + P[:, j]).astype(np.float32)
    d_want = (np.sqrt(tr) * np.float32(1.05)).astype(np.float32) + np.float32(1e-6)
    assert np.array_equal(d.view(np.uint32), d_want.astype(np.float32).view(np.uint32))
    Xn, An = O.normalize(X, A, d_want[:, None, None])
    assert np.array_equal(from_gpu(Xd), Xn)
    assert np.array_equal(from_gpu(a), An)


@pytest.mark.parametrize("g,m,n", SHAPES)
def test_poly(gpu_lib, g, m, n):
    rng = np.random.default_rng(13 + m)
    _, A = oracle_normalised_pair(rng, g, m, n)
    Ad = to_gpu_bf16(A)
    for k in (0, 3, 5):
        _, b, c = O.ANVIL_MAPS[k]
        got = from_gpu(gpu_lib.anvil_poly(Ad, b, c))
        assert np.array_equal(got, np.swapaxes(got, 1, 2))
        assert_gemm_close(got, O.poly(A, b, c), f"poly map {k}")


@pytest.mark.parametrize("g,m,n", SHAPES)
@pytest.mark.parametrize("split", [False, True])
def test_apply(gpu_lib, g, m, n, split):
    rng = np.random.default_rng(17 + n)
    X, A = oracle_normalised_pair(rng, g, m, n)
    a, b, c = O.ANVIL_MAPS[1]
    B = O.poly(A, b, c)
    got = from_gpu(gpu_lib.anvil_apply(to_gpu_bf16(X), to_gpu_bf16(B), a, split))
    assert_gemm_close(got, O.apply(X, B, a, m > n, split), f"apply split={split}")


def test_apply_split_golden(gpu_lib):
    """The hand-worked rounding case (tests/golden/rounding_points.json), padded to the minimum
    supported 8x8 with zeros: split and fused roundings must differ exactly as derived."""
    import json, os
    c = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rounding_points.json")))["apply_tall"]
    # tall 16x8 X with the worked value in [0, 0]; B = diag(1 + 2^-7, 0, ...)
    X = np.zeros((1, 16, 8), np.float32)
    X[0, 0, 0] = c["X"][0][0]
    B = np.zeros((1, 8, 8), np.float32)
    B[0, 0, 0] = c["B"][0][0]
    for split, key in ((True, "split"), (False, "fused")):
        got = from_gpu(gpu_lib.anvil_apply(to_gpu_bf16(X), to_gpu_bf16(B), c["a"], split))
        assert got[0, 0, 0] == c[key][0][0], (split, got[0, 0, 0])
        assert np.all(got[0].ravel()[1:] == 0)
