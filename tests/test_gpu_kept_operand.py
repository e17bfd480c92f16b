"""Exact checks of the GEMM epilogues' own operand.

The polynomial's b*A and the apply's a*X do not come from memory: each wave keeps the MFMA
fragments of the k loop that hold its block's A or X (the P operand at k = j for the polynomial and
the tall apply, the Q operand at k = i for the wide apply) and turns them into the accumulators'
layout in its epilogue.  With the product term taken out (B = 0 for the apply, c = 0 for the
polynomial) the result is exactly the rounded epilogue term, so every element must equal the
oracle's bit for bit, and a single misplaced element fails.  The shapes cover both orientations,
ragged edges, the square case, blocks that lie past the matrix edge, and the tile configurations:
32x128, 128x128 and 128x256 apply tiles; 32x32, 64x64 and 128x128 polynomial tiles.
"""
import numpy as np
import pytest

from oracle import anvil_oracle as O
from tests.helpers import bf16_bits_of, oracle_normalised_pair, to_gpu_bf16

pytestmark = pytest.mark.gpu

SHAPES = [(3, 200, 328), (3, 392, 136), (2, 264, 264), (2, 1096, 136), (2, 136, 1096),
          (1, 8, 8), (2, 8, 72), (2, 72, 8), (1, 256, 768), (1, 768, 256), (12, 256, 768),
          (44, 392, 264), (8, 2816, 768), (6, 768, 2816)]


def _bits(x):
    return O.bf16_bits(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("g,m,n", SHAPES)
@pytest.mark.parametrize("split", [False, True])
def test_apply_epilogue_operand_exact(gpu_lib, g, m, n, split):
    rng = np.random.default_rng(101 + m + 7 * n)
    X, _ = oracle_normalised_pair(rng, g, m, n)
    assert np.all(X != 0), "the check needs nonzero X (the sign of a zero sum is not pinned)"
    s = min(m, n)
    B = np.zeros((g, s, s), np.float32)
    a = O.ANVIL_MAPS[2][0]
    got = bf16_bits_of(gpu_lib.anvil_apply(to_gpu_bf16(X), to_gpu_bf16(B), a, split))
    want = _bits(O.apply(X, B, a, m > n, split))
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} elements differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("g,m,n", SHAPES)
def test_poly_epilogue_operand_exact(gpu_lib, g, m, n):
    rng = np.random.default_rng(211 + m + 7 * n)
    _, A = oracle_normalised_pair(rng, g, m, n)
    assert np.all(A != 0), "the check needs nonzero A (the sign of a zero sum is not pinned)"
    b = O.ANVIL_MAPS[4][1]
    got = bf16_bits_of(gpu_lib.anvil_poly(to_gpu_bf16(A), b, 0.0))
    want = _bits(O.poly(A, b, 0.0))
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} elements differ, first at {bad[:3].tolist()}"
