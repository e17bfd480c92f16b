"""The GPU parity tests' comparison helpers must fail on a planted NaN or Inf, on a diverged oracle
and on an error above the bar, and pass a correct result.  Runs on the CPU: the "GPU" side here is
the oracle's own output with a mistake planted in it."""
import numpy as np
import pytest

from oracle import anvil_oracle as O
from tests.helpers import (FLOOR_CAP, OUT_TOL, assert_gemm_close, assert_rails_close,
                           assert_sigma_band, assert_update_close, update_error)


def _want():
    rng = np.random.default_rng(3)
    X = O.R(rng.standard_normal((1, 48, 32)).astype(np.float32))
    return O.cascade(X)[0]


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_planted_nonfinite_fails_update_check(bad):
    want = _want()
    got = want.copy()
    got[3, 5] = bad
    with pytest.raises(AssertionError):
        assert_update_close(got, want)
    with pytest.raises(AssertionError):
        assert_update_close(got, want, floor_fn=lambda: 0.01)
    with pytest.raises(AssertionError):
        update_error(got, want)


def test_all_nan_output_fails():
    want = _want()
    with pytest.raises(AssertionError):
        assert_update_close(np.full_like(want, np.nan), want, floor_fn=lambda: 0.0)


def test_diverged_oracle_fails_even_when_both_sides_agree():
    want = _want()
    want[0, 0] = np.nan
    with pytest.raises(AssertionError):
        assert_update_close(want.copy(), want)
    # only where non-finite entries are expected (NaN propagation) may they match
    assert update_error(want.copy(), want, allow_nonfinite=True) == 0.0


def test_bar_and_floor_cap():
    want = _want()
    noise = np.random.default_rng(4).standard_normal(want.shape)
    noise *= np.linalg.norm(want) / np.linalg.norm(noise)
    ok = want + 0.5 * OUT_TOL * noise
    r, tol, floor = assert_update_close(ok, want)
    assert r <= OUT_TOL and tol == OUT_TOL and floor is None
    over = want + 1.2 * OUT_TOL * noise
    with pytest.raises(AssertionError):
        assert_update_close(over, want)                        # no floor: the plain bar
    r, tol, floor = assert_update_close(over, want, floor_fn=lambda: 0.01)
    assert tol == pytest.approx(0.015)
    with pytest.raises(AssertionError):                        # floor too high: capped
        assert_update_close(over, want, floor_fn=lambda: FLOOR_CAP)
    with pytest.raises(AssertionError):                        # NaN floor
        assert_update_close(over, want, floor_fn=lambda: np.nan)


def test_rails_check_is_nan_safe():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((2, 1, 8, 8)).astype(np.float32)
    assert_rails_close(v.copy(), v)
    bad = v.copy()
    bad[1, 0, 2, 2] = np.nan
    with pytest.raises(AssertionError):
        assert_rails_close(bad, v)
    off = v.copy()
    off[0, 0, 0, 0] = np.nextafter(off[0, 0, 0, 0], np.float32(np.inf)) * np.float32(1 + 1e-5)
    with pytest.raises(AssertionError):
        assert_rails_close(off, v)


def test_gemm_check_is_nan_safe():
    rng = np.random.default_rng(6)
    A = O.R(rng.standard_normal((2, 16, 16)).astype(np.float32))
    assert_gemm_close(A.copy(), A, "gram")
    bad = A.copy()
    bad[1, 3, 3] = np.nan
    with pytest.raises(AssertionError):
        assert_gemm_close(bad, A, "gram")
    want_nan = A.copy()
    want_nan[0, 0, 0] = np.nan
    with pytest.raises(AssertionError):
        assert_gemm_close(want_nan.copy(), want_nan, "gram")


def test_sigma_band_check():
    q, _ = np.linalg.qr(np.random.default_rng(7).standard_normal((32, 16)))
    assert_sigma_band(q)
    with pytest.raises(AssertionError):
        assert_sigma_band(q * 1.4)
    bad = q.copy()
    bad[0, 0] = np.nan
    with pytest.raises((AssertionError, np.linalg.LinAlgError)):
        assert_sigma_band(bad)
