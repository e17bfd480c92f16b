"""Shared helpers of the GPU parity tests: moving oracle-side numpy arrays to and from the GPU and
the comparison rules.  No arithmetic of the method lives here."""
import numpy as np

from oracle import anvil_oracle as O


def to_gpu_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_gpu_bf16(a):
    """fp32 array of bf16-representable values -> GPU bf16 tensor (exact)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()


def from_gpu(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def bf16_bits_of(t):
    """GPU bf16 tensor -> numpy uint16 bit patterns."""
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def rel_fro(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


# The parity bars of the bf16 update and the fp32 rails.  The update bar is the relative Frobenius
# error per matrix; on inputs whose normalised singular values lie far below the maps' window the
# bf16 rounding noise is amplified and two correct accumulation orders of the oracle itself drift
# apart, so there the bar is FLOOR_FACTOR times that measured drift, and an input whose drift
# would put the bar above FLOOR_CAP fails outright (it is too ill-conditioned to tell a correct
# implementation from a wrong one).
OUT_TOL = 1e-2
RAIL_TOL = 1e-6
FLOOR_FACTOR = 1.5
FLOOR_CAP = 2e-2


def update_error(got, want, allow_nonfinite=False):
    """Relative Frobenius error of one update matrix against the oracle's.

    Every entry the oracle has finite must be finite on the GPU and vice versa (a NaN or Inf can
    never hide behind a comparison that is False for NaN).  Unless allow_nonfinite, the oracle's
    matrix must be finite throughout, so a diverged oracle cannot pass a comparison vacuously."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    fin = np.isfinite(want)
    if not allow_nonfinite:
        assert fin.all(), f"the oracle's matrix has {np.count_nonzero(~fin)} non-finite entries"
    bad = np.isfinite(got) != fin
    assert not bad.any(), f"{np.count_nonzero(bad)} entries finite on one side only"
    if not fin.any():
        return 0.0
    r = rel_fro(got[fin], want[fin])
    assert np.isfinite(r), r
    return r


def assert_update_close(got, want, floor_fn=None, what="update"):
    """The parity bar on one matrix of the bf16 update.  floor_fn, when given, returns the relative
    Frobenius drift between the oracle's fp32- and fp64-accumulation variants on the same input;
    it is only evaluated when the error exceeds OUT_TOL.  Returns (error, bar used, floor or None)."""
    r = update_error(got, want)
    if r <= OUT_TOL:
        return r, OUT_TOL, None
    assert floor_fn is not None, f"{what}: relative Frobenius {r:.3e} above {OUT_TOL:.0e}"
    floor = float(floor_fn())
    assert np.isfinite(floor), f"{what}: noise floor {floor}"
    tol = max(OUT_TOL, FLOOR_FACTOR * floor)
    assert tol <= FLOOR_CAP, (f"{what}: noise floor {floor:.3e} puts the bar at {tol:.3e}, above "
                              f"the cap {FLOOR_CAP:.0e}")
    assert r <= tol, f"{what}: relative Frobenius {r:.3e} above {tol:.3e} (floor {floor:.3e})"
    return r, tol, floor


def assert_rails_close(got, want, what="rails"):
    """fp32 rails within RAIL_TOL relative, element by element, with non-finite entries in the
    same places (NaN-safe: the error of a NaN entry is never compared)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: non-finite entries differ"
    err = np.abs(got[fin] - want[fin]) / np.maximum(np.abs(want[fin]), 1e-30)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= RAIL_TOL, f"{what}: relative error {worst:.2e}"
    return worst


def assert_sigma_band(out, what="update", band=0.3):
    """Every singular value of one output matrix within `band` of 1."""
    sv = np.linalg.svd(np.asarray(out, dtype=np.float64), compute_uv=False)
    assert np.all(np.isfinite(sv)), what
    assert np.all(np.abs(sv - 1.0) <= band), f"{what}: singular values in [{sv.min():.3f}, {sv.max():.3f}]"
    return float(sv.min()), float(sv.max())


def well_conditioned(x_bf16, lo=0.002):
    """Every singular value of the normalised input (sigma / (1.05 ||X||_F)) at least lo: inside
    the window of the six maps, where the composite map lands within 0.3 of 1."""
    X = np.asarray(x_bf16, dtype=np.float64)
    sv = np.linalg.svd(X, compute_uv=False)
    d = np.sqrt(np.sum(X * X)) * 1.05
    return bool(d > 0 and sv.min() / d >= lo)


def assert_gemm_close(got, want, what, equal_frac=0.9):
    """A bf16 GEMM output against the oracle's: the two differ only in fp32 accumulation order, so
    the relative Frobenius error stays at bf16 rounding level, most entries are identical and no
    entry is off by more than a couple of bf16 ulps of the matrix scale."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, what
    assert np.all(np.isfinite(got)), what
    for i in range(got.shape[0]):
        r = rel_fro(got[i], want[i])
        assert r <= 2e-3, f"{what}[{i}]: relative Frobenius {r:.3e}"
        scale = np.max(np.abs(want[i]))
        worst = np.max(np.abs(got[i] - want[i]))
        assert worst <= 2 ** -6 * scale, f"{what}[{i}]: max abs diff {worst:.3e} vs scale {scale:.3e}"
    frac = float(np.mean(got == want))
    assert frac >= equal_frac, f"{what}: only {frac:.3f} of entries identical"


def oracle_normalised_pair(rng, g, m, n):
    """A bf16 X normalised the oracle's way, and its bf16 Gram (inputs for poly/apply tests)."""
    X = O.R(rng.standard_normal((g, m, n)).astype(np.float32))
    tall = m > n
    A = O.gram(X, tall)
    _, d = O.trace_scale(A)
    return O.normalize(X, A, d)


def sigma_classes(s):
    """Counts (c1, c2, c3) of the values 1, 1/2, 1/4 on the diagonal of the large matrix and a
    number r of filler values 16 for a 64x64 diagonal stand-in, with equal traces:
    c1 + c2/4 + c3/16 = 1 + 1/4 + 1/16 + 256 r.  Every square and partial sum is exact in fp32,
    so both traces (and d) are the same whatever the summation order.  The most even split."""
    best = None
    for r in range(1, 62):
        rhs = 21 + 4096 * r - s          # 15 c1 + 3 c2 = 16 * trace - s
        if rhs < 0 or rhs % 3:
            continue
        k = rhs // 3                     # 5 c1 + c2 = k, c1 + c2 <= s
        for c1 in range(max(0, -(-(k - s) // 4)), k // 5 + 1):
            c2 = k - 5 * c1
            c3 = s - c1 - c2
            if c2 >= 0 and c3 >= 0 and (best is None or min(c1, c2, c3) > min(best[1])):
                best = (r, (c1, c2, c3))
    return best
