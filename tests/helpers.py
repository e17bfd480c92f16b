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
