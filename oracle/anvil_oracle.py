"""CPU oracle for the ANVIL bank step.  TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark may import this
module.  The product path (the HIP library and its Python binding) never calls it, and the two
share no code: this file restates the method from the source page in plain numpy.

What it computes (source: modded-nanogpt, `track_1_short/optim/anvil.py`, function
`anvil_cascade` and the module constants above it):

  1. twin-rail momentum in fp32: a fast and a slow lerp of each velocity rail toward the gradient,
     a weighted blend of the two rails, and a Nesterov lerp of the gradient toward the blend;
  2. a cast of the lookahead to bf16 (round to nearest, ties to even);
  3. the first Gram matrix of that bf16 matrix (X^T X when rows > cols, X X^T otherwise), whose
     bf16 diagonal sums to ||X||_F^2; the scale d = sqrt(trace) * 1.05 + 1e-6 then divides X
     and d^2 divides the Gram;
  4. six quintic maps: B = b*A + c*A@A, then X <- a*X + X@B (tall) or a*X + B@X (wide), with the
     Gram recomputed from the current X for every map after the first.

Precision model (the plainest reading of the page where it leaves the precision open):
  * elementwise steps are fp32 operations, each rounded separately (numpy float32 arithmetic),
    except the lerps: the page calls torch's `lerp_`, whose definition in the library takes the
    difference of the end points and then one fused multiply-add about the nearer end point
    (`lerp` below, pinned bit for bit against torch.lerp on the CPU);
  * every matrix product is taken in fp64 from the bf16 operands, rounded once to fp32 (the
    accumulator type of a bf16 GEMM), and only then rounded to bf16 where the page stores bf16;
  * the polynomial epilogue b*A + c*(A@A) and the apply epilogue a*X + P are fp32 before their one
    bf16 rounding; banks with more than 1024 rows round P to bf16 first (the page's two-kernel
    form, a bmm into a bf16 buffer followed by an in-place add of a*X).

`exact=True` replaces every rounding by the identity and runs in fp64; the spectral tests use it.
`acc="fp32"` accumulates the products in fp32 (library sgemm order) instead of fp64: a second,
equally valid accumulation order, used to measure the rounding-noise floor of an input (how far two
correct implementations of the same rounding points drift apart on it).

Pins (tests/test_oracle_*.py): bf16 rounding against torch's CPU cast over edge bit patterns;
the rails against the closed form of a constant-gradient EMA; the Gram against exact rational
arithmetic on tiny inputs and the trace identity; the cascade against the SVD closed form
U F(S/d) V^T; tall/wide transpose symmetry; the split rounding against a hand-worked case.
"""

from __future__ import annotations

import numpy as np

# Six (a, b, c) triples of the quintic maps p(s) = a s + b s^3 + c s^5, applied in this order
# (modded-nanogpt anvil.py, the module-level table of maps used by `anvil_cascade`).
ANVIL_MAPS = (
    (3.923798038567, -6.095026865488, 3.905234618423),
    (3.278126713798, -3.328923386476, 0.989127286973),
    (3.505298394150, -5.137358782410, 1.968325560615),
    (2.815058591845, -3.685181239622, 1.417196497642),
    (2.245503932403, -2.443826979899, 0.963091710461),
    (2.256537145403, -2.166840097229, 0.929501253245),
)

# Rail constants (same page, the twin-rail comment block and constants).
RAIL_FAST_BETA = 0.85
RAIL_SLOW_BETA = 0.98
RAIL_FAST_WEIGHT = 0.4385
RAIL_ENGAGE_STEP = 514

# Frobenius normalisation constants and the split-apply row threshold (same page).
FROBENIUS_MARGIN = 1.05
FROBENIUS_EPS = 1e-6
SPLIT_BADDBMM_MIN_ROWS = 1024

F32 = np.float32


# --------------------------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------------------------

def bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest with ties to even.

    bf16 keeps the upper 16 bits of the fp32 pattern.  The discarded low half decides: above half
    an ulp rounds the magnitude up, below rounds down, exactly half rounds to the even upper
    pattern.  A carry out of the mantissa moves to the next binade (and from the largest binade to
    infinity), which is what nearest rounding requires.  NaN stays NaN (quiet, sign kept).
    """
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32)
    hi = (u >> np.uint32(16)).astype(np.uint32)
    lo = u & np.uint32(0xFFFF)
    half = np.uint32(0x8000)
    round_up = (lo > half) | ((lo == half) & ((hi & np.uint32(1)) == 1))
    out = hi + round_up.astype(np.uint32)
    is_nan = ((u & np.uint32(0x7F800000)) == np.uint32(0x7F800000)) & ((u & np.uint32(0x007FFFFF)) != 0)
    out = np.where(is_nan, (hi & np.uint32(0x8000)) | np.uint32(0x7FC0), out)
    return out.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> the fp32 values they denote (exact: pad the low half with zeros)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(F32)


def R(x) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value, returned as fp32."""
    return bf16_to_f32(bf16_bits(x))


# --------------------------------------------------------------------------------------------
# Step 1-2: twin-rail momentum and the bf16 cast
# --------------------------------------------------------------------------------------------

def rail_scalars(step: int):
    """(momentum, fast_beta, fast_weight) for a training step.

    The page keeps the fast rail alone until the engage step and blends it with the slow rail
    (weight 0.4385 on the fast one) afterwards; the slow rail is updated at every step.  The
    scheduler that sets the fast beta before the engage step is not on the page, so the fast beta
    is held at its post-engage value 0.85 throughout, and the Nesterov momentum at 0.95.  A step
    counts as engaged from step 514 on.
    """
    fast_weight = 1.0 if step < RAIL_ENGAGE_STEP else RAIL_FAST_WEIGHT
    return 0.95, RAIL_FAST_BETA, fast_weight


def fma32(a, b, c):
    """fp32 fused multiply-add: a*b + c rounded once to fp32 (round to nearest, ties to even).

    The product of two fp32 values is exact in fp64.  The fp64 sum s = a*b + c and its exact error
    e (Knuth's two-sum, a*b + c == s + e) then decide the one fp32 rounding: rounding s is already
    the correctly rounded result unless s lies exactly halfway between two fp32 values, and then
    the sign of e says on which side of that midpoint the exact sum lies (e == 0: ties to even,
    which is what the cast of s does).  A midpoint in fp32's normal range has the fp64 pattern
    1 followed by 28 zeros below the fp32 mantissa; those entries and the ones in fp32's
    subnormal range take the careful path.
    """
    a = np.asarray(a, dtype=F32).astype(np.float64)
    b = np.asarray(b, dtype=F32).astype(np.float64)
    c = np.asarray(c, dtype=F32).astype(np.float64)
    a, b, c = np.broadcast_arrays(a, b, c)
    with np.errstate(over="ignore", invalid="ignore"):
        p = a * b
        s = p + c
        r = s.astype(F32)
        low = np.ascontiguousarray(s).view(np.uint64) & np.uint64(0x1FFFFFFF)
        careful = (low == np.uint64(0x10000000)) | (np.abs(s) < 2.0 ** -126)
        if not careful.any():
            return r
        idx = np.nonzero(careful)
        pi, ci, si = p[idx], c[idx], s[idx]
        bv = si - pi
        e = (pi - (si - bv)) + (ci - bv)
        ri = r[idx]
        r64 = ri.astype(np.float64)
        other = np.where(si > r64, np.nextafter(ri, F32(np.inf)), np.nextafter(ri, F32(-np.inf)))
        o64 = other.astype(np.float64)
        at_midpoint = np.isfinite(o64) & (si == (r64 + o64) / 2) & (e != 0)
        beyond = np.sign(e) == np.sign(o64 - r64)
        r = np.array(r, copy=True)
        r[idx] = np.where(at_midpoint & beyond, other, ri)
        return r


def lerp(start, end, weight):
    """torch's lerp, which the page calls (`lerp_`) for both rails and the Nesterov lookahead.

    The library forms it about the nearer end: for |weight| < 1/2 it is start + weight*(end - start),
    otherwise end + (weight - 1)*(end - start); the difference end - start is one fp32 operation and
    the multiply-add that follows is fused (one rounding).  weight - 1 is an fp32 subtraction
    (exact for weights in [1/2, 1]).  The weight is one scalar for the whole call.
    """
    start = np.asarray(start, dtype=F32)
    end = np.asarray(end, dtype=F32)
    w = F32(weight)
    diff = (end - start).astype(F32)
    if abs(w) < F32(0.5):
        return fma32(w, diff, start)
    return fma32(w - F32(1.0), diff, end)


def momentum_step(grad, velocity, momentum, fast_beta, fast_weight):
    """Twin-rail Nesterov momentum (anvil.py, first block of `anvil_cascade`).

    grad: fp32 [g, m, n]; velocity: fp32 [2, g, m, n], rail 0 fast, rail 1 slow.  Returns the new
    velocity (a copy) and the fp32 lookahead.  All arithmetic is fp32.  The scalar weights are
    formed the way the page forms them: 1 - fast_beta on an fp32 device scalar (an fp32
    subtraction), 1 - 0.98 as a host double that the lerp kernel then takes as fp32.
    """
    g = np.asarray(grad, dtype=F32)
    v = np.array(velocity, dtype=F32, copy=True)
    wf = F32(1.0) - F32(fast_beta)
    ws = F32(1.0 - RAIL_SLOW_BETA)
    w = F32(fast_weight)
    omw = F32(1.0) - w
    mu = F32(momentum)
    v[0] = lerp(v[0], g, wf)
    v[1] = lerp(v[1], g, ws)
    blend = w * v[0] + omw * v[1]
    y = lerp(g, blend, mu)
    return v, y.astype(F32)


# --------------------------------------------------------------------------------------------
# Step 3-4: Gram, trace normalisation, the quintic maps
# --------------------------------------------------------------------------------------------

def _mm(p, q, acc: str = "fp64"):
    """Product of two operands (bf16 values held in fp32, or fp64 in exact mode).

    acc="fp64": accumulated in fp64 (the default, the closest to the exact product).
    acc="fp32": accumulated in fp32 by the BLAS sgemm -- another valid accumulation order, used
    only to measure how far two correct implementations drift apart on a given input.
    """
    if acc == "fp32":
        return np.matmul(np.asarray(p, dtype=F32), np.asarray(q, dtype=F32))
    return np.matmul(np.asarray(p, dtype=np.float64), np.asarray(q, dtype=np.float64))


def _swapT(x):
    return np.swapaxes(x, -1, -2)


def gram(X, tall: bool, exact: bool = False, acc: str = "fp64"):
    """A = X^T X (tall) or X X^T (wide); fp32 accumulation result rounded to bf16."""
    P = _mm(_swapT(X), X, acc) if tall else _mm(X, _swapT(X), acc)
    if exact:
        return P
    return R(P.astype(F32))


def trace_scale(A, exact: bool = False):
    """Trace of the (bf16) Gram's diagonal and the scale d = sqrt(trace) * margin + eps.

    Returns (trace, d) with shape [..., 1, 1].  In bf16 mode the diagonal entries are the stored
    bf16 values, widened to fp32 and summed in fp32.
    """
    diag = np.diagonal(A, axis1=-2, axis2=-1)
    if exact:
        tr = diag.sum(axis=-1)
        d = np.sqrt(tr) * FROBENIUS_MARGIN + FROBENIUS_EPS
        return tr[..., None, None], d[..., None, None]
    diag = diag.astype(F32)
    tr = np.zeros(diag.shape[:-1], dtype=F32)
    for i in range(diag.shape[-1]):          # fp32 running sum, one entry at a time
        tr = (tr + diag[..., i]).astype(F32)
    d = (np.sqrt(tr).astype(F32) * F32(FROBENIUS_MARGIN)).astype(F32) + F32(FROBENIUS_EPS)
    return tr[..., None, None], d.astype(F32)[..., None, None]


def normalize(X, A, d, exact: bool = False):
    """X / d and A / d^2, each rounded back to bf16 (d^2 is an fp32 square)."""
    if exact:
        return X / d, A / (d * d)
    d = d.astype(F32)
    return R(X.astype(F32) / d), R(A.astype(F32) / (d * d))


def poly(A, b, c, exact: bool = False, acc: str = "fp64"):
    """B = b*A + c*(A @ A); the product is fp32 and the sum is formed in fp32 before rounding."""
    if exact:
        return b * A + c * _mm(A, A)
    Q = _mm(A, A, acc).astype(F32)
    return R(F32(b) * A + F32(c) * Q)


def apply(X, B, a, tall: bool, split: bool, exact: bool = False, acc: str = "fp64"):
    """C = a*X + X@B (tall) or a*X + B@X (wide).

    Fused form: the fp32 product plus a*X, rounded once.  Split form (banks with more than 1024
    rows): the product is stored as bf16 first, and a*X is added to that bf16 value in fp32.
    """
    P = _mm(X, B, acc) if tall else _mm(B, X, acc)
    if exact:
        return a * X + P
    P = P.astype(F32)
    aX = F32(a) * X.astype(F32)
    if split:
        return R(R(P) + aX)
    return R(aX + P)


def cascade(X, split: bool | None = None, exact: bool = False, maps=ANVIL_MAPS,
            return_trace: bool = False, acc: str = "fp64"):
    """The orthogonalising cascade on a bf16 stack X [g, m, n] (values held as fp32).

    `split` defaults to the page's rule (more than 1024 rows).  Orientation: tall iff rows > cols,
    so square matrices take the wide branch.  Returns the final bf16 X (fp32 values), or fp64 in
    exact mode; with return_trace=True also the trace and d of the first Gram.
    """
    X = np.asarray(X, dtype=np.float64 if exact else F32)
    m, n = X.shape[-2], X.shape[-1]
    tall = m > n
    if split is None:
        split = m > SPLIT_BADDBMM_MIN_ROWS
    A = gram(X, tall, exact, acc)
    tr, d = trace_scale(A, exact)
    X, A = normalize(X, A, d, exact)
    for k, (a, b, c) in enumerate(maps):
        if k > 0:
            A = gram(X, tall, exact, acc)
        B = poly(A, b, c, exact, acc)
        X = apply(X, B, a, tall, split, exact, acc)
    if return_trace:
        return X, tr, d
    return X


def bank_step(grad, velocity, momentum, fast_beta, fast_weight, split: bool | None = None):
    """One ANVIL bank step: momentum, cast, cascade.

    Returns (out_bits uint16 [g, m, n], new velocity fp32 [2, g, m, n]).
    """
    v, y = momentum_step(grad, velocity, momentum, fast_beta, fast_weight)
    X = R(y)
    out = cascade(X, split=split)
    return bf16_bits(out), v


# --------------------------------------------------------------------------------------------
# The rest of the bank update: per-lane energy equalizer, sign-aligned decay with a
# mantissa-tracked fp32 master (modded-nanogpt anvil.py, `_rail_equalizer`,
# `_sign_aligned_decay_update`, `anvil_bank_update`)
# --------------------------------------------------------------------------------------------

def lane_axis(m: int, n: int) -> int:
    """Axis the equalizer reduces over: the columns (axis -1) when rows >= cols, else the rows.

    The page's docstring calls it the longer dimension, but its code sets the reduction axis to
    the last one whenever rows >= cols; the code is followed.  The lanes are what remains: one per
    row (rows >= cols) or one per column."""
    return -1 if m >= n else -2


def equalizer_terms(v, lane_energy, beta2):
    """The per-lane terms of the equalizer: (lane power, new lane energy, bf16 lane scale).

    v: bf16 values (fp32 array) [g, m, n]; lane_energy: fp32 [g, m, 1] (rows >= cols) or
    [g, 1, n]; every result has lane_energy's shape.  Steps, all fp32:
      lane power  = mean of v^2 along the reduction axis (sum taken in fp64, rounded to fp32,
                    then divided by the lane length);
      pre norm    = sqrt(sum over lanes of lane power * lane length);
      energy      = energy + (1 - beta2) * (power - energy)      (lerp; 1 - beta2 a host double);
      gain        = 1 / sqrt(max(energy, 1e-10))                 (correctly rounded);
      post norm   = sqrt(sum over lanes of (power * length) * gain^2);
      scale       = bf16(gain * (pre norm / max(post norm, 1e-10))).
    """
    v = np.asarray(v, dtype=F32)
    g, m, n = v.shape
    ax = lane_axis(m, n)
    length = n if ax == -1 else m
    sq = v * v
    power = (sq.astype(np.float64).sum(axis=ax, keepdims=True).astype(F32) / F32(length)).astype(F32)
    psum = power.astype(np.float64).sum(axis=(-2, -1), keepdims=True).astype(F32)
    pre = np.sqrt((psum * F32(length)).astype(F32)).astype(F32)
    e = np.asarray(lane_energy, dtype=F32)
    e = lerp(e, power, F32(1.0 - beta2)).astype(F32)
    gain = (1.0 / np.sqrt(np.maximum(e, F32(1e-10)).astype(np.float64))).astype(F32)
    post_power = ((power * F32(length)).astype(F32) * (gain * gain).astype(F32)).astype(F32)
    post = np.sqrt(post_power.astype(np.float64).sum(axis=(-2, -1), keepdims=True).astype(F32)).astype(F32)
    scale = (gain * (pre / np.maximum(post, F32(1e-10))).astype(F32)).astype(F32)
    return power, e, R(scale)


def equalizer(v, lane_energy, beta2):
    """Per-lane energy equalizer (the terms above), then v <- bf16(v * scale).

    Returns (equalized bf16 values, new lane_energy)."""
    _, e, scale = equalizer_terms(v, lane_energy, beta2)
    return R(np.asarray(v, dtype=F32) * scale), e


def decay_update(p_bits, mantissa, update, eff_wd, eff_lr, gate):
    """Sign-aligned decay and parameter update on a bf16 parameter with a 16-bit mantissa.

    The fp32 master is the parameter's bf16 bits (high half) joined with the mantissa (low half).
    Decay applies where gate * master >= 0 (gate: the slow rail).  master <- (master -
    ((master * aligned) * wd) * lr) - update * lr, each operation fp32; lr is per matrix.  The new
    master splits back into its high half (the new bf16 parameter: a truncation) and low half.
    Returns (new p_bits, new mantissa), both uint16.
    """
    raw = (np.asarray(p_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)) | \
        np.asarray(mantissa, dtype=np.uint16).astype(np.uint32)
    p = raw.view(F32)
    gate = np.asarray(gate, dtype=F32)
    aligned = ((gate * p).astype(F32) >= 0).astype(F32)
    lr = np.asarray(eff_lr, dtype=F32).reshape(-1, 1, 1)
    t1 = (((p * aligned).astype(F32) * F32(eff_wd)).astype(F32) * lr).astype(F32)
    t2 = (np.asarray(update, dtype=F32) * lr).astype(F32)
    newp = ((p - t1).astype(F32) - t2).astype(F32)
    raw2 = newp.view(np.uint32)
    return (raw2 >> np.uint32(16)).astype(np.uint16), (raw2 & np.uint32(0xFFFF)).astype(np.uint16)


def bank_update(grad, velocity, momentum, fast_beta, fast_weight, lane_energy, beta2, p_bits,
                mantissa, eff_wd, eff_lr):
    """The whole bank update: momentum and cascade, equalizer, sign-aligned decay (gate = the new
    slow rail).  Returns (update bits, velocity, lane_energy, p_bits, mantissa)."""
    out_bits, v = bank_step(grad, velocity, momentum, fast_beta, fast_weight)
    upd, e = equalizer(bf16_to_f32(out_bits), lane_energy, beta2)
    pb, mb = decay_update(p_bits, mantissa, upd, eff_wd, eff_lr, v[1])
    return bf16_bits(upd), v, e, pb, mb
