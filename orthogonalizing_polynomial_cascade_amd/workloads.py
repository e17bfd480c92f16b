"""Seeded synthetic gradient stacks for the ANVIL bank-step workloads.

This module only draws inputs; it holds none of the method's arithmetic, so the HIP path and the
CPU oracle can both take their inputs from it.  Every generator uses numpy's PCG64 with a fixed
seed and returns C-contiguous fp32 arrays of shape [g, m, n].

The five workloads follow the bank shapes of the source page (modded-nanogpt anvil.py: qk, vo and
mlp banks of a 768-wide model) and the stacked V/U masters of the param-decomp pull request #989
(same-shape stacks Vs [g, d_in, C], Us [g, C, d_out]).  The value distributions are synthetic
stand-ins chosen to exercise the cascade: row-scaled, spiked, badly column-scaled, low-rank-plus-
noise and heavy-tailed gradients.

Each workload lists its steps as training-step ids; the rail scalars for a step come from the
caller's own schedule (momentum 0.95, fast beta 0.85, fast weight 1.0 before step 514 and 0.4385
from then on).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = np.float32


def _rng(seed: int, index: int | None = None) -> np.random.Generator:
    """PCG64 stream for a seed, or for (seed, matrix index) when each matrix of a stack draws its
    own fixed part -- so any prefix of a stack is the same whatever its length."""
    return np.random.Generator(np.random.PCG64(seed if index is None else [seed, index]))


@dataclass
class Workload:
    """A named stack shape, the step ids it runs, and a seeded gradient per step."""
    name: str
    g: int
    m: int
    n: int
    step_ids: list
    measured: list            # indices into step_ids whose cascade output is checked / timed
    _fixed: dict = field(default_factory=dict, repr=False)

    def grad(self, t: int, g: int | None = None) -> np.ndarray:
        """Gradient for local step t (0-based index into step_ids).  g limits the stack."""
        return _GRADS[self.name](self, t, self.g if g is None else g)


def _fixed(w: Workload, key, make):
    if key not in w._fixed:
        w._fixed[key] = make()
    return w._fixed[key]


def _single_wide(w, t, g):
    out = np.empty((g, w.m, w.n), F32)
    for i in range(g):
        r = _rng(101 + 7919 * t, i)
        z = r.standard_normal((w.m, w.n))
        scale = np.exp(r.standard_normal((w.m, 1)))
        out[i] = z * scale
    return out


def _qk(w, t, g):
    def spikes():
        us, vs = [], []
        for i in range(w.g):
            r = _rng(2999, i)
            us.append(np.linalg.qr(r.standard_normal((w.m, 8)))[0])
            vs.append(np.linalg.qr(r.standard_normal((w.n, 8)))[0])
        return np.stack(us), np.stack(vs)
    U, V = _fixed(w, "spikes", spikes)
    noise_std = 0.02
    # spike singular value: 100x the largest singular value a Gaussian noise matrix of this shape
    # has (Marchenko-Pastur edge, std * (sqrt(m) + sqrt(n)))
    sig = 100.0 * noise_std * (np.sqrt(w.m) + np.sqrt(w.n))
    noise = noise_std * _rng(2000 + t).standard_normal((g, w.m, w.n))
    spike = sig * np.matmul(U[:g], np.swapaxes(V[:g], 1, 2))
    return (noise + spike).astype(F32)


def _vo(w, t, g):
    cols = _fixed(w, "cols", lambda: np.stack(
        [np.exp(2.0 * _rng(3999, i).standard_normal((1, w.n))) for i in range(w.g)]))
    z = _rng(3000 + t).standard_normal((g, w.m, w.n))
    return (z * cols[:g]).astype(F32)


def _mlp(w, t, g):
    def lowrank():
        P = np.empty((w.g, w.m, 32))
        Q = np.empty((w.g, 32, w.n))
        for i in range(w.g):
            r = _rng(4999, i)
            P[i] = r.standard_normal((w.m, 32))
            Q[i] = r.standard_normal((32, w.n))
        return P, Q
    def low_part():
        P, Q = _fixed(w, "lowrank", lowrank)
        return 10.0 * np.matmul(P, Q) / np.sqrt(32.0)
    low = _fixed(w, "low", low_part)[:g]
    z = _rng(4000 + t).standard_normal((g, w.m, w.n))
    return (z + low).astype(F32)


def _student_t(seed, g, m, n):
    # Student-t with 3 degrees of freedom has variance 3; rescale to std 1e-3
    return (1e-3 * _rng(seed).standard_t(3, size=(g, m, n)) / np.sqrt(3.0)).astype(F32)


def _vs(w, t, g):
    return _student_t(5000 + t, g, w.m, w.n)


def _us(w, t, g):
    return _student_t(6000 + t, g, w.m, w.n)


def _gauss(w, t, g):
    return _rng(w._fixed.get("seed", 0) + 104729 * t).standard_normal((g, w.m, w.n)).astype(F32)


_GRADS = {
    "single_wide": _single_wide,
    "qk": _qk,
    "vo": _vo,
    "mlp": _mlp,
    "vs": _vs,
    "us": _us,
    "gauss": _gauss,
}


def single_wide() -> Workload:
    """One 256x768 matrix, rows scaled by lognormal(0, 1); one step from zero rails."""
    return Workload("single_wide", 1, 256, 768, step_ids=[0], measured=[0])


def qk_bank(g: int = 24) -> Workload:
    """g x 256x768 (wide): N(0, 0.02^2) noise plus a fixed rank-8 spike 100x the noise edge;
    20 warm-up steps then the measured step, all before the engage step."""
    return Workload("qk", g, 256, 768, step_ids=list(range(21)), measured=[20])


def vo_bank(g: int = 24) -> Workload:
    """g x 768x768 (square, wide branch): N(0,1) with fixed lognormal(0, 2) column scales
    (condition number around 1e4); 10 consecutive engaged steps."""
    return Workload("vo", g, 768, 768, step_ids=list(range(514, 524)), measured=list(range(10)))


def mlp_bank(g: int = 24) -> Workload:
    """g x 2816x768 (tall, split apply): N(0,1) plus a fixed rank-32 part with entries of std 10;
    20 warm-up steps (470-489) then steps 490-539 across the engage step 514."""
    ids = list(range(470, 540))
    measured = [ids.index(s) for s in (490, 513, 514, 539)]
    return Workload("mlp", g, 2816, 768, step_ids=ids, measured=measured)


def vs_stack(g: int = 32) -> Workload:
    """Vs [g, 4096, 512] (tall, split): Student-t(3) entries with std 1e-3; 3 engaged steps."""
    return Workload("vs", g, 4096, 512, step_ids=[514, 515, 516], measured=[0, 1, 2])


def us_stack(g: int = 32) -> Workload:
    """Us [g, 512, 4096] (wide, fused): Student-t(3) entries with std 1e-3; 3 engaged steps."""
    return Workload("us", g, 512, 4096, step_ids=[514, 515, 516], measured=[0, 1, 2])


def gaussian(g: int, m: int, n: int, seed: int = 0, steps=(0,)) -> Workload:
    """A plain N(0,1) stack of any shape, for parity sweeps over shapes and tails."""
    w = Workload("gauss", g, m, n, step_ids=list(steps), measured=list(range(len(steps))))
    w._fixed["seed"] = seed
    return w


def scaled(w: Workload, g: int | None = None, m: int | None = None, n: int | None = None) -> Workload:
    """The same distribution at a smaller shape (for oracle-sized parity cases)."""
    return Workload(w.name, g or w.g, m or w.m, n or w.n, list(w.step_ids), list(w.measured))


@dataclass
class UpdateState:
    """Parameter-side inputs of a whole bank update for a [g, m, n] bank (synthetic values: the
    page names the fields but not their magnitudes)."""
    param_bits: np.ndarray    # uint16 [g, m, n]: high halves of N(0, 0.02^2) fp32 masters
    mantissa: np.ndarray      # uint16 [g, m, n]: their low halves
    lane_energy: np.ndarray   # fp32 [g, lanes]: zeros (a fresh optimizer)
    eff_lr: np.ndarray        # fp32 [g]: 0.02, doubled on odd matrices of the mlp bank
    eff_wd: float             # 0.02 * 0.025: an lr times a weight decay
    beta2: float              # 0.95


def update_state(w: Workload, g: int | None = None, seed: int = 7) -> UpdateState:
    """fp32 master weights N(0, 0.02^2) stored the page's way: the high 16 bits as the bf16
    parameter, the low 16 bits as the mantissa."""
    g = w.g if g is None else g
    r = _rng(seed + 31 * w.m + w.n)
    master = (r.standard_normal((g, w.m, w.n)) * 0.02).astype(F32).view(np.uint32)
    lanes = w.m if w.m >= w.n else w.n
    mult = [2.0 if (w.name == "mlp" and i % 2 == 1) else 1.0 for i in range(g)]
    eff_lr = np.array([0.02 * k for k in mult], dtype=F32)
    return UpdateState((master >> np.uint32(16)).astype(np.uint16),
                       (master & np.uint32(0xFFFF)).astype(np.uint16),
                       np.zeros((g, lanes), F32), eff_lr, 0.02 * 0.025, 0.95)

ALL = {
    "single_wide": single_wide,
    "qk": qk_bank,
    "vo": vo_bank,
    "mlp": mlp_bank,
    "vs": vs_stack,
    "us": us_stack,
}
