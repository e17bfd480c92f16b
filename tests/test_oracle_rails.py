"""Pins for the twin-rail momentum (modded-nanogpt anvil.py, `anvil_cascade` momentum block and the
rail constants): closed forms of the EMA recursions, the engage schedule and the blend.
"""
import numpy as np

from oracle import anvil_oracle as O


def _run(G, steps, start_step=0):
    v = np.zeros((2,) + G.shape, np.float32)
    ys = []
    for s in range(start_step, start_step + steps):
        mu, fb, fw = O.rail_scalars(s)
        v, y = O.momentum_step(G, v, mu, fb, fw)
        ys.append((s, v.copy(), y))
    return ys


def test_constant_gradient_closed_form():
    """Constant G from zero rails: v0_t = (1 - fb^t) G, v1_t = (1 - 0.98^t) G, and the lookahead
    y_t = G (1 - mu (w fb^t + (1 - w) 0.98^t)), across the engage step."""
    rng = np.random.default_rng(1)
    G = rng.standard_normal((2, 8, 16)).astype(np.float32)
    start = 480
    for t, (s, v, y) in enumerate(_run(G, 60, start), start=1):
        mu, fb, fw = O.rail_scalars(s)
        f = 0.85 ** t
        sl = 0.98 ** t
        np.testing.assert_allclose(v[0], (1 - f) * G, rtol=2e-5, atol=1e-6)
        np.testing.assert_allclose(v[1], (1 - sl) * G, rtol=2e-5, atol=1e-6)
        want = G * (1 - mu * (fw * f + (1 - fw) * sl))
        np.testing.assert_allclose(y, want, rtol=2e-5, atol=1e-6)


def test_engage_schedule():
    assert O.rail_scalars(0) == (0.95, 0.85, 1.0)
    assert O.rail_scalars(513)[2] == 1.0
    assert O.rail_scalars(514)[2] == 0.4385
    assert O.rail_scalars(539)[2] == 0.4385


def test_pre_engage_ignores_slow_rail_but_updates_it():
    """With fast weight 1 the blend is the fast rail exactly, so the lookahead does not depend on
    the slow rail at all; the slow rail still moves (it is updated at every step, engaged or
    not)."""
    rng = np.random.default_rng(2)
    G = rng.standard_normal((1, 16, 8)).astype(np.float32)
    v = rng.standard_normal((2, 1, 16, 8)).astype(np.float32)
    v_other = v.copy()
    v_other[1] = rng.standard_normal((1, 16, 8)).astype(np.float32) * 100
    va, ya = O.momentum_step(G, v, 0.95, 0.85, 1.0)
    vb, yb = O.momentum_step(G, v_other, 0.95, 0.85, 1.0)
    assert np.array_equal(ya, yb)
    assert not np.array_equal(va[1], v[1])
    # post-engage the slow rail does enter the lookahead
    _, yc = O.momentum_step(G, v, 0.95, 0.85, 0.4385)
    _, yd = O.momentum_step(G, v_other, 0.95, 0.85, 0.4385)
    assert not np.array_equal(yc, yd)


def test_fp32_scalar_weights():
    """The fast-rail weight is the fp32 difference 1 - 0.85f; the slow weight is 0.02f."""
    G = np.ones((1, 1, 8), np.float32)
    v = np.zeros((2, 1, 1, 8), np.float32)
    v1, _ = O.momentum_step(G, v, 0.95, 0.85, 1.0)
    assert v1[0, 0, 0, 0].view(np.uint32) == 0x3E199998
    assert v1[1, 0, 0, 0].view(np.uint32) == 0x3CA3D70A


def test_grad_not_written():
    G = np.arange(16, dtype=np.float32).reshape(1, 4, 4)
    G0 = G.copy()
    O.momentum_step(G, np.zeros((2, 1, 4, 4), np.float32), 0.95, 0.85, 0.4385)
    assert np.array_equal(G, G0)
