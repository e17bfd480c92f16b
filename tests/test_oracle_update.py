"""Pins for the rest of the bank update (modded-nanogpt anvil.py, `_rail_equalizer`,
`_sign_aligned_decay_update`, `anvil_bank_update`)."""
import numpy as np
import pytest

from oracle import anvil_oracle as O


def _bf16(rng, shape, scale=1.0):
    return O.R((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("shape", [(2, 64, 24), (2, 24, 64), (1, 40, 40)])
def test_fresh_equalizer_equalises_lane_energy(shape):
    """With beta2 = 0 the energy EMA equals this step's lane power, the gain is its inverse root,
    so every lane ends with the same mean square (the matrix mean square, by norm preservation)."""
    rng = np.random.default_rng(sum(shape))
    scales = np.exp(rng.standard_normal((shape[0], shape[1], 1)))     # very unequal rows
    v = O.R(_bf16(rng, shape) * scales.astype(np.float32))
    g, m, n = shape
    ax = -1 if m >= n else -2
    e = np.zeros((g, m, 1) if ax == -1 else (g, 1, n), np.float32)
    out, e2 = O.equalizer(v, e, 0.0)
    lane_ms = (out.astype(np.float64) ** 2).mean(axis=ax)
    total_ms = (out.astype(np.float64) ** 2).mean(axis=(1, 2))[:, None]
    assert np.all(np.abs(lane_ms / total_ms - 1) < 2e-2)
    np.testing.assert_allclose(e2.squeeze(), (v.astype(np.float64) ** 2).mean(axis=ax).squeeze(), rtol=1e-6)


@pytest.mark.parametrize("beta2", [0.0, 0.5, 0.95])
def test_equalizer_preserves_frobenius_norm(beta2):
    rng = np.random.default_rng(3)
    v = _bf16(rng, (3, 48, 32))
    e = np.abs(rng.standard_normal((3, 48, 1))).astype(np.float32)
    out, _ = O.equalizer(v, e, beta2)
    for i in range(3):
        r = np.linalg.norm(out[i]) / np.linalg.norm(v[i])
        assert abs(r - 1) < 1e-2


def test_uniform_state_and_frozen_ema_is_identity():
    """Equal energies and beta2 = 1 (the EMA does not move): every gain is the same, the rescale
    brings the norm back, the scale rounds to exactly 1 in bf16 and the update is unchanged."""
    rng = np.random.default_rng(4)
    v = _bf16(rng, (2, 40, 24))
    e = np.full((2, 40, 1), 0.37, np.float32)
    out, e2 = O.equalizer(v, e, 1.0)
    assert np.array_equal(out, v)
    assert np.array_equal(e2, e)


def test_orientation_by_transpose():
    """Tall matrices reduce over their columns, wide ones over their rows: the wide equalizer on
    v^T is the transpose of the tall one on v."""
    rng = np.random.default_rng(5)
    v = _bf16(rng, (2, 56, 24)) * np.exp(rng.standard_normal((2, 56, 1))).astype(np.float32)
    v = O.R(v)
    e = np.abs(rng.standard_normal((2, 56, 1))).astype(np.float32)
    a, ea = O.equalizer(v, e, 0.9)
    b, eb = O.equalizer(np.swapaxes(v, 1, 2).copy(), np.swapaxes(e, 1, 2).copy(), 0.9)
    assert np.mean(a == np.swapaxes(b, 1, 2)) > 0.999
    np.testing.assert_allclose(ea, np.swapaxes(eb, 1, 2), rtol=1e-6)


def test_zero_update_stays_zero_and_energy_decays():
    v = np.zeros((1, 16, 8), np.float32)
    e = np.full((1, 16, 1), 2.0, np.float32)
    out, e2 = O.equalizer(v, e, 0.75)
    assert np.all(out == 0)
    assert np.allclose(e2, 2.0 * 0.75)


def _raw(p_bits, mant):
    return ((np.uint32(p_bits) << np.uint32(16)) | np.uint32(mant)).view(np.float32)


def test_master_round_trip_and_truncation():
    """Without update or decay the bits come back unchanged, and the parameter is the high half of
    the fp32 master (a truncation: 1 + 2^-8 + 2^-9 keeps 0x3F80 where nearest rounding would give
    0x3F81)."""
    p = np.array([[[0x3F80, 0xBF12, 0x0001, 0x7F7F]]], np.uint16)
    mnt = np.array([[[0xC000, 0x1234, 0xFFFF, 0x0000]]], np.uint16)
    u = np.zeros((1, 1, 4), np.float32)
    gate = np.ones((1, 1, 4), np.float32)
    pb, mb = O.decay_update(p, mnt, u, 0.0, np.array([0.5], np.float32), gate)
    assert np.array_equal(pb, p) and np.array_equal(mb, mnt)
    assert np.float32(1 + 2 ** -8 + 2 ** -9).view(np.uint32) == 0x3F80C000


def test_decay_hand_worked():
    """master 1.0, update 2, wd 0.5, lr 0.25: aligned gate gives 1 - 0.125 - 0.5 = 0.375
    (0x3EC00000), an opposite gate skips the decay: 1 - 0.5 = 0.5 (0x3F000000).  A zero gate
    counts as aligned (the test is >= 0)."""
    p = np.full((1, 1, 3), 0x3F80, np.uint16)
    mnt = np.zeros((1, 1, 3), np.uint16)
    u = np.full((1, 1, 3), 2.0, np.float32)
    gate = np.array([[[3.0, -3.0, 0.0]]], np.float32)
    pb, mb = O.decay_update(p, mnt, u, 0.5, np.array([0.25], np.float32), gate)
    assert list(pb.ravel()) == [0x3EC0, 0x3F00, 0x3EC0]
    assert list(mb.ravel()) == [0, 0, 0]


def test_per_matrix_lr_and_frozen_matrix():
    rng = np.random.default_rng(6)
    p = O.bf16_bits(rng.standard_normal((2, 8, 8)).astype(np.float32))
    mnt = rng.integers(0, 1 << 16, (2, 8, 8)).astype(np.uint16)
    u = _bf16(rng, (2, 8, 8))
    gate = rng.standard_normal((2, 8, 8)).astype(np.float32)
    pb, mb = O.decay_update(p, mnt, u, 0.1, np.array([0.0, 0.01], np.float32), gate)
    assert np.array_equal(pb[0], p[0]) and np.array_equal(mb[0], mnt[0])   # lr 0: frozen
    assert not np.array_equal(pb[1], p[1]) or not np.array_equal(mb[1], mnt[1])


def test_bank_update_gates_on_the_new_slow_rail():
    """The decay gate is the slow rail after this step's lerp.  Each old slow-rail entry has the
    opposite sign of a large (|g| >= 60), full-rank gradient, so the lerp (weight 0.02) flips it;
    the parameter takes the old rail's sign, so with the new rail nothing is aligned and no decay
    applies (with the old rail everything would be)."""
    rng = np.random.default_rng(7)
    g, m, n = 1, 16, 8
    z = rng.standard_normal((g, m, n))
    grad = (np.sign(z) * (60.0 + 10.0 * np.abs(rng.standard_normal((g, m, n))))).astype(np.float32)
    vel = np.zeros((2, g, m, n), np.float32)
    vel[1] = -np.sign(grad)
    p = np.where(vel[1] > 0, 0x3F80, 0xBF80).astype(np.uint16)     # +1 or -1, sign of the old rail
    mnt = np.zeros((g, m, n), np.uint16)
    e = np.ones((g, m, 1), np.float32)
    lr = np.array([1e-3], np.float32)
    upd_bits, v, e2, pb, mb = O.bank_update(grad, vel, 0.95, 0.85, 1.0, e, 0.95, p, mnt, 0.5, lr)
    assert np.all(np.sign(v[1]) == np.sign(grad))
    u = O.bf16_to_f32(upd_bits)
    p0 = ((p.astype(np.uint32) << 16)).view(np.float32)
    want = (p0 - (u * lr[0]).astype(np.float32)).astype(np.float32)   # no decay term
    got = ((pb.astype(np.uint32) << 16) | mb.astype(np.uint32)).view(np.float32)
    assert np.array_equal(got, want)


def test_scale_is_rounded_to_bf16_golden():
    import json, os
    c = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "rounding_points.json")))["equalizer_scale_rounded"]
    v = np.array(c["update"], np.float32)[None]
    e = np.array(c["lane_energy"], np.float32)[None]
    out, e2 = O.equalizer(v, e, c["beta2"])
    assert np.array_equal(out[0], np.array(c["out"], np.float32))
    assert np.array_equal(e2, e)
