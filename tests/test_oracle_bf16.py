"""Pin: the oracle's fp32 -> bf16 rounding against torch's CPU cast (round to nearest even).

torch is an independent library witness here; it is used only as a checker.
"""
import numpy as np
import torch

from oracle import anvil_oracle as O


def _torch_bits(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(f32.copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _edge_patterns() -> np.ndarray:
    pats = []
    for sign in (0, 1):
        for exp in list(range(0, 4)) + list(range(100, 140)) + list(range(250, 256)):
            for hi_mant in (0, 1, 2, 0x3E, 0x3F, 0x40, 0x7E, 0x7F):
                for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
                    u = (sign << 31) | (exp << 23) | (hi_mant << 16) | lo
                    pats.append(u)
    pats += [0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F7FFF, 0x7F7F8000, 0x7F7E8000, 0x00008000, 0x00018000,
             0x7F800000, 0xFF800000, 0x00000000, 0x80000000, 0x00000001, 0x007FFFFF]
    return np.array(pats, dtype=np.uint32)


def test_bf16_edge_patterns_match_torch():
    u = _edge_patterns()
    f = u.view(np.float32)
    ours = O.bf16_bits(f)
    ref = _torch_bits(f)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN
    assert np.all(np.isnan(O.bf16_to_f32(ours[nan])))


def test_bf16_random_patterns_match_torch():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    nan = np.isnan(f)
    assert np.array_equal(O.bf16_bits(f)[~nan], _torch_bits(f)[~nan])


def test_ties_go_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even is 1.
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    x = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8)], dtype=np.float32)
    assert list(O.R(x)) == [1.0, 1 + 2**-6, -1.0]


def test_widening_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_to_f32(bits)
    ok = ~np.isnan(f)
    assert np.array_equal(O.bf16_bits(f)[ok], bits[ok])
