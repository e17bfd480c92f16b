"""Large single matrices, ragged against every tile size (16392 = 64*256 + 8 rows, 4104 = 8*513
columns), checked by properties that hold at any size (the oracle's fp64 cascade would take
minutes here): the rails bit-exact against the oracle's momentum on sampled elements, and every
output singular value near 1 (the input's normalised spectrum lies inside the maps' window, where
the composed maps land within 0.01 of 1; the bar is 0.3, and 0.1 is checked as well)."""
import numpy as np
import pytest

from oracle import anvil_oracle as O
from orthogonalizing_polynomial_cascade_amd import workloads as W
from tests.helpers import (assert_gemm_close, bf16_bits_of, from_gpu, sigma_classes, to_gpu_f32,
                           update_error)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n", [(16392, 4104), (4104, 16392)])
def test_large_ragged_matrix(gpu_lib, m, n):
    import torch
    G = W.gaussian(1, m, n, seed=21).grad(0)
    vel = torch.zeros((2, 1, m, n), dtype=torch.float32, device="cuda")
    out = gpu_lib.anvil_bank_step(to_gpu_f32(G), vel, 0.95, 0.85, 0.4385)
    torch.cuda.synchronize()
    # rails: the oracle's momentum on sampled elements (elementwise, so any subset is exact)
    rng = np.random.default_rng(3)
    idx = rng.choice(m * n, size=4096, replace=False)
    g_s = G.reshape(-1)[idx].reshape(1, 1, -1)
    v_want, _ = O.momentum_step(g_s, np.zeros((2, 1, 1, idx.size), np.float32), 0.95, 0.85, 0.4385)
    v_got = from_gpu(vel).reshape(2, -1)[:, idx]
    assert np.array_equal(v_got.view(np.uint32), v_want.reshape(2, -1).view(np.uint32))
    # the update's spectrum
    o = out[0].float()
    gram = o.T @ o if m > n else o @ o.T
    ev = torch.linalg.eigvalsh(gram.double()).cpu().numpy()
    sv = np.sqrt(np.clip(ev, 0, None))
    assert sv.min() > 0.7 and sv.max() < 1.3, (sv.min(), sv.max())
    assert sv.min() > 0.9 and sv.max() < 1.1, (sv.min(), sv.max())
    assert torch.isfinite(o).all()



@pytest.mark.parametrize("m,n", [(32768, 32768), (65536, 16384), (16384, 65536)])
def test_max_size_permuted_diagonal(gpu_lib, m, n):
    """One matrix of exactly 2^30 elements (the largest supported: 2 GiB of bf16 per buffer) whose
    nonzeros form a permuted diagonal of powers of two.  Every product in the cascade then has at
    most one nonzero term, so it is exact in any summation order, and the update must be the same
    permutation of the cascade of the bare diagonal, bit for bit: the oracle's cascade of a 64x64
    diagonal with the same trace gives those values (split rounding, as for more than 1024 rows).
    Checked for the six maps and, through the map-table entry point, for the first two (where the
    three values are still apart, so a value paired with the wrong line would show).  The rails
    are set to the gradient and fast_weight is 1, so the lookahead is the gradient."""
    import torch
    s = min(m, n)
    r, counts = sigma_classes(s)
    classes = np.array([1.0, 0.5, 0.25], np.float32)
    diag = np.zeros(64, np.float32)
    diag[:3] = classes
    diag[3:3 + r] = 16.0
    want = {}
    for k in (6, 2):      # the six maps, and the first two (whose three values are still apart)
        small = O.cascade(np.diag(diag)[None], split=True, maps=O.ANVIL_MAPS[:k])[0]
        assert np.count_nonzero(small) == 3 + r
        want[k] = np.array([small[i, i] for i in range(3)], np.float32)
    assert len(set(want[2].tolist())) == 3

    gen = torch.Generator().manual_seed(m + 3 * n)
    cls = torch.cat([torch.full((c,), i, dtype=torch.int64) for i, c in enumerate(counts)])
    cls = cls[torch.randperm(s, generator=gen)]
    lines = torch.randperm(max(m, n), generator=gen)[:s]     # distinct rows (tall) or columns
    idx = torch.arange(s)
    rows, cols = (lines, idx) if m > n else (idx, lines)
    dev = torch.device("cuda")
    rows, cols, cls = rows.to(dev), cols.to(dev), cls.to(dev)
    grad = torch.zeros((1, m, n), dtype=torch.float32, device=dev)
    grad[0, rows, cols] = torch.from_numpy(classes).to(dev)[cls]
    vel = torch.stack([grad, grad])
    for k in (6, 2):
        if k == 6:
            out = gpu_lib.anvil_bank_step(grad, vel, 0.95, 0.85, 1.0)
        else:
            out = gpu_lib.anvil_bank_step_maps(grad, vel, 0.95, 0.85, 1.0, list(O.ANVIL_MAPS[:k]))
        torch.cuda.synchronize()
        assert torch.equal(vel[0], grad) and torch.equal(vel[1], grad)
        got = out[0, rows, cols].float()
        exp = torch.from_numpy(want[k]).to(dev)[cls]
        assert torch.equal(got, exp), (k, got[:8], exp[:8])
        assert int(torch.count_nonzero(out)) == s
        del out
    del grad, vel
    gpu_lib.release_workspaces()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m,n", [(65536, 16384), (16384, 65536)])
def test_max_size_bank_update_composes_the_stages(gpu_lib, m, n):
    """The whole bank update on one matrix of 2^30 elements (row lanes for 65536 x 16384, column
    lanes for the transpose) equals, bit for bit, the step followed by the equalizer and the decay
    entry points (each checked against the oracle at smaller sizes): every index and grid of the
    update kernels at the largest supported size."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(m + n)
    dev = torch.device("cuda")
    G = torch.randn((1, m, n), generator=gen, device=dev) * 1e-3
    lanes = gpu_lib.equalizer_lanes(m, n)
    p0 = (torch.randn((1, m, n), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    m0 = torch.randint(-32768, 32767, (1, m, n), generator=gen, device=dev,
                       dtype=torch.int32).to(torch.int16)
    e0 = torch.rand((1, lanes), generator=gen, device=dev) * 1e-6
    lr = torch.full((1,), 0.02, device=dev)
    wd = 0.0125
    print(f"bank update {m}x{n}", flush=True)

    vel_a = torch.zeros((2, 1, m, n), device=dev)
    p_a, m_a, e_a = p0.clone(), m0.clone(), e0.clone()
    u_a = gpu_lib.anvil_bank_update(G, vel_a, 0.95, 0.85, 0.4385, e_a, 0.95, p_a, m_a, wd, lr)
    torch.cuda.synchronize()

    vel_b = torch.zeros((2, 1, m, n), device=dev)
    p_b, m_b, e_b = p0.clone(), m0.clone(), e0.clone()
    u_b = gpu_lib.anvil_bank_step(G, vel_b, 0.95, 0.85, 0.4385)
    gpu_lib.anvil_equalize(u_b, e_b, 0.95)
    gpu_lib.anvil_decay_update(p_b, m_b, u_b, wd, lr, vel_b[1])
    torch.cuda.synchronize()

    assert torch.equal(vel_a, vel_b)
    assert torch.equal(u_a.view(torch.int16), u_b.view(torch.int16))
    assert torch.equal(e_a, e_b)
    assert torch.equal(p_a.view(torch.int16), p_b.view(torch.int16))
    assert torch.equal(m_a, m_b)
    assert torch.isfinite(u_a.float()).all()
    assert not torch.equal(p_a.view(torch.int16), p0.view(torch.int16))   # the decay moved it
    del G, vel_a, vel_b, p_a, p_b, m_a, m_b, u_a, u_b
    gpu_lib.release_workspaces()
    torch.cuda.empty_cache()


def test_apply_stack_beyond_one_dispatch(gpu_lib):
    """Eight tall 2^27 x 8 matrices (2^33 elements): their apply has 2^23 tiles of 512 work-items,
    more than one dispatch counts (32 bits), so it goes out as two launches (7 + 1 matrices).
    Each matrix of the stack must equal, bit for bit, the apply of that matrix alone (one launch),
    and sampled rows must match the oracle's apply (split rounding: more than 1024 rows)."""
    import torch
    g, m, n = 8, 1 << 27, 8
    dev = torch.device("cuda")
    gen = torch.Generator(device="cuda").manual_seed(29)
    print(f"apply stack {g}x{m}x{n}", flush=True)
    X = torch.empty((g, m, n), dtype=torch.bfloat16, device=dev)
    for i in range(g):
        X[i] = (torch.randn((m, n), generator=gen, device=dev) * 0.1).to(torch.bfloat16)
    S = torch.randn((g, n, n), generator=gen, device=dev) * 0.3
    B = (S + S.transpose(1, 2)).to(torch.bfloat16).contiguous()
    a = O.ANVIL_MAPS[2][0]
    C = gpu_lib.anvil_apply(X, B, a, True)
    torch.cuda.synchronize()
    rows = torch.randint(0, m, (4096,), generator=gen, device=dev)
    rows[:2] = torch.tensor([0, m - 1], device=dev)
    Bh = from_gpu(B)
    for i in (0, 6, 7):
        Ci = gpu_lib.anvil_apply(X[i:i + 1], B[i:i + 1], a, True)
        torch.cuda.synchronize()
        assert torch.equal(C[i].view(torch.int16), Ci[0].view(torch.int16)), i
        del Ci
        want = O.apply(from_gpu(X[i, rows])[None], Bh[i:i + 1], a, True, True)
        assert_gemm_close(from_gpu(C[i, rows])[None], want, f"apply rows of matrix {i}")
    del X, C, B
    torch.cuda.empty_cache()


def test_row_lanes_beyond_the_grid_cap(gpu_lib):
    """Row lanes of a 4195336 x 8 update: more rows than the row-lane kernel's capped grid holds
    waves (2^22), so waves take a second row.  Powers, energies, scales and the rescaled update
    against the oracle's equalizer, with the bars of the equalizer parity tests."""
    from tests.test_gpu_update import _check_equalizer, _gpu_equalize
    g, m, n = 1, (1 << 22) + 1032, 8
    rng = np.random.default_rng(31)
    v = rng.standard_normal((g, m, n)) * np.exp(rng.standard_normal((g, m, 1)))
    u = O.R((v / np.sqrt(m)).astype(np.float32))
    power = (u.astype(np.float64) ** 2).mean(axis=-1, keepdims=True)
    energy = (power * np.exp(rng.standard_normal(power.shape))).astype(np.float32)
    _check_equalizer(u, energy, 0.95, *_gpu_equalize(gpu_lib, u, energy, 0.95))


@pytest.mark.parametrize("m,n", [(8, 16), (16, 8)])
def test_max_stack_count(gpu_lib, m, n):
    """The largest stack count the ABI takes (65535 matrices): every kernel's grid spans the
    whole stack.  Sampled matrices (first, middle, last) against the oracle, the rails bit for bit,
    and a matrix stepped alone equal to its slice of the stack."""
    import torch
    g = 65535
    G = W.gaussian(g, m, n, seed=61).grad(0)
    vel = torch.zeros((2, g, m, n), dtype=torch.float32, device="cuda")
    out = gpu_lib.anvil_bank_step(to_gpu_f32(G), vel, 0.95, 0.85, 0.4385)
    torch.cuda.synchronize()
    got = from_gpu(out)
    v_gpu = from_gpu(vel)
    for i in (0, g // 2, g - 1):
        v_or, y = O.momentum_step(G[i:i + 1], np.zeros((2, 1, m, n), np.float32), 0.95, 0.85,
                                  0.4385)
        assert np.array_equal(v_gpu[:, i:i + 1].view(np.uint32), v_or.view(np.uint32))
        want = O.cascade(O.R(y))[0]
        assert update_error(got[i], want) <= 1e-2, i
        one = gpu_lib.anvil_bank_step(to_gpu_f32(G[i:i + 1]),
                                      torch.zeros((2, 1, m, n), dtype=torch.float32,
                                                  device="cuda"), 0.95, 0.85, 0.4385)
        assert np.array_equal(bf16_bits_of(one)[0], bf16_bits_of(out[i:i + 1])[0]), i
