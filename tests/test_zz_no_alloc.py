"""anvil_bank_step_noalloc (the bank step on the library's built-in device scratch, for callers
that cannot allocate) against anvil_bank_step (the same kernels on an allocated workspace), through
the C ABI: bit-identical updates and rails on two calls in a row, the second with a smaller bank,
and a clear refusal of a bank larger than the scratch."""
import numpy as np
import pytest

from orthogonalizing_polynomial_cascade_amd import workloads as W
from tests.helpers import bf16_bits_of, to_gpu_f32

pytestmark = pytest.mark.gpu


def _pair(gpu_lib, G, v, mu, fb, fw):
    import torch
    g, m, n = G.shape
    v_ref, v_na = v.clone(), v.clone()
    ref = gpu_lib.anvil_bank_step(G, v_ref, mu, fb, fw)
    out = torch.full((g, m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    got = gpu_lib.anvil_bank_step_noalloc(G, v_na, mu, fb, fw, out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert np.array_equal(bf16_bits_of(got), bf16_bits_of(ref))
    assert torch.equal(v_na, v_ref)
    return got


def test_noalloc_matches_bank_step_two_calls(gpu_lib):
    """The mlp bank (the largest benchmark bank of this shape family) and then a smaller, ragged
    bank on the same scratch: each equals anvil_bank_step bit for bit, so nothing of the first
    call's scratch contents leaks into the second."""
    import torch
    w = W.mlp_bank()
    assert gpu_lib.workspace_bytes(w.g, w.m, w.n) <= gpu_lib.NOALLOC_SCRATCH_BYTES
    G = to_gpu_f32(w.grad(w.measured[-1]))
    v = torch.randn((2, w.g, w.m, w.n), dtype=torch.float32, device="cuda")
    _pair(gpu_lib, G, v, 0.95, 0.85, 0.4385)
    g, m, n = 3, 200, 328
    G2 = to_gpu_f32(W.gaussian(g, m, n, seed=77).grad(0))
    v2 = torch.randn((2, g, m, n), dtype=torch.float32, device="cuda")
    _pair(gpu_lib, G2, v2, 0.95, 0.85, 1.0)
    # and the tall/split path once more at a small size after the wide one
    g, m, n = 2, 1096, 136
    G3 = to_gpu_f32(W.gaussian(g, m, n, seed=78).grad(0))
    _pair(gpu_lib, G3, torch.zeros((2, g, m, n), dtype=torch.float32, device="cuda"), 0.95, 0.85,
          1.0)


def test_noalloc_refuses_banks_beyond_its_scratch(gpu_lib):
    """A bank whose workspace exceeds the scratch is refused before anything is enqueued: the
    rails and `out` stay as they were."""
    import torch
    g, m, n = 48, 2816, 768          # twice the mlp bank: about 322 MB of workspace
    assert gpu_lib.workspace_bytes(g, m, n) > gpu_lib.NOALLOC_SCRATCH_BYTES
    G = torch.ones((g, m, n), dtype=torch.float32, device="cuda")
    v = torch.zeros((2, g, m, n), dtype=torch.float32, device="cuda")
    out = torch.zeros((g, m, n), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.AnvilError) as err:
        gpu_lib.anvil_bank_step_noalloc(G, v, 0.95, 0.85, 1.0, out)
    assert err.value.status == gpu_lib.ANVIL_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert not v.any() and not out.float().any()


def test_noalloc_empty_and_invalid(gpu_lib):
    import torch
    G = torch.zeros((0, 64, 32), dtype=torch.float32, device="cuda")
    v = torch.zeros((2, 0, 64, 32), dtype=torch.float32, device="cuda")
    out = torch.zeros((0, 64, 32), dtype=torch.bfloat16, device="cuda")
    gpu_lib.anvil_bank_step_noalloc(G, v, 0.95, 0.85, 1.0, out)
    G = torch.zeros((1, 64, 36), dtype=torch.float32, device="cuda")      # n not a multiple of 8
    v = torch.zeros((2, 1, 64, 36), dtype=torch.float32, device="cuda")
    out = torch.zeros((1, 64, 36), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.AnvilError) as err:
        gpu_lib.anvil_bank_step_noalloc(G, v, 0.95, 0.85, 1.0, out)
    assert err.value.status == gpu_lib.ANVIL_ERR_UNSUPPORTED
