"""Property tests of the bank step on the GPU that need no oracle value:

* poisoned buffers: `out`, the workspace and the stage outputs filled with NaN bit patterns before
  a call must not change a single bit of the result, so every element of every intermediate (the
  mirrored halves of the Gram and the polynomial, ragged tile edges, diagonal tiles) is written
  before it is read;
* checkpoint and resume: rails (and the update's lane energies, parameter and mantissa) copied to
  the host after N steps and restored into fresh buffers continue bit-identically to an
  uninterrupted run (the step keeps no hidden state between calls).

The source of the step is modded-nanogpt anvil.py, `anvil_cascade` and `anvil_bank_update`."""
import numpy as np
import pytest

from orthogonalizing_polynomial_cascade_amd import workloads as W
from tests.helpers import bf16_bits_of, to_gpu_f32

pytestmark = pytest.mark.gpu

SHAPES = [(3, 200, 328), (2, 392, 136), (2, 264, 264), (2, 1096, 136), (1, 8, 16), (2, 136, 1096)]


def _nan_fill(t):
    """Fill a tensor's bytes with 0xFF (a NaN in bf16 and in fp32)."""
    import torch
    t.view(torch.uint8).fill_(0xFF)
    return t


@pytest.mark.parametrize("g,m,n", SHAPES)
def test_poisoned_out_and_workspace(gpu_lib, g, m, n):
    import torch
    G = to_gpu_f32(W.gaussian(g, m, n, seed=31).grad(0))
    v0 = torch.randn((2, g, m, n), dtype=torch.float32, device="cuda")
    nb = gpu_lib.workspace_bytes(g, m, n)
    ws_clean = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    out_clean = torch.zeros((g, m, n), dtype=torch.bfloat16, device="cuda")
    ref = gpu_lib.anvil_bank_step(G, v0.clone(), 0.95, 0.85, 0.4385, out=out_clean,
                                  workspace=ws_clean)
    ws = _nan_fill(torch.empty(nb, dtype=torch.uint8, device="cuda"))
    out = _nan_fill(torch.empty((g, m, n), dtype=torch.bfloat16, device="cuda"))
    v = v0.clone()
    got = gpu_lib.anvil_bank_step(G, v, 0.95, 0.85, 0.4385, out=out, workspace=ws)
    assert torch.isfinite(got.float()).all()
    assert np.array_equal(bf16_bits_of(got), bf16_bits_of(ref))
    # the same through a table of odd length (X starts in the workspace copy)
    maps = [(3.4445, -4.7750, 2.0315)] * 3
    ref3 = gpu_lib.anvil_bank_step_maps(G, v0.clone(), 0.95, 0.85, 0.4385, maps,
                                        workspace=ws_clean.zero_())
    got3 = gpu_lib.anvil_bank_step_maps(G, v0.clone(), 0.95, 0.85, 0.4385, maps,
                                        out=_nan_fill(torch.empty_like(out)),
                                        workspace=_nan_fill(ws))
    assert np.array_equal(bf16_bits_of(got3), bf16_bits_of(ref3))


@pytest.mark.parametrize("g,m,n", SHAPES)
def test_poisoned_stage_outputs(gpu_lib, g, m, n):
    """Each stage entry point writes every element of its output: the Gram and the polynomial
    (upper-triangle tiles, mirrored), the trace partials, the apply."""
    import torch
    x = torch.randn((g, m, n), device="cuda").to(torch.bfloat16)
    s = min(m, n)
    a_ref, t_ref = gpu_lib.anvil_gram(x, want_trace=True)
    a_bad = _nan_fill(torch.empty((g, s, s), dtype=torch.bfloat16, device="cuda"))
    t_bad = _nan_fill(torch.empty_like(t_ref))
    a, t = gpu_lib.anvil_gram(x, a_out=a_bad, trace_partials=t_bad)
    assert np.array_equal(bf16_bits_of(a), bf16_bits_of(a_ref))
    assert torch.equal(t, t_ref)
    a_n = (a_ref.float() / a_ref.float().abs().max()).to(torch.bfloat16)
    b_ref = gpu_lib.anvil_poly(a_n, -4.7750, 2.0315)
    b = gpu_lib.anvil_poly(a_n, -4.7750, 2.0315, b_out=_nan_fill(torch.empty_like(b_ref)))
    assert np.array_equal(bf16_bits_of(b), bf16_bits_of(b_ref))
    for split in (False, True):
        c_ref = gpu_lib.anvil_apply(x, b_ref, 3.4445, split)
        c = gpu_lib.anvil_apply(x, b_ref, 3.4445, split, c_out=_nan_fill(torch.empty_like(x)))
        assert np.array_equal(bf16_bits_of(c), bf16_bits_of(c_ref))


@pytest.mark.parametrize("g,m,n", [(2, 1096, 136), (3, 200, 328)])
def test_checkpoint_resume_bank_step(gpu_lib, g, m, n):
    """Six steps straight through, against three steps, the rails saved to host memory, a restore
    into fresh device buffers (and a fresh workspace) and three more steps: bit-identical rails and
    update at every step after the restore."""
    import torch
    w = W.gaussian(g, m, n, seed=41, steps=range(6))
    grads = [to_gpu_f32(w.grad(t)) for t in range(6)]
    sched = [(0.95, 0.85, 1.0)] * 3 + [(0.95, 0.85, 0.4385)] * 3
    vel = torch.zeros((2, g, m, n), dtype=torch.float32, device="cuda")
    straight = []
    for G, (mu, fb, fw) in zip(grads, sched):
        u = gpu_lib.anvil_bank_step(G, vel, mu, fb, fw)
        straight.append((bf16_bits_of(u), vel.cpu().numpy().copy()))
    vel = torch.zeros((2, g, m, n), dtype=torch.float32, device="cuda")
    for G, (mu, fb, fw) in zip(grads[:3], sched[:3]):
        gpu_lib.anvil_bank_step(G, vel, mu, fb, fw)
    saved = vel.cpu().numpy().copy()
    del vel
    gpu_lib.release_workspaces()
    restored = torch.from_numpy(saved).cuda()
    ws = torch.empty(gpu_lib.workspace_bytes(g, m, n), dtype=torch.uint8, device="cuda")
    for k in range(3, 6):
        mu, fb, fw = sched[k]
        u = gpu_lib.anvil_bank_step(grads[k], restored, mu, fb, fw, workspace=ws)
        assert np.array_equal(bf16_bits_of(u), straight[k][0]), f"update at step {k}"
        assert np.array_equal(restored.cpu().numpy().view(np.uint32),
                              straight[k][1].view(np.uint32)), f"rails at step {k}"


def test_checkpoint_resume_bank_update(gpu_lib):
    """The same for the whole bank update, whose state also holds the lane energies, the bf16
    parameter and its mantissa."""
    import torch
    g, m, n = 2, 392, 136
    w = W.gaussian(g, m, n, seed=43, steps=range(4))
    grads = [to_gpu_f32(w.grad(t)) for t in range(4)]
    st = W.update_state(w)

    def fresh():
        vel = torch.zeros((2, g, m, n), dtype=torch.float32, device="cuda")
        pb = torch.from_numpy(st.param_bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
        mt = torch.from_numpy(st.mantissa.view(np.int16).copy()).cuda()
        en = torch.from_numpy(st.lane_energy.copy()).cuda()
        return vel, pb, mt, en

    lr = torch.from_numpy(st.eff_lr.copy()).cuda()

    def step(state, G):
        vel, pb, mt, en = state
        return bf16_bits_of(gpu_lib.anvil_bank_update(G, vel, 0.95, 0.85, 0.4385, en, st.beta2,
                                                      pb, mt, st.eff_wd, lr))

    def snapshot(state):
        return [t.view(torch.uint8).cpu().numpy().copy() for t in state]

    a = fresh()
    straight = []
    for G in grads:
        straight.append((step(a, G), snapshot(a)))
    b = fresh()
    for G in grads[:2]:
        step(b, G)
    saved = snapshot(b)
    del b
    gpu_lib.release_workspaces()
    dtypes = (torch.float32, torch.bfloat16, torch.int16, torch.float32)
    shapes = ((2, g, m, n), (g, m, n), (g, m, n), tuple(st.lane_energy.shape))
    c = tuple(torch.from_numpy(s).cuda().view(dt).reshape(sh)
              for s, dt, sh in zip(saved, dtypes, shapes))
    for k in (2, 3):
        u = step(c, grads[k])
        assert np.array_equal(u, straight[k][0]), f"update at step {k}"
        for got, want in zip(snapshot(c), straight[k][1]):
            assert np.array_equal(got, want), f"state at step {k}"
