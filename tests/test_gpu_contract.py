"""The page's bank contract (anvil.py, `AnvilBank`, `anvil_bank_update`): a bf16 gradient, per-step
scalars held on the device, fixed buffers and a caller workspace, and capture of the whole update
into a HIP graph replayed with new gradients and scalars.

Every comparison here is bit-exact: the device-scalar entry points run the same kernels as the
by-value ones, and a bf16 gradient is widened to fp32 exactly before the first lerp, so it must
give what the fp32 entry point gives on the widened values."""
import numpy as np
import pytest

from oracle import anvil_oracle as O
from orthogonalizing_polynomial_cascade_amd import workloads as W
from tests.helpers import bf16_bits_of, from_gpu, to_gpu_f32

pytestmark = pytest.mark.gpu

SHAPES = [(3, 200, 328), (3, 392, 136), (2, 264, 264), (2, 1096, 136)]


def _state(gpu_lib, g, m, n, seed=1):
    import torch
    w = W.gaussian(g, m, n, seed=seed)
    st = W.update_state(w)
    dev = "cuda"
    return dict(
        vel=torch.zeros((2, g, m, n), dtype=torch.float32, device=dev),
        param=torch.from_numpy(st.param_bits.view(np.int16).copy()).to(dev).view(torch.bfloat16),
        mant=torch.from_numpy(st.mantissa.view(np.int16).copy()).to(dev),
        energy=torch.from_numpy(st.lane_energy.copy()).to(dev),
        lr=torch.from_numpy(st.eff_lr.copy()).to(dev),
        wd=st.eff_wd, beta2=st.beta2,
        ws=torch.empty(gpu_lib.workspace_bytes(g, m, n), dtype=torch.uint8, device=dev),
        out=torch.empty((g, m, n), dtype=torch.bfloat16, device=dev))


def _snapshot(s):
    return [bf16_bits_of(s["out"]), from_gpu(s["vel"]).view(np.uint32), from_gpu(s["energy"]),
            bf16_bits_of(s["param"]), s["mant"].cpu().numpy()]


def _same(a, b):
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("g,m,n", SHAPES)
def test_bf16_gradient_and_device_scalars(gpu_lib, g, m, n):
    """bf16 gradient + device scalars == fp32 entry point on the widened gradient; the rails are
    the oracle's (bit-exact) on the widened values."""
    import torch
    G32 = W.gaussian(g, m, n, seed=2).grad(0)
    Gw = O.R(G32)                                   # the bf16 gradient's values
    Gb = torch.from_numpy(Gw).cuda().to(torch.bfloat16)
    a, b = _state(gpu_lib, g, m, n), _state(gpu_lib, g, m, n)
    for t, fw in enumerate((1.0, 0.4385)):
        scal = torch.tensor([0.95, 0.85, fw], dtype=torch.float32, device="cuda")
        gpu_lib.anvil_bank_step_dev(Gb, a["vel"], scal, a["out"], a["ws"])
        gpu_lib.anvil_bank_step(to_gpu_f32(Gw), b["vel"], 0.95, 0.85, fw, out=b["out"],
                                workspace=b["ws"])
        assert np.array_equal(bf16_bits_of(a["out"]), bf16_bits_of(b["out"]))
        assert torch.equal(a["vel"], b["vel"])
    v = np.zeros((2, g, m, n), np.float32)
    for fw in (1.0, 0.4385):
        v, _ = O.momentum_step(Gw, v, 0.95, 0.85, fw)
    assert np.array_equal(from_gpu(a["vel"]).view(np.uint32), v.view(np.uint32))


@pytest.mark.parametrize("g,m,n", SHAPES)
@pytest.mark.parametrize("bf16_grad", [False, True])
def test_update_dev_equals_update(gpu_lib, g, m, n, bf16_grad):
    import torch
    G = O.R(W.gaussian(g, m, n, seed=4).grad(0)) if bf16_grad else W.gaussian(g, m, n, seed=4).grad(0)
    Gd = to_gpu_f32(G)
    Gdev = Gd.to(torch.bfloat16) if bf16_grad else Gd
    a, b = _state(gpu_lib, g, m, n), _state(gpu_lib, g, m, n)
    scal = torch.tensor([0.95, 0.85, 0.4385, a["wd"]], dtype=torch.float32, device="cuda")
    for _ in range(2):
        gpu_lib.anvil_bank_update_dev(Gdev, a["vel"], scal, a["out"], a["energy"], a["beta2"],
                                      a["param"], a["mant"], a["lr"], a["ws"])
        gpu_lib.anvil_bank_update(Gd, b["vel"], 0.95, 0.85, 0.4385, b["energy"], b["beta2"],
                                  b["param"], b["mant"], b["wd"], b["lr"], update=b["out"],
                                  workspace=b["ws"])
        torch.cuda.synchronize()
        _same(_snapshot(a), _snapshot(b))


def test_graph_capture_replays_match_eager(gpu_lib):
    """Capture one whole update into a graph; replay it over five steps that cross the engage
    step (the blend weight and momentum change through the device scalars), with new gradients
    copied into the fixed gradient buffer, eager work and synchronisation between replays; every
    replay must equal the same call made eagerly on a twin state."""
    import torch
    g, m, n = 3, 392, 136
    w = W.scaled(W.mlp_bank(), g=g, m=m, n=n)
    grads = [torch.from_numpy(O.R(w.grad(t, g=g))).cuda().to(torch.bfloat16) for t in range(5)]
    cap, eag = _state(gpu_lib, g, m, n), _state(gpu_lib, g, m, n)
    gbuf = torch.empty_like(grads[0])
    sc_cap = torch.zeros(4, dtype=torch.float32, device="cuda")
    sc_eag = torch.zeros(4, dtype=torch.float32, device="cuda")
    sched = [(0.95, 0.85, 1.0 if step < 514 else 0.4385, cap["wd"]) for step in (511, 512, 513, 514, 515)]

    def call(s, sc, grad):
        gpu_lib.anvil_bank_update_dev(grad, s["vel"], sc, s["out"], s["energy"], s["beta2"],
                                      s["param"], s["mant"], s["lr"], s["ws"])

    # warm-up outside capture on a scratch twin (sets kernel attributes), as graph capture needs
    warm = _state(gpu_lib, g, m, n)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sc_cap.copy_(torch.tensor(sched[0], dtype=torch.float32))
        gbuf.copy_(grads[0])
        call(warm, sc_cap, gbuf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(cap, sc_cap, gbuf)
    torch.cuda.synchronize()

    for t in range(5):
        sc_cap.copy_(torch.tensor(sched[t], dtype=torch.float32))
        gbuf.copy_(grads[t])
        graph.replay()
        torch.cuda.synchronize()
        sc_eag.copy_(torch.tensor(sched[t], dtype=torch.float32))
        call(eag, sc_eag, grads[t])
        torch.cuda.synchronize()
        _same(_snapshot(cap), _snapshot(eag))


@pytest.mark.parametrize("wname", ["mlp", "us"])
def test_bf16_gradient_full_size(gpu_lib, wname):
    """Full stack, benchmark configuration: the bf16-gradient, device-scalar step equals the fp32
    entry point on the widened gradient bit-exactly (rails and update)."""
    import torch
    w = W.ALL[wname]()
    g, m, n = w.g, w.m, w.n
    Gw = O.R(w.grad(w.measured[0]))
    Gb = torch.from_numpy(Gw).cuda().to(torch.bfloat16)
    mu, fb, fw = gpu_lib.rail_scalars(w.step_ids[w.measured[0]])
    a, b = _state(gpu_lib, g, m, n), _state(gpu_lib, g, m, n)
    scal = torch.tensor([mu, fb, fw], dtype=torch.float32, device="cuda")
    gpu_lib.anvil_bank_step_dev(Gb, a["vel"], scal, a["out"], a["ws"])
    gpu_lib.anvil_bank_step(to_gpu_f32(Gw), b["vel"], mu, fb, fw, out=b["out"], workspace=b["ws"])
    assert np.array_equal(bf16_bits_of(a["out"]), bf16_bits_of(b["out"]))
    assert torch.equal(a["vel"], b["vel"])


def test_cached_workspace_refuses_capture(gpu_lib):
    """The entry points without a workspace may allocate and synchronise, so on a capturing stream
    they return ANVIL_ERR_CAPTURING and enqueue nothing; the caller-workspace form of the same
    call captures and replays normally."""
    import torch
    g, m, n = 2, 200, 328
    G = torch.randn((g, m, n), dtype=torch.float32, device="cuda")
    vel = torch.zeros((2, g, m, n), dtype=torch.float32, device="cuda")
    out = torch.empty((g, m, n), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gpu_lib.workspace_bytes(g, m, n), dtype=torch.uint8, device="cuda")
    # warm-up outside capture (kernel attributes are set on first launch)
    gpu_lib.anvil_bank_step(G, vel.clone(), 0.95, 0.85, 1.0, out=out, workspace=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        graph.capture_begin()
        try:
            with pytest.raises(gpu_lib.AnvilError) as err:
                gpu_lib.anvil_bank_step(G, vel, 0.95, 0.85, 1.0, out=out)
            assert err.value.status == gpu_lib.ANVIL_ERR_CAPTURING
            gpu_lib.anvil_bank_step(G, vel, 0.95, 0.85, 1.0, out=out, workspace=ws)
        finally:
            graph.capture_end()
    torch.cuda.synchronize()
    assert torch.equal(vel, torch.zeros_like(vel))      # nothing ran during capture
    v_ref = torch.zeros_like(vel)
    for _ in range(2):
        graph.replay()
        ref = gpu_lib.anvil_bank_step(G, v_ref, 0.95, 0.85, 1.0)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(vel, v_ref)
