"""Benchmark of the ANVIL bank step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload mlp|qk|vo|vs|us|single_wide] [--all]
                    [--no-cpu-baseline] [--copy-calibration BYTES]

A step is one anvil_bank_step call over the whole stack (momentum, normalisation and the six
Gram / polynomial / apply maps) on a gradient already resident in HBM.  The default workload is
the 24 x 2816 x 768 mlp bank.  One JSON line goes to stdout; --all adds one line per workload
(to stderr, so the first stdout line stays the contract line).

Roofline: the dominant kernel is the apply GEMM (61% of the cascade's flops on the mlp bank).
`achieved` = algorithmic flops of one launch / its average duration over 20 back-to-back launches
between HIP events on the one stream (the duration rocprofv3 reports for those launches).  The
step's own launch sequence is also replayed through the stage entry points with a HIP event
between every two launches (`in_step_us`, which includes each kernel's dispatch gap); the
cascade's share of peak (`cascade_pct_bf16_peak`) and `achieved_in_step` come from it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ANVIL bank-step matrices/s + TFLOP/s (% bf16 MFMA peak), 24×2816×768 mlp bank"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published


def flops(g, m, n):
    """Algorithmic flops of one bank step (symmetric halves of A and B not counted).

    Per matrix and map: Gram s(s+1)L, polynomial s^2(s+1), apply 2 s^2 L; six maps."""
    s, L = min(m, n), max(m, n)
    gram = s * (s + 1) * L
    poly = s * s * (s + 1)
    apply = 2 * s * s * L
    dense = 2 * s * s * L + 2 * s * s * s + 2 * s * s * L   # full Gram and full A*A
    return {"gram": 6 * g * gram, "poly": 6 * g * poly, "apply": 6 * g * apply,
            "total": 6 * g * (gram + poly + apply), "dense": 6 * g * dense}


def momentum_bytes(g, m, n):
    return 22 * g * m * n


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "apply_mlp_24x2816x768_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "orthogonalizing_polynomial_cascade_amd", "csrc", "gemm.hip")


def measured_apply_traffic():
    """HBM bytes per apply launch on the mlp bank from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of known size), or None when the GEMM
    source has changed since the counters were taken."""
    import hashlib
    try:
        fields = dict(l.split(": ", 1) for l in open(TRAFFIC_PROFILE).read().splitlines()
                      if l.startswith(("traffic_bytes_per_launch: ", "gemm_source_sha256_16: ")))
        digest = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    if fields.get("gemm_source_sha256_16", "").strip() != digest:
        return None
    return int(fields["traffic_bytes_per_launch"])


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_bank_step(anvil, w, steps, warmup):
    import torch
    g, m, n = w.g, w.m, w.n
    dev = torch.device("cuda:0")
    G = torch.from_numpy(w.grad(w.measured[0])).to(dev)
    vel = torch.zeros((2, g, m, n), dtype=torch.float32, device=dev)
    out = torch.empty((g, m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(anvil.workspace_bytes(g, m, n), dtype=torch.uint8, device=dev)
    mu, fb, fw = anvil.rail_scalars(w.step_ids[w.measured[0]])
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        anvil.anvil_bank_step(G, vel, mu, fb, fw, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = _events()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        anvil.anvil_bank_step(G, vel, mu, fb, fw, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    return ms, wall, (G, vel, out)


def time_bank_step_graph(anvil, w, steps):
    """The bank step (caller workspace: nothing allocated) captured once into a HIP graph and
    replayed `steps` times: ms per step without the host's per-launch cost."""
    import torch
    g, m, n = w.g, w.m, w.n
    dev = torch.device("cuda:0")
    G = torch.from_numpy(w.grad(w.measured[0])).to(dev)
    vel = torch.zeros((2, g, m, n), dtype=torch.float32, device=dev)
    out = torch.empty((g, m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(anvil.workspace_bytes(g, m, n), dtype=torch.uint8, device=dev)
    mu, fb, fw = anvil.rail_scalars(w.step_ids[w.measured[0]])

    def call():
        anvil.anvil_bank_step(G, vel, mu, fb, fw, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = _events()
    e0.record(stream)
    for _ in range(steps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def step_percentiles(anvil, w, steps=100):
    """Median, p10 and p90 of single bank steps (HIP events around each call), after the timed
    region of the headline, on the same inputs."""
    import torch
    g, m, n = w.g, w.m, w.n
    dev = torch.device("cuda:0")
    G = torch.from_numpy(w.grad(w.measured[0])).to(dev)
    vel = torch.zeros((2, g, m, n), dtype=torch.float32, device=dev)
    out = torch.empty((g, m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(anvil.workspace_bytes(g, m, n), dtype=torch.uint8, device=dev)
    mu, fb, fw = anvil.rail_scalars(w.step_ids[w.measured[0]])
    stream = torch.cuda.current_stream()
    ev = [_events() for _ in range(steps)]
    for _ in range(5):
        anvil.anvil_bank_step(G, vel, mu, fb, fw, out=out, workspace=ws, stream=stream)
    for e0, e1 in ev:
        e0.record(stream)
        anvil.anvil_bank_step(G, vel, mu, fb, fw, out=out, workspace=ws, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    t = np.sort([e0.elapsed_time(e1) for e0, e1 in ev])
    return {"p10": float(np.percentile(t, 10)), "p50": float(np.median(t)),
            "p90": float(np.percentile(t, 90)), "steps": steps}


def update_tensors(anvil, w):
    import torch
    from orthogonalizing_polynomial_cascade_amd import workloads
    st = workloads.update_state(w)
    dev = torch.device("cuda:0")
    pb = torch.from_numpy(st.param_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    mt = torch.from_numpy(st.mantissa.view(np.int16)).to(dev)
    en = torch.from_numpy(st.lane_energy).to(dev)
    lr = torch.from_numpy(st.eff_lr).to(dev)
    return st, pb, mt, en, lr


def time_bank_update(anvil, w, steps, warmup):
    """The whole bank update (step, equalizer, decay) and its tail kernels alone."""
    import torch
    g, m, n = w.g, w.m, w.n
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    G = torch.from_numpy(w.grad(w.measured[0])).to(dev)
    vel = torch.zeros((2, g, m, n), dtype=torch.float32, device=dev)
    out = torch.empty((g, m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(anvil.workspace_bytes(g, m, n), dtype=torch.uint8, device=dev)
    st, pb, mt, en, lr = update_tensors(anvil, w)
    mu, fb, fw = anvil.rail_scalars(w.step_ids[w.measured[0]])

    def upd():
        anvil.anvil_bank_update(G, vel, mu, fb, fw, en, st.beta2, pb, mt, st.eff_wd, lr,
                                update=out, workspace=ws, stream=stream)

    for _ in range(warmup):
        upd()
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record(stream)
    for _ in range(steps):
        upd()
    e1.record(stream)
    torch.cuda.synchronize()
    res = {"ms_per_update": e0.elapsed_time(e1) / steps}
    lanes = anvil.equalizer_lanes(m, n)
    scratch = torch.empty(2 * g * lanes, dtype=torch.float32, device=dev)
    gate = vel[1]
    reps = 20
    for name, fn in (("equalize", lambda: anvil.anvil_equalize(out, en, 1.0, scratch, stream=stream)),
                     ("decay", lambda: anvil.anvil_decay_update(pb, mt, out, st.eff_wd, lr, gate,
                                                                stream=stream))):
        fn()
        torch.cuda.synchronize()
        e0, e1 = _events()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[f"{name}_us"] = e0.elapsed_time(e1) / reps * 1e3
    return res


def time_contract(anvil, w, steps, warmup):
    """The whole update in the page's bank contract: bf16 gradient, device scalars, fixed buffers,
    captured once into a HIP graph and replayed; against the same call made eagerly."""
    import torch
    g, m, n = w.g, w.m, w.n
    dev = torch.device("cuda:0")
    G = torch.from_numpy(w.grad(w.measured[0])).to(dev).to(torch.bfloat16)
    vel = torch.zeros((2, g, m, n), dtype=torch.float32, device=dev)
    out = torch.empty((g, m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(anvil.workspace_bytes(g, m, n), dtype=torch.uint8, device=dev)
    st, pb, mt, en, lr = update_tensors(anvil, w)
    mu, fb, fw = anvil.rail_scalars(w.step_ids[w.measured[0]])
    scal = torch.tensor([mu, fb, fw, st.eff_wd], dtype=torch.float32, device=dev)

    def call():
        anvil.anvil_bank_update_dev(G, vel, scal, out, en, st.beta2, pb, mt, lr, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(1, warmup)):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    res = {}
    for name, fn in (("eager", call), ("graph", graph.replay)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = _events()
        stream = torch.cuda.current_stream()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[f"{name}_ms_per_update"] = e0.elapsed_time(e1) / steps
    return res


def time_stages(anvil, w, reps=20):
    """Average duration of each stage kernel (HIP events around `reps` launches on one stream)."""
    import torch
    g, m, n = w.g, w.m, w.n
    s = min(m, n)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    G = torch.from_numpy(w.grad(w.measured[0])).to(dev)
    vel = torch.zeros((2, g, m, n), dtype=torch.float32, device=dev)
    x = anvil.anvil_momentum(G, vel, 0.95, 0.85, 1.0)
    a, parts = anvil.anvil_gram(x, want_trace=True)
    anvil.anvil_normalize(x, a, parts)
    b = anvil.anvil_poly(a, -6.095026865488, 3.905234618423)
    c = torch.empty_like(x)
    xs = torch.empty_like(x)
    split = m > 1024
    res = {}

    def timed(name, fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = _events()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / reps * 1e3   # microseconds per launch

    timed("momentum", lambda: anvil.anvil_momentum(G, vel, 0.95, 0.85, 1.0, x_out=xs, stream=stream))
    timed("gram", lambda: anvil.anvil_gram(x, a_out=a, stream=stream))
    timed("poly", lambda: anvil.anvil_poly(a, -3.3, 0.99, b_out=b, stream=stream))
    timed("apply", lambda: anvil.anvil_apply(x, b, 3.2, split, c_out=c, stream=stream))
    return res


def time_library_products(w, reps=20):
    """Context for the GEMM kernels: torch.bmm (hipBLASLt) on the same bf16 products with fp32
    accumulation and bf16 output, but without the fused epilogues and computing the symmetric
    products in full: the apply's X·B (tall) or B·X (wide), the Gram's full XᵀX or XXᵀ, and A·A.
    Every operand is contiguous.  Microseconds per launch (HIP events around `reps` launches)."""
    import torch
    g, m, n = w.g, w.m, w.n
    s = min(m, n)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    x = torch.randn((g, m, n), generator=gen, device=dev).to(torch.bfloat16)
    xt = x.transpose(1, 2).contiguous()
    sq = torch.randn((g, s, s), generator=gen, device=dev).to(torch.bfloat16)
    tall = m > n
    prods = {
        "apply_product": (x, sq) if tall else (sq, x),
        "gram_full_product": (xt, x) if tall else (x, xt),
        "poly_full_product": (sq, sq),
    }
    stream = torch.cuda.current_stream()
    res = {}
    for name, (p, q) in prods.items():
        out = torch.bmm(p, q)
        torch.cuda.synchronize()
        e0, e1 = _events()
        e0.record(stream)
        for _ in range(reps):
            torch.bmm(p, q, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / reps * 1e3
    return res


# The six (a, b, c) maps of the cascade, as the library applies them (for the staged replay).
ANVIL_MAPS = (
    (3.923798038567, -6.095026865488, 3.905234618423),
    (3.278126713798, -3.328923386476, 0.989127286973),
    (3.505298394150, -5.137358782410, 1.968325560615),
    (2.815058591845, -3.685181239622, 1.417196497642),
    (2.245503932403, -2.443826979899, 0.963091710461),
    (2.256537145403, -2.166840097229, 0.929501253245),
)


def time_step_kernels(anvil, w, reps=20, warmup=2):
    """Per-kernel durations inside the step: the bank step's own launch sequence (momentum, first
    Gram with trace, normalisation, then Gram / polynomial / apply per map, ping-ponging X) made
    through the stage entry points, which launch the same kernels, with a HIP event between every
    two launches on the one stream.  Returns the mean duration (microseconds) of each kernel kind
    and of the whole staged step."""
    import torch
    g, m, n = w.g, w.m, w.n
    s = min(m, n)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    G = torch.from_numpy(w.grad(w.measured[0])).to(dev)
    vel = torch.zeros((2, g, m, n), dtype=torch.float32, device=dev)
    X = torch.empty((g, m, n), dtype=torch.bfloat16, device=dev)
    Y = torch.empty_like(X)
    A = torch.empty((g, s, s), dtype=torch.bfloat16, device=dev)
    B = torch.empty_like(A)
    parts = torch.empty((g, anvil.trace_slots(m, n)), dtype=torch.float32, device=dev)
    d = torch.empty((g,), dtype=torch.float32, device=dev)
    mu, fb, fw = anvil.rail_scalars(w.step_ids[w.measured[0]])
    split = m > 1024

    def staged(events):
        x, y = X, Y
        seq = [("momentum", lambda: anvil.anvil_momentum(G, vel, mu, fb, fw, x_out=x, stream=stream)),
               ("gram", lambda: anvil.anvil_gram(x, a_out=A, trace_partials=parts, stream=stream)),
               ("normalize", lambda: anvil.anvil_normalize(x, A, parts, d_out=d, stream=stream))]
        for name, fn in seq:
            fn()
            events.append((name, torch.cuda.Event(enable_timing=True)))
            events[-1][1].record(stream)
        for k, (a, b, c) in enumerate(ANVIL_MAPS):
            if k > 0:
                anvil.anvil_gram(x, a_out=A, stream=stream)
                events.append(("gram", torch.cuda.Event(enable_timing=True)))
                events[-1][1].record(stream)
            anvil.anvil_poly(A, b, c, b_out=B, stream=stream)
            events.append(("poly", torch.cuda.Event(enable_timing=True)))
            events[-1][1].record(stream)
            anvil.anvil_apply(x, B, a, split, c_out=y, stream=stream)
            events.append(("apply", torch.cuda.Event(enable_timing=True)))
            events[-1][1].record(stream)
            x, y = y, x

    for _ in range(warmup):
        staged([])
    torch.cuda.synchronize()
    runs = []
    for _ in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        ev = [("start", start)]
        staged(ev)
        runs.append(ev)
    torch.cuda.synchronize()
    acc, cnt, total = {}, {}, 0.0
    for ev in runs:
        for (_, e0), (name, e1) in zip(ev[:-1], ev[1:]):
            t = e0.elapsed_time(e1) * 1e3
            acc[name] = acc.get(name, 0.0) + t
            cnt[name] = cnt.get(name, 0) + 1
        total += ev[0][1].elapsed_time(ev[-1][1]) * 1e3
    res = {k: acc[k] / cnt[k] for k in acc}
    res["staged_step"] = total / len(runs)
    return res


def cpu_baseline(w, budget_s=15.0):
    """The oracle on a bounded sample of the same workload: whole bank steps of single matrices
    until about budget_s of CPU time, reported as matrices/s."""
    from oracle import anvil_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    G = w.grad(w.measured[0], g=1)
    v = np.zeros((2,) + G.shape, np.float32)
    mu, fb, fw = 0.95, 0.85, 1.0
    done, t0 = 0, time.perf_counter()
    while True:
        O.bank_step(G, v, mu, fb, fw)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or done >= 64:
            break
    return {"value": done / el, "unit": "matrices/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} single-matrix bank steps ({w.m}x{w.n}, numpy fp64 products with "
                      f"bf16 rounding emulation), {el:.1f} s"}


def run_workload(anvil, name, steps, warmup, with_stages=True, share=1):
    from orthogonalizing_polynomial_cascade_amd import workloads
    w = workloads.ALL[name]()
    if share > 1:
        # one GPU's part of the bank when whole matrices are spread over `share` GPUs
        w = workloads.scaled(w, g=-(-w.g // share))
    ms, wall, _ = time_bank_step(anvil, w, steps, warmup)
    f = flops(w.g, w.m, w.n)
    rec = {
        "workload": name, "g": w.g, "m": w.m, "n": w.n,
        "ms_per_step": ms, "matrices_per_s": w.g / (ms * 1e-3),
        "tflops": f["total"] / (ms * 1e-3) / 1e12,
        "wall_s": wall,
    }
    rec["pct_bf16_peak"] = 100.0 * rec["tflops"] / PEAK_BF16_TFLOPS
    if with_stages:
        st = time_stages(anvil, w)
        rec["stage_us"] = st
        rec["momentum_gbs"] = momentum_bytes(w.g, w.m, w.n) / (st["momentum"] * 1e-6) / 1e9
        rec["momentum_pct_hbm"] = 100.0 * rec["momentum_gbs"] / PEAK_HBM_GBS
        for k in ("gram", "poly", "apply"):
            rec[f"{k}_tflops"] = f[k] / 6 / (st[k] * 1e-6) / 1e12
            rec[f"{k}_pct_bf16_peak"] = 100.0 * rec[f"{k}_tflops"] / PEAK_BF16_TFLOPS
        # the cascade alone: the algorithmic flops over six maps' worth of the three GEMMs, with
        # the kernels timed alone in back-to-back loops ...
        cascade_s = 6 * (st["gram"] + st["poly"] + st["apply"]) * 1e-6
        rec["cascade_tflops_stage_loops"] = (f["gram"] + f["poly"] + f["apply"]) / cascade_s / 1e12
        # ... and inside the step's own launch sequence (the figure the cascade target is read on)
        ins = time_step_kernels(anvil, w)
        rec["in_step_us"] = ins
        cascade_s = 6 * (ins["gram"] + ins["poly"] + ins["apply"]) * 1e-6
        rec["cascade_tflops"] = (f["gram"] + f["poly"] + f["apply"]) / cascade_s / 1e12
        rec["cascade_pct_bf16_peak"] = 100.0 * rec["cascade_tflops"] / PEAK_BF16_TFLOPS
        for k in ("gram", "poly", "apply"):
            rec[f"{k}_in_step_tflops"] = f[k] / 6 / (ins[k] * 1e-6) / 1e12
        rec["momentum_in_step_gbs"] = momentum_bytes(w.g, w.m, w.n) / (ins["momentum"] * 1e-6) / 1e9
    rec["dense_equiv_tflops"] = f["dense"] / (ms * 1e-3) / 1e12
    gms = time_bank_step_graph(anvil, w, steps)
    rec["graph_ms_per_step"] = gms
    rec["graph_matrices_per_s"] = w.g / (gms * 1e-3)
    return w, rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mlp")
    ap.add_argument("--all", action="store_true", help="also report every workload (stderr)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--share", type=int, default=1, metavar="K",
                    help="time one GPU's share of the bank split by whole matrices over K GPUs "
                         "(ceil(g/K) matrices) instead of the whole bank")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes three times (the reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the ANVIL bank step runs on a single GPU and has no "
              "cross-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.share < 1:
        print("--share must be at least 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from orthogonalizing_polynomial_cascade_amd import anvil
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 * n, "launches": 3}), flush=True)
        return
    anvil.load()

    w, rec = run_workload(anvil, args.workload, args.steps, args.warmup, share=args.share)
    f = flops(w.g, w.m, w.n)
    apply_flops = f["apply"] / 6
    # kernel duration: the apply launched back to back (agrees with rocprofv3's duration of the
    # same launches); inside the step's launch sequence each event-bracketed duration also holds
    # the dispatch gap before the kernel, so that figure is reported beside it
    achieved = apply_flops / (rec["stage_us"]["apply"] * 1e-6) / 1e12
    achieved_in_step = apply_flops / (rec["in_step_us"]["apply"] * 1e-6) / 1e12
    metric = METRIC
    if w.name != "mlp" or args.share != 1:
        metric = (f"ANVIL bank-step matrices/s + TFLOP/s (% bf16 MFMA peak), "
                  f"{w.g}\u00d7{w.m}\u00d7{w.n} {w.name} bank"
                  + ("" if args.share == 1 else f" (1/{args.share} share)"))
    line = {
        "metric": metric,
        "value": rec["matrices_per_s"],
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} bank {w.g}x{w.m}x{w.n} (fp32 grads, fp32 rails, "
                               f"bf16 cascade, 6 maps)", "g": w.g, "m": w.m, "n": w.n,
                   "parallelism": "single GPU" if args.share == 1 else
                   f"one GPU's share of the bank split by whole matrices over {args.share} GPUs"},
        "tflops": rec["tflops"],
        "pct_bf16_peak": rec["pct_bf16_peak"],
        "stage_us": rec["stage_us"],
        "momentum_gbs": rec["momentum_gbs"],
        "momentum_pct_hbm": 100.0 * rec["momentum_gbs"] / PEAK_HBM_GBS,
        "in_step_us": rec["in_step_us"],
        "momentum_in_step_gbs": rec["momentum_in_step_gbs"],
        "cascade_tflops": rec["cascade_tflops"],
        "cascade_pct_bf16_peak": rec["cascade_pct_bf16_peak"],
        "cascade_tflops_stage_loops": rec["cascade_tflops_stage_loops"],
        "dense_equiv_tflops": rec["dense_equiv_tflops"],
        "step_ms_percentiles": step_percentiles(anvil, w),
        "graph_ms_per_step": rec["graph_ms_per_step"],
        "gram_tflops": rec["gram_in_step_tflops"],
        "poly_tflops": rec["poly_in_step_tflops"],
        "apply_tflops": rec["apply_in_step_tflops"],
        "stage_loop_tflops": {k: rec[f"{k}_tflops"] for k in ("gram", "poly", "apply")},
        "roofline": {"bound": "mfma", "kernel": "tall apply (gemm_kernel<3>)", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "achieved_in_step": achieved_in_step,
                     "frac_in_step": achieved_in_step / PEAK_BF16_TFLOPS,
                     "traffic": measured_apply_traffic() if w.name == "mlp" else None,
                     "traffic_unit": "bytes per launch",
                     "algorithmic_bytes": 2 * w.g * (2 * w.m * w.n + min(w.m, w.n) ** 2),
                     "flops_per_launch": apply_flops},
    }
    # the vendor library on the same products, for context (not part of the step)
    lib = time_library_products(w)
    line["library_bmm_us"] = dict(lib, note="torch.bmm (hipBLASLt), bf16 in and out, fp32 "
                                  "accumulation, full products without the fused epilogues")
    # the rest of the bank update (equalizer and decay) on the same workload, timed after the
    # headline step; its tail is HBM-bound at 18 bytes per element (lane powers read the update,
    # the fused rescale-and-decay pass moves 16)
    u = time_bank_update(anvil, w, max(10, args.steps // 2), args.warmup)
    count = w.g * w.m * w.n
    tail_ms = u["ms_per_update"] - rec["ms_per_step"]
    line["bank_update"] = {
        "ms_per_update": u["ms_per_update"],
        "matrices_per_s": w.g / (u["ms_per_update"] * 1e-3),
        "tail_us": tail_ms * 1e3,
        "tail_gbs": 18 * count / (tail_ms * 1e-3) / 1e9 if tail_ms > 0 else None,
        "equalize_us": u["equalize_us"], "equalize_gbs": 6 * count / (u["equalize_us"] * 1e-6) / 1e9,
        "decay_us": u["decay_us"], "decay_gbs": 14 * count / (u["decay_us"] * 1e-6) / 1e9,
    }
    # the page's bank contract: bf16 gradient, device scalars, one graph replay per update
    c = time_contract(anvil, w, max(10, args.steps // 2), args.warmup)
    line["bank_update"]["bf16_grad_device_scalars"] = c
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)
    if args.all:
        for name in ("single_wide", "qk", "vo", "mlp", "vs", "us"):
            _, r = run_workload(anvil, name, max(10, args.steps // 2), args.warmup)
            print(json.dumps(r), file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
