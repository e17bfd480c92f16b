"""The bank step called from plain C (tests/c_bank_step.c: HIP runtime API for memory, the C ABI of
libanvil.so for the step, no torch or Python in the process) on seeded inputs: the rails must equal
the oracle's momentum bit for bit, the update must equal the Python binding's call on the same
input bit for bit (same kernels), and lie within the update bar of the oracle's cascade."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import anvil_oracle as O
from orthogonalizing_polynomial_cascade_amd import anvil
from orthogonalizing_polynomial_cascade_amd import workloads as W
from tests.helpers import from_gpu, to_gpu_f32, update_error

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def c_exe(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    pkg = os.path.dirname(anvil.LIB_PATH)
    exe = str(tmp_path_factory.mktemp("c") / "c_bank_step")
    r = subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
                        os.path.join(ROOT, "tests", "c_bank_step.c"), "-L", pkg, "-lanvil",
                        "-L", os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,{pkg}",
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("g,m,n", [(3, 392, 136), (2, 200, 328), (2, 1096, 136)])
def test_bank_step_from_c(gpu_lib, c_exe, tmp_path, g, m, n):
    import torch
    G = W.gaussian(g, m, n, seed=31).grad(0)
    mu, fb, fw = 0.95, 0.85, 1.0
    gfile, ofile, vfile = tmp_path / "grad.f32", tmp_path / "out.bf16", tmp_path / "vel.f32"
    G.astype(np.float32).tofile(gfile)
    print(f"c_bank_step {g}x{m}x{n}", flush=True)
    r = subprocess.run([c_exe, str(g), str(m), str(n), repr(mu), repr(fb), repr(fw), str(gfile),
                        str(ofile), str(vfile)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    out_bits = np.fromfile(ofile, dtype=np.uint16).reshape(g, m, n)
    vel = np.fromfile(vfile, dtype=np.float32).reshape(2, g, m, n)

    v_want, y = O.momentum_step(G, np.zeros((2, g, m, n), np.float32), mu, fb, fw)
    assert np.array_equal(vel.view(np.uint32), v_want.view(np.uint32))

    v_py = torch.zeros((2, g, m, n), dtype=torch.float32, device="cuda")
    out_py = gpu_lib.anvil_bank_step(to_gpu_f32(G), v_py, mu, fb, fw)
    py_bits = out_py.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(out_bits, py_bits)

    out = (out_bits.astype(np.uint32) << 16).view(np.float32)
    want = O.cascade(O.R(y))
    for i in range(g):
        assert update_error(out[i], want[i]) <= 1e-2, i
    assert np.array_equal(from_gpu(v_py).view(np.uint32), v_want.view(np.uint32))
