"""Host-side checks of bench.py's contract that need no GPU: a request for more than one GPU is
refused with a message before anything touches a device, and the algorithmic flop and byte counts
the roofline uses follow the per-map formulas (Gram s(s+1)L, polynomial s^2(s+1), apply 2 s^2 L,
six maps; momentum 22 bytes per element)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_share_must_be_positive():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--share", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--share" in r.stderr
    assert r.stdout == ""


def test_flop_and_byte_counts():
    sys.path.insert(0, ROOT)
    import bench
    g, m, n = 24, 2816, 768
    s, L = 768, 2816
    f = bench.flops(g, m, n)
    assert f["gram"] == 6 * g * s * (s + 1) * L
    assert f["poly"] == 6 * g * s * s * (s + 1)
    assert f["apply"] == 6 * g * 2 * s * s * L
    assert f["total"] == f["gram"] + f["poly"] + f["apply"]
    assert f["dense"] == 6 * g * (4 * s * s * L + 2 * s ** 3)   # full Gram and full A*A
    assert bench.flops(g, n, m) == f                  # wide is the transpose of tall
    assert bench.momentum_bytes(g, m, n) == 22 * g * m * n
