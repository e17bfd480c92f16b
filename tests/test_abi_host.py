"""Host-side checks of the C ABI: the library loads, exports every symbol include/anvil.h declares,
and rejects bad arguments before any HIP call (so these run without a GPU).  Fake, never
dereferenced pointer values are used for the rejected calls."""
import ctypes
import os
import re

import pytest

from orthogonalizing_polynomial_cascade_amd import anvil

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "anvil.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(anvil_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return anvil.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) >= 13
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(anvil.SIGNATURES), set(names) ^ set(anvil.SIGNATURES)


def test_status_strings(lib):
    for code in range(9):
        s = lib.anvil_status_string(code)
        assert s and len(s) > 1
    assert lib.anvil_status_string(0) == b"ok"
    assert b"unknown" in lib.anvil_status_string(99)
    assert lib.anvil_version() >= 100
    assert lib.anvil_last_hip_error() == 0


A = 0x10000000      # fake, 256-byte aligned addresses far apart
B = 0x20000000
C = 0x30000000
W = 0x40000000


def _step(lib, grad=A, vel=B, out=C, g=2, m=64, n=32):
    return lib.anvil_bank_step(grad, vel, 0.95, 0.85, 1.0, out, g, m, n, None)


def _step_ws(lib, grad=A, vel=B, out=C, g=2, m=64, n=32, ws=W, wsb=1 << 30):
    return lib.anvil_bank_step_ws(grad, vel, 0.95, 0.85, 1.0, out, g, m, n, ws, wsb, None)


def test_empty_stack_is_a_noop(lib):
    for g, m, n in [(0, 64, 32), (2, 0, 32), (2, 64, 0)]:
        assert lib.anvil_bank_step(None, None, 0.95, 0.85, 1.0, None, g, m, n, None) == 0
        assert lib.anvil_gram(None, None, None, g, m, n, None) == 0
        assert lib.anvil_apply(None, None, None, 1.0, 0, g, m, n, None) == 0
    assert lib.anvil_workspace_bytes(0, 64, 32) == 0


def test_invalid_arguments(lib):
    assert _step(lib, g=-1) == anvil.ANVIL_ERR_INVALID_ARG
    assert _step(lib, m=-8) == anvil.ANVIL_ERR_INVALID_ARG
    assert _step(lib, grad=None) == anvil.ANVIL_ERR_INVALID_ARG
    assert _step(lib, vel=None) == anvil.ANVIL_ERR_INVALID_ARG
    assert _step(lib, out=None) == anvil.ANVIL_ERR_INVALID_ARG
    assert _step_ws(lib, ws=None) == anvil.ANVIL_ERR_INVALID_ARG
    assert lib.anvil_apply(A, B, C, 1.0, 2, 1, 64, 32, None) == anvil.ANVIL_ERR_INVALID_ARG
    assert lib.anvil_normalize(A, B, None, None, 1, 64, 32, None) == anvil.ANVIL_ERR_INVALID_ARG


def test_unsupported_shapes(lib):
    assert _step(lib, m=60) == anvil.ANVIL_ERR_UNSUPPORTED
    assert _step(lib, n=30) == anvil.ANVIL_ERR_UNSUPPORTED
    assert _step(lib, g=70000) == anvil.ANVIL_ERR_UNSUPPORTED
    assert _step(lib, m=65536, n=32768) == anvil.ANVIL_ERR_UNSUPPORTED
    # one matrix may hold at most 2^30 elements (2 GiB of bf16)
    assert _step(lib, m=32768, n=32776) == anvil.ANVIL_ERR_UNSUPPORTED
    assert lib.anvil_workspace_bytes(1, 32768, 32768) > 0
    assert lib.anvil_workspace_bytes(1, 32768, 32776) == 0
    # whole stack at most 2^35 elements
    assert lib.anvil_workspace_bytes(32, 32768, 32768) > 0
    assert lib.anvil_workspace_bytes(33, 32768, 32768) == 0
    assert lib.anvil_workspace_bytes(65535, 32768, 32768) == 0
    assert lib.anvil_workspace_bytes(1, 60, 32) == 0
    need = lib.anvil_workspace_bytes(2, 64, 32)
    assert _step_ws(lib, wsb=need - 1) == anvil.ANVIL_ERR_UNSUPPORTED


def test_misaligned(lib):
    assert _step(lib, grad=A + 4) == anvil.ANVIL_ERR_MISALIGNED
    assert _step(lib, vel=B + 8) == anvil.ANVIL_ERR_MISALIGNED
    assert _step(lib, out=C + 2) == anvil.ANVIL_ERR_MISALIGNED
    assert _step_ws(lib, ws=W + 16) == anvil.ANVIL_ERR_MISALIGNED


def test_aliasing(lib):
    assert _step(lib, out=A) == anvil.ANVIL_ERR_ALIAS
    assert _step(lib, out=B + 64) == anvil.ANVIL_ERR_ALIAS
    assert _step(lib, vel=A + 256) == anvil.ANVIL_ERR_ALIAS
    assert _step_ws(lib, ws=C) == anvil.ANVIL_ERR_ALIAS
    assert lib.anvil_apply(A, B, A, 1.0, 0, 1, 64, 32, None) == anvil.ANVIL_ERR_ALIAS
    assert lib.anvil_apply(A, B, B, 1.0, 0, 1, 64, 32, None) == anvil.ANVIL_ERR_ALIAS
    assert lib.anvil_poly(A, A, 1.0, 1.0, 1, 64, None) == anvil.ANVIL_ERR_ALIAS
    assert lib.anvil_gram(A, A, None, 1, 64, 32, None) == anvil.ANVIL_ERR_ALIAS


def test_workspace_size_and_trace_slots(lib):
    g, m, n = 24, 2816, 768
    ws = lib.anvil_workspace_bytes(g, m, n)
    s = 768
    assert ws >= g * m * n * 2 + 2 * g * s * s * 2 + g * 4
    assert ws % 256 == 0
    assert lib.anvil_trace_slots(2816, 768) >= 1
    # one partial per diagonal tile of the Gram: 128x128 tiles, or 32x32 for Grams of at most
    # 256 rows read along the rows (wide and square matrices)
    assert lib.anvil_trace_slots(2816, 768) == 6
    assert lib.anvil_trace_slots(768, 256) == 2
    assert lib.anvil_trace_slots(256, 768) == 8
    assert lib.anvil_trace_slots(264, 264) == 3
    assert lib.anvil_trace_slots(7, 8) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    g = torch.zeros(1, 8, 8)
    with pytest.raises(ValueError):
        anvil.anvil_bank_step(g, torch.zeros(2, 1, 8, 8), 0.95, 0.85, 1.0)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError):
        anvil.load(str(tmp_path / "libanvil.so"))


D = 0x50000000
E = 0x60000000
F = 0x70000000
L = 0x80000000


def _upd(lib, grad=A, vel=B, out=C, energy=D, param=E, mant=F, lr=L, g=2, m=64, n=32):
    return lib.anvil_bank_update(grad, vel, 0.95, 0.85, 1.0, out, energy, 0.95, param, mant,
                                 0.01, lr, g, m, n, None)


def test_update_entry_points_reject_before_launching(lib):
    assert lib.anvil_equalizer_lanes(64, 32) == 64
    assert lib.anvil_equalizer_lanes(32, 64) == 64
    assert lib.anvil_equalizer_lanes(48, 48) == 48
    assert lib.anvil_equalizer_lanes(60, 32) == 0
    assert lib.anvil_bank_update(None, None, 0.95, 0.85, 1.0, None, None, 0.95, None, None, 0.0,
                                 None, 0, 64, 32, None) == 0
    assert lib.anvil_equalize(None, None, 0.95, None, 2, 0, 32, None) == 0
    assert lib.anvil_decay_update(None, None, None, 0.0, None, None, 0, 8, 8, None) == 0
    assert _upd(lib, energy=None) == anvil.ANVIL_ERR_INVALID_ARG
    assert _upd(lib, lr=None) == anvil.ANVIL_ERR_INVALID_ARG
    assert _upd(lib, g=-2) == anvil.ANVIL_ERR_INVALID_ARG
    assert _upd(lib, n=36) == anvil.ANVIL_ERR_UNSUPPORTED
    assert _upd(lib, param=E + 2) == anvil.ANVIL_ERR_MISALIGNED
    assert _upd(lib, mant=E) == anvil.ANVIL_ERR_ALIAS
    assert _upd(lib, energy=C + 64) == anvil.ANVIL_ERR_ALIAS
    assert _upd(lib, lr=F + 16) == anvil.ANVIL_ERR_ALIAS
    assert _upd(lib, param=B + 4096) == anvil.ANVIL_ERR_ALIAS
    need = lib.anvil_workspace_bytes(2, 64, 32)
    args = (A, B, 0.95, 0.85, 1.0, C, D, 0.95, E, F, 0.01, L, 2, 64, 32)
    assert lib.anvil_bank_update_ws(*args, W, need - 1, None) == anvil.ANVIL_ERR_UNSUPPORTED
    assert lib.anvil_bank_update_ws(*args, E, need, None) == anvil.ANVIL_ERR_ALIAS
    assert lib.anvil_bank_update_ws(*args, W + 64, need, None) == anvil.ANVIL_ERR_MISALIGNED
    assert lib.anvil_equalize(C, D, 0.95, D + 8, 2, 64, 32, None) == anvil.ANVIL_ERR_ALIAS
    assert lib.anvil_equalize(C + 2, D, 0.95, E, 2, 64, 32, None) == anvil.ANVIL_ERR_MISALIGNED
    assert lib.anvil_equalize(C, None, 0.95, E, 2, 64, 32, None) == anvil.ANVIL_ERR_INVALID_ARG
    assert lib.anvil_decay_update(E, F, C, 0.01, L, E, 2, 64, 32, None) == anvil.ANVIL_ERR_ALIAS
    assert lib.anvil_decay_update(E, F, C, 0.01, L, D + 4, 2, 64, 32, None) == \
        anvil.ANVIL_ERR_MISALIGNED
    assert lib.anvil_decay_update(E, F, C, 0.01, None, D, 2, 64, 32, None) == \
        anvil.ANVIL_ERR_INVALID_ARG


def test_workspace_covers_the_equalizer_scratch(lib):
    for g, m, n in [(24, 2816, 768), (24, 256, 768), (3, 8, 4096)]:
        lanes = lib.anvil_equalizer_lanes(m, n)
        base = g * m * n * 2 + 2 * g * min(m, n) ** 2 * 2
        assert lib.anvil_workspace_bytes(g, m, n) >= base + 2 * g * lanes * 4


def test_plain_c_consumer(lib, tmp_path):
    """tests/c_consumer.c, compiled as C11 by the host compiler against include/anvil.h alone and
    linked to libanvil.so, runs the host-side contract (status strings, workspace sizes, empty
    stacks, argument checks that reject a call before anything is launched) with no GPU."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.dirname(anvil.LIB_PATH)
    exe = str(tmp_path / "c_consumer")
    src = os.path.join(root, "tests", "c_consumer.c")
    r = subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-I",
                        os.path.join(root, "include"), src, "-L", pkg, "-lanvil",
                        f"-Wl,-rpath,{pkg}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_map_table_entry_point_checks(lib):
    table = (ctypes.c_float * 6)(3.0, -4.0, 2.0, 3.0, -4.0, 2.0)
    tp = ctypes.cast(table, ctypes.c_void_p)
    args = (A, B, 0.95, 0.85, 1.0)
    assert lib.anvil_bank_step_maps(*args, tp, 0, C, 2, 64, 32, None, 0, None) == \
        anvil.ANVIL_ERR_INVALID_ARG
    assert lib.anvil_bank_step_maps(*args, tp, 17, C, 2, 64, 32, None, 0, None) == \
        anvil.ANVIL_ERR_INVALID_ARG
    assert lib.anvil_bank_step_maps(*args, None, 2, C, 2, 64, 32, None, 0, None) == \
        anvil.ANVIL_ERR_INVALID_ARG
    assert lib.anvil_bank_step_maps(*args, tp, 2, C, 0, 64, 32, None, 0, None) == 0
    assert lib.anvil_bank_step_maps(*args, tp, 2, A, 2, 64, 32, None, 0, None) == \
        anvil.ANVIL_ERR_ALIAS
    need = lib.anvil_workspace_bytes(2, 64, 32)
    assert lib.anvil_bank_step_maps(*args, tp, 2, C, 2, 64, 32, W, need - 1, None) == \
        anvil.ANVIL_ERR_UNSUPPORTED
    assert lib.anvil_bank_step_maps(*args, tp, 2, C, 2, 64, 32, W + 32, need, None) == \
        anvil.ANVIL_ERR_MISALIGNED


def test_device_scalar_entry_points_checks(lib):
    need = lib.anvil_workspace_bytes(2, 64, 32)
    S = 0x90000000
    assert lib.anvil_bank_step_dev(A, 2, B, S, C, 2, 64, 32, W, need, None) == \
        anvil.ANVIL_ERR_INVALID_ARG                       # bad grad dtype
    assert lib.anvil_bank_step_dev(A, 1, B, None, C, 2, 64, 32, W, need, None) == \
        anvil.ANVIL_ERR_INVALID_ARG                       # no scalars
    assert lib.anvil_bank_step_dev(A, 1, B, S, C, 2, 64, 32, None, 0, None) == \
        anvil.ANVIL_ERR_INVALID_ARG                       # the workspace is required
    assert lib.anvil_bank_step_dev(A, 1, B, S + 2, C, 2, 64, 32, W, need, None) == \
        anvil.ANVIL_ERR_MISALIGNED
    assert lib.anvil_bank_step_dev(A, 1, B, C + 8, C, 2, 64, 32, W, need, None) == \
        anvil.ANVIL_ERR_ALIAS                             # scalars inside out
    # a bf16 gradient is half the bytes: `out` right after it passes the overlap checks (and the
    # call then stops at the too-small workspace); with an fp32 gradient it overlaps
    after = A + 2 * 64 * 32 * 2
    assert lib.anvil_bank_step_dev(A, 1, B, S, after, 2, 64, 32, W, need - 1, None) == \
        anvil.ANVIL_ERR_UNSUPPORTED
    assert lib.anvil_bank_step_ws(A, B, 0.95, 0.85, 1.0, after, 2, 64, 32, W, need - 1, None) == \
        anvil.ANVIL_ERR_ALIAS
    args = (A, 1, B, S, C, D, 0.95, E, F, L, 2, 64, 32)
    assert lib.anvil_bank_update_dev(*args, W, need - 1, None) == anvil.ANVIL_ERR_UNSUPPORTED
    assert lib.anvil_bank_update_dev(A, 1, B, E + 8, C, D, 0.95, E, F, L, 2, 64, 32, W, need,
                                     None) == anvil.ANVIL_ERR_ALIAS


def test_noalloc_refuses_oversized_banks_on_the_host(lib):
    """anvil_bank_step_noalloc checks its scratch limit before any HIP call: a bank needing more
    than ANVIL_NOALLOC_SCRATCH_BYTES is refused with ANVIL_ERR_TOO_LARGE (fake, disjoint
    addresses; nothing is dereferenced), the usual argument checks still come first."""
    far = [0x1000000000, 0x2000000000, 0x3000000000]
    g, m, n = 48, 2816, 768
    assert lib.anvil_workspace_bytes(g, m, n) > anvil.NOALLOC_SCRATCH_BYTES
    assert lib.anvil_workspace_bytes(24, m, n) <= anvil.NOALLOC_SCRATCH_BYTES
    assert lib.anvil_bank_step_noalloc(far[0], far[1], 0.95, 0.85, 1.0, far[2], g, m, n,
                                       None) == anvil.ANVIL_ERR_TOO_LARGE
    assert lib.anvil_bank_step_noalloc(far[0], far[1], 0.95, 0.85, 1.0, None, g, m, n,
                                       None) == anvil.ANVIL_ERR_INVALID_ARG
    assert lib.anvil_bank_step_noalloc(far[0], far[0], 0.95, 0.85, 1.0, far[2], 2, 64, 32,
                                       None) == anvil.ANVIL_ERR_ALIAS
    assert lib.anvil_bank_step_noalloc(None, None, 0.95, 0.85, 1.0, None, 0, 64, 32, None) == 0
    assert lib.anvil_status_string(anvil.ANVIL_ERR_TOO_LARGE).startswith(b"the bank step needs")
