"""Python binding of libanvil.so (ctypes): argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks dtype, shape, device and
contiguity, and passes raw device pointers and the current HIP stream to the C ABI declared in
include/anvil.h.  All arithmetic happens in the library's HIP kernels; if the library is missing
the functions raise instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libanvil.so")

ANVIL_OK = 0
ANVIL_ERR_INVALID_ARG = 1
ANVIL_ERR_UNSUPPORTED = 2
ANVIL_ERR_MISALIGNED = 3
ANVIL_ERR_ALIAS = 4
ANVIL_ERR_OOM = 5
ANVIL_ERR_HIP = 6
ANVIL_ERR_CAPTURING = 7
ANVIL_ERR_TOO_LARGE = 8
NOALLOC_SCRATCH_BYTES = 192 << 20   # ANVIL_NOALLOC_SCRATCH_BYTES of include/anvil.h

ANVIL_GRAD_F32 = 0
ANVIL_GRAD_BF16 = 1

# Every symbol include/anvil.h declares, with its ctypes signature (restype, argtypes).
_vp, _i64, _f, _i, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
_d = ctypes.c_double
SIGNATURES = {
    "anvil_status_string": (ctypes.c_char_p, [_i]),
    "anvil_last_hip_error": (_i, []),
    "anvil_version": (_i, []),
    "anvil_bank_step": (_i, [_vp, _vp, _f, _f, _f, _vp, _i64, _i64, _i64, _vp]),
    "anvil_bank_step_ws": (_i, [_vp, _vp, _f, _f, _f, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "anvil_bank_step_noalloc": (_i, [_vp, _vp, _f, _f, _f, _vp, _i64, _i64, _i64, _vp]),
    "anvil_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "anvil_release_workspaces": (_i, []),
    "anvil_momentum": (_i, [_vp, _vp, _f, _f, _f, _vp, _i64, _i64, _i64, _vp]),
    "anvil_trace_slots": (_i64, [_i64, _i64]),
    "anvil_gram": (_i, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "anvil_normalize": (_i, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "anvil_poly": (_i, [_vp, _vp, _f, _f, _i64, _i64, _vp]),
    "anvil_apply": (_i, [_vp, _vp, _vp, _f, _i, _i64, _i64, _i64, _vp]),
    "anvil_bank_update": (_i, [_vp, _vp, _f, _f, _f, _vp, _vp, _d, _vp, _vp, _f, _vp,
                               _i64, _i64, _i64, _vp]),
    "anvil_bank_update_ws": (_i, [_vp, _vp, _f, _f, _f, _vp, _vp, _d, _vp, _vp, _f, _vp,
                                  _i64, _i64, _i64, _vp, _sz, _vp]),
    "anvil_equalizer_lanes": (_i64, [_i64, _i64]),
    "anvil_bank_step_dev": (_i, [_vp, _i, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "anvil_bank_update_dev": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _d, _vp, _vp, _vp, _i64, _i64,
                                   _i64, _vp, _sz, _vp]),
    "anvil_bank_step_maps": (_i, [_vp, _vp, _f, _f, _f, _vp, _i, _vp, _i64, _i64, _i64, _vp, _sz,
                                  _vp]),
    "anvil_equalize": (_i, [_vp, _vp, _d, _vp, _i64, _i64, _i64, _vp]),
    "anvil_decay_update": (_i, [_vp, _vp, _vp, _f, _vp, _vp, _i64, _i64, _i64, _vp]),
}

_lib = None


class AnvilError(RuntimeError):
    def __init__(self, fn: str, status: int, lib):
        self.status = status
        msg = lib.anvil_status_string(status).decode()
        if status == ANVIL_ERR_HIP:
            msg += f" (hipError {lib.anvil_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")


def load(path: str | None = None):
    """Load libanvil.so (built in-tree by build.py) and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run `python -m orthogonalizing_polynomial_cascade_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != ANVIL_OK:
        raise AnvilError(fn, status, load())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, name, dtype, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.device.index is not None and t.device.index != torch.cuda.current_device():
        # the library launches on the current HIP device and takes plain device pointers
        raise ValueError(f"{name} is on {t.device}, not on the current device "
                         f"cuda:{torch.cuda.current_device()} (use torch.cuda.set_device)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _gmn(grad):
    if grad.dim() != 3:
        raise ValueError("expected a [g, m, n] stack")
    return tuple(int(v) for v in grad.shape)


def workspace_bytes(g: int, m: int, n: int) -> int:
    return int(load().anvil_workspace_bytes(g, m, n))


def trace_slots(m: int, n: int) -> int:
    return int(load().anvil_trace_slots(m, n))


def release_workspaces():
    _check("anvil_release_workspaces", load().anvil_release_workspaces())


def anvil_bank_step(grad, velocity, momentum, fast_beta, fast_weight, out=None, workspace=None,
                    stream=None):
    """One ANVIL bank step on a [g, m, n] fp32 gradient stack.

    velocity (fp32 [2, g, m, n]) is updated in place; the bf16 update is written to `out`
    (allocated when None) and returned.  With `workspace` (a uint8 device tensor of at least
    workspace_bytes(g, m, n) bytes) the call allocates nothing.
    """
    import torch
    lib = load()
    _need(grad, "grad", torch.float32)
    g, m, n = _gmn(grad)
    _need(velocity, "velocity", torch.float32, (2, g, m, n))
    if out is None:
        out = torch.empty((g, m, n), dtype=torch.bfloat16, device=grad.device)
    _need(out, "out", torch.bfloat16, (g, m, n))
    if workspace is None:
        st = lib.anvil_bank_step(_ptr(grad), _ptr(velocity), momentum, fast_beta, fast_weight,
                                 _ptr(out), g, m, n, _stream(stream))
        _check("anvil_bank_step", st)
    else:
        _need(workspace, "workspace", torch.uint8)
        st = lib.anvil_bank_step_ws(_ptr(grad), _ptr(velocity), momentum, fast_beta, fast_weight,
                                    _ptr(out), g, m, n, _ptr(workspace), workspace.numel(),
                                    _stream(stream))
        _check("anvil_bank_step_ws", st)
    return out


def anvil_bank_step_noalloc(grad, velocity, momentum, fast_beta, fast_weight, out, stream=None):
    """anvil_bank_step with the library's built-in device scratch: the C call allocates nothing.
    `out` (bf16 [g, m, n]) must be given; the bank's workspace_bytes(g, m, n) may be at most
    NOALLOC_SCRATCH_BYTES.  Calls on one device share that scratch (order them)."""
    import torch
    lib = load()
    _need(grad, "grad", torch.float32)
    g, m, n = _gmn(grad)
    _need(velocity, "velocity", torch.float32, (2, g, m, n))
    _need(out, "out", torch.bfloat16, (g, m, n))
    _check("anvil_bank_step_noalloc", lib.anvil_bank_step_noalloc(
        _ptr(grad), _ptr(velocity), momentum, fast_beta, fast_weight, _ptr(out), g, m, n,
        _stream(stream)))
    return out


def anvil_bank_step_maps(grad, velocity, momentum, fast_beta, fast_weight, maps, out=None,
                         workspace=None, stream=None):
    """The bank step with a caller-chosen list of (a, b, c) quintic maps (1 to 16 of them)."""
    import torch
    lib = load()
    _need(grad, "grad", torch.float32)
    g, m, n = _gmn(grad)
    _need(velocity, "velocity", torch.float32, (2, g, m, n))
    table = [float(v) for abc in maps for v in abc]
    if len(table) != 3 * len(maps):
        raise ValueError("maps must be (a, b, c) triples")
    host = (ctypes.c_float * max(1, len(table)))(*table)
    if out is None:
        out = torch.empty((g, m, n), dtype=torch.bfloat16, device=grad.device)
    _need(out, "out", torch.bfloat16, (g, m, n))
    ws, wsb = None, 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
        ws, wsb = _ptr(workspace), workspace.numel()
    _check("anvil_bank_step_maps", lib.anvil_bank_step_maps(
        _ptr(grad), _ptr(velocity), momentum, fast_beta, fast_weight,
        ctypes.cast(host, ctypes.c_void_p), len(maps), _ptr(out), g, m, n, ws, wsb,
        _stream(stream)))
    return out


def _grad_dtype(grad):
    import torch
    if grad.dtype == torch.float32:
        return ANVIL_GRAD_F32
    if grad.dtype == torch.bfloat16:
        return ANVIL_GRAD_BF16
    raise TypeError("grad must be float32 or bfloat16")


def anvil_bank_step_dev(grad, velocity, scalars, out, workspace, stream=None):
    """The bank step with an fp32 or bf16 gradient and device scalars (fp32 [>= 3]: momentum,
    fast_beta, fast_weight) into fixed buffers; allocates nothing (graph-capturable)."""
    import torch
    lib = load()
    kind = _grad_dtype(grad)
    _need(grad, "grad", grad.dtype)
    g, m, n = _gmn(grad)
    _need(velocity, "velocity", torch.float32, (2, g, m, n))
    _need(scalars, "scalars", torch.float32)
    if scalars.numel() < 3:
        raise ValueError("scalars must hold momentum, fast_beta, fast_weight")
    _need(out, "out", torch.bfloat16, (g, m, n))
    _need(workspace, "workspace", torch.uint8)
    _check("anvil_bank_step_dev", lib.anvil_bank_step_dev(
        _ptr(grad), kind, _ptr(velocity), _ptr(scalars), _ptr(out), g, m, n, _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return out


def anvil_bank_update_dev(grad, velocity, scalars, update, lane_energy, beta2, param, mantissa,
                          eff_lr, workspace, stream=None):
    """The whole bank update in the page's bank contract: device scalars (fp32 [4]: momentum,
    fast_beta, fast_weight, eff_wd), fixed buffers, caller workspace; graph-capturable."""
    import torch
    lib = load()
    kind = _grad_dtype(grad)
    _need(grad, "grad", grad.dtype)
    g, m, n = _gmn(grad)
    _need(velocity, "velocity", torch.float32, (2, g, m, n))
    _need(scalars, "scalars", torch.float32)
    if scalars.numel() < 4:
        raise ValueError("scalars must hold momentum, fast_beta, fast_weight, eff_wd")
    _need(update, "update", torch.bfloat16, (g, m, n))
    _need(lane_energy, "lane_energy", torch.float32)
    if lane_energy.numel() != g * equalizer_lanes(m, n):
        raise ValueError("lane_energy must hold g * lanes values")
    _need(param, "param", torch.bfloat16, (g, m, n))
    if mantissa.dtype not in (torch.int16, torch.uint16):
        raise TypeError("mantissa must be a 16-bit integer tensor")
    _need(mantissa, "mantissa", mantissa.dtype, (g, m, n))
    _need(eff_lr, "eff_lr", torch.float32, (g,))
    _need(workspace, "workspace", torch.uint8)
    _check("anvil_bank_update_dev", lib.anvil_bank_update_dev(
        _ptr(grad), kind, _ptr(velocity), _ptr(scalars), _ptr(update), _ptr(lane_energy), beta2,
        _ptr(param), _ptr(mantissa), _ptr(eff_lr), g, m, n, _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return update


def anvil_momentum(grad, velocity, momentum, fast_beta, fast_weight, x_out=None, stream=None):
    import torch
    lib = load()
    _need(grad, "grad", torch.float32)
    g, m, n = _gmn(grad)
    _need(velocity, "velocity", torch.float32, (2, g, m, n))
    if x_out is None:
        x_out = torch.empty((g, m, n), dtype=torch.bfloat16, device=grad.device)
    _need(x_out, "x_out", torch.bfloat16, (g, m, n))
    _check("anvil_momentum", lib.anvil_momentum(_ptr(grad), _ptr(velocity), momentum, fast_beta,
                                                fast_weight, _ptr(x_out), g, m, n, _stream(stream)))
    return x_out


def anvil_gram(x, a_out=None, trace_partials=None, want_trace=False, stream=None):
    """Gram of each matrix of the bf16 stack x; returns (a_out, trace_partials or None)."""
    import torch
    lib = load()
    _need(x, "x", torch.bfloat16)
    g, m, n = _gmn(x)
    s = min(m, n)
    if a_out is None:
        a_out = torch.empty((g, s, s), dtype=torch.bfloat16, device=x.device)
    _need(a_out, "a_out", torch.bfloat16, (g, s, s))
    if want_trace and trace_partials is None:
        trace_partials = torch.empty((g, trace_slots(m, n)), dtype=torch.float32, device=x.device)
    if trace_partials is not None:
        _need(trace_partials, "trace_partials", torch.float32, (g, trace_slots(m, n)))
    _check("anvil_gram", lib.anvil_gram(_ptr(x), _ptr(a_out), _ptr(trace_partials), g, m, n,
                                        _stream(stream)))
    return a_out, trace_partials


def anvil_normalize(x, a, trace_partials, d_out=None, stream=None):
    """In-place x <- bf16(x / d), a <- bf16(a / d^2); returns d (fp32 [g])."""
    import torch
    lib = load()
    _need(x, "x", torch.bfloat16)
    g, m, n = _gmn(x)
    s = min(m, n)
    _need(a, "a", torch.bfloat16, (g, s, s))
    _need(trace_partials, "trace_partials", torch.float32, (g, trace_slots(m, n)))
    if d_out is None:
        d_out = torch.empty((g,), dtype=torch.float32, device=x.device)
    _need(d_out, "d_out", torch.float32, (g,))
    _check("anvil_normalize", lib.anvil_normalize(_ptr(x), _ptr(a), _ptr(trace_partials),
                                                  _ptr(d_out), g, m, n, _stream(stream)))
    return d_out


def anvil_poly(a, coef_b, coef_c, b_out=None, stream=None):
    import torch
    lib = load()
    _need(a, "a", torch.bfloat16)
    g, s, s2 = _gmn(a)
    if s != s2:
        raise ValueError("a must be a stack of square matrices")
    if b_out is None:
        b_out = torch.empty_like(a)
    _need(b_out, "b_out", torch.bfloat16, (g, s, s))
    _check("anvil_poly", lib.anvil_poly(_ptr(a), _ptr(b_out), coef_b, coef_c, g, s, _stream(stream)))
    return b_out


def anvil_apply(x, b, coef_a, split, c_out=None, stream=None):
    import torch
    lib = load()
    _need(x, "x", torch.bfloat16)
    g, m, n = _gmn(x)
    s = min(m, n)
    _need(b, "b", torch.bfloat16, (g, s, s))
    if c_out is None:
        c_out = torch.empty_like(x)
    _need(c_out, "c_out", torch.bfloat16, (g, m, n))
    _check("anvil_apply", lib.anvil_apply(_ptr(x), _ptr(b), _ptr(c_out), coef_a, int(bool(split)),
                                          g, m, n, _stream(stream)))
    return c_out


def equalizer_lanes(m: int, n: int) -> int:
    return int(load().anvil_equalizer_lanes(m, n))


def anvil_bank_update(grad, velocity, momentum, fast_beta, fast_weight, lane_energy, beta2,
                      param, mantissa, eff_wd, eff_lr, update=None, workspace=None, stream=None):
    """One whole bank update (step, equalizer, sign-aligned decay).

    grad fp32 [g,m,n]; velocity fp32 [2,g,m,n], lane_energy fp32 [g, lanes], param bf16 [g,m,n]
    and mantissa int16/uint16 [g,m,n] are updated in place; eff_lr fp32 [g].  Returns the
    equalized bf16 update."""
    import torch
    lib = load()
    _need(grad, "grad", torch.float32)
    g, m, n = _gmn(grad)
    _need(velocity, "velocity", torch.float32, (2, g, m, n))
    _need(lane_energy, "lane_energy", torch.float32)
    if lane_energy.numel() != g * equalizer_lanes(m, n):
        raise ValueError("lane_energy must hold g * lanes values")
    _need(param, "param", torch.bfloat16, (g, m, n))
    if mantissa.dtype not in (torch.int16, torch.uint16):
        raise TypeError("mantissa must be a 16-bit integer tensor")
    _need(mantissa, "mantissa", mantissa.dtype, (g, m, n))
    _need(eff_lr, "eff_lr", torch.float32, (g,))
    if update is None:
        update = torch.empty((g, m, n), dtype=torch.bfloat16, device=grad.device)
    _need(update, "update", torch.bfloat16, (g, m, n))
    args = [_ptr(grad), _ptr(velocity), momentum, fast_beta, fast_weight, _ptr(update),
            _ptr(lane_energy), beta2, _ptr(param), _ptr(mantissa), eff_wd, _ptr(eff_lr), g, m, n]
    if workspace is None:
        _check("anvil_bank_update", lib.anvil_bank_update(*args, _stream(stream)))
    else:
        _need(workspace, "workspace", torch.uint8)
        _check("anvil_bank_update_ws", lib.anvil_bank_update_ws(*args, _ptr(workspace),
                                                                workspace.numel(), _stream(stream)))
    return update


def anvil_equalize(update, lane_energy, beta2, lane_scratch=None, stream=None):
    """In-place equalizer on a bf16 [g,m,n] update; lane_energy fp32 [g, lanes] in place."""
    import torch
    lib = load()
    _need(update, "update", torch.bfloat16)
    g, m, n = _gmn(update)
    lanes = equalizer_lanes(m, n)
    _need(lane_energy, "lane_energy", torch.float32)
    if lane_energy.numel() != g * lanes:
        raise ValueError("lane_energy must hold g * lanes values")
    if lane_scratch is None:
        lane_scratch = torch.empty(2 * g * lanes, dtype=torch.float32, device=update.device)
    _need(lane_scratch, "lane_scratch", torch.float32)
    if lane_scratch.numel() < 2 * g * lanes:
        raise ValueError("lane_scratch must hold 2 * g * lanes values")
    _check("anvil_equalize", lib.anvil_equalize(_ptr(update), _ptr(lane_energy), beta2,
                                                _ptr(lane_scratch), g, m, n, _stream(stream)))
    return update


def anvil_decay_update(param, mantissa, update, eff_wd, eff_lr, gate, stream=None):
    """In-place sign-aligned decay of (param bf16, mantissa uint16) by the bf16 update."""
    import torch
    lib = load()
    _need(param, "param", torch.bfloat16)
    g, m, n = _gmn(param)
    if mantissa.dtype not in (torch.int16, torch.uint16):
        raise TypeError("mantissa must be a 16-bit integer tensor")
    _need(mantissa, "mantissa", mantissa.dtype, (g, m, n))
    _need(update, "update", torch.bfloat16, (g, m, n))
    _need(eff_lr, "eff_lr", torch.float32, (g,))
    _need(gate, "gate", torch.float32, (g, m, n))
    _check("anvil_decay_update", lib.anvil_decay_update(_ptr(param), _ptr(mantissa), _ptr(update),
                                                        eff_wd, _ptr(eff_lr), _ptr(gate), g, m, n,
                                                        _stream(stream)))


def rail_scalars(step: int):
    """(momentum, fast_beta, fast_weight) of a training step under the source's rail schedule:
    fast rail only before step 514, blend weight 0.4385 on the fast rail from step 514 on; fast
    beta 0.85 and Nesterov momentum 0.95 throughout (the pre-engage beta scheduler is not given)."""
    return 0.95, 0.85, (1.0 if step < 514 else 0.4385)
