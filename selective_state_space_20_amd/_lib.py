"""ctypes binding of libsss.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module checks
tensor properties, allocates the workspace and outputs with torch (device memory and the
current stream are the only things torch provides) and calls the C ABI of include/sss.h.
There is no fallback: if the shared library is missing the import of the function fails.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsss.so")

SSS_F32, SSS_BF16 = 0, 1
STATUS = {0: "SSS_OK", -1: "SSS_ERR_NULL_ARG", -2: "SSS_ERR_BAD_DIM", -3: "SSS_ERR_UNSUPPORTED",
          -4: "SSS_ERR_WORKSPACE", -5: "SSS_ERR_ALIAS", -6: "SSS_ERR_HIP"}

SSS_EXACT_ZOH, SSS_DELTA_SOFTPLUS, SSS_LAYOUT_BDL = 1, 2, 4

EXPORTED = ("selective_scan_fwd", "selective_scan_fwd_ex", "selective_scan_fwd_workspace_size",
            "selective_scan_fwd_ex_workspace_size", "selective_state_update",
            "causal_conv1d_fwd", "selective_scan_bwd", "selective_scan_bwd_workspace_size",
            "elementwise_scan", "elementwise_scan_workspace_size", "sss_status_string",
            "selective_scan_fwd_noalloc", "selective_scan_states_size", "selective_scan_fwd_save",
            "selective_scan_bwd_saved", "selective_scan_bwd_ex")


class SSSError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


_lib = None


def load() -> ctypes.CDLL:
    """Load libsss.so (raises if it has not been built).

    torch is imported first: it ships its own HIP runtime, and libsss.so must bind to that
    same runtime.  Loaded first, the library would pull in the system ROCm's runtime and the
    process would hold two, of which torch's then finds no GPU."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with selective_state_space_20_amd.build.build()")
        import torch  # noqa: F401  (see above: one HIP runtime per process)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        lib.selective_scan_fwd.argtypes = [vp] * 10 + [i64] * 4 + [i32, vp, sz, vp]
        lib.selective_scan_fwd.restype = i32
        lib.selective_scan_fwd_ex.argtypes = [vp] * 11 + [ctypes.c_uint] + [i64] * 4 + [i32, vp, sz, vp]
        lib.selective_scan_fwd_ex.restype = i32
        lib.selective_scan_fwd_workspace_size.argtypes = [i64] * 4 + [i32]
        lib.selective_scan_fwd_workspace_size.restype = sz
        lib.selective_scan_fwd_ex_workspace_size.argtypes = [i64] * 4 + [ctypes.c_uint, i32]
        lib.selective_scan_fwd_ex_workspace_size.restype = sz
        lib.selective_state_update.argtypes = [vp] * 9 + [i64] * 3 + [i32, vp]
        lib.selective_state_update.restype = i32
        lib.causal_conv1d_fwd.argtypes = [vp] * 4 + [i64] * 4 + [i32, i32, vp]
        lib.causal_conv1d_fwd.restype = i32
        lib.selective_scan_bwd.argtypes = [vp] * 18 + [i64] * 4 + [i32, vp, sz, vp]
        lib.selective_scan_bwd.restype = i32
        lib.selective_scan_bwd_workspace_size.argtypes = [i64] * 4 + [i32]
        lib.selective_scan_bwd_workspace_size.restype = sz
        lib.elementwise_scan.argtypes = [vp] * 7 + [i64] * 3 + [vp, sz, vp]
        lib.elementwise_scan.restype = i32
        lib.elementwise_scan_workspace_size.argtypes = [i64] * 3 + [i32]
        lib.elementwise_scan_workspace_size.restype = sz
        lib.selective_scan_fwd_noalloc.argtypes = [vp] * 10 + [i64] * 4 + [i32, vp]
        lib.selective_scan_fwd_noalloc.restype = i32
        lib.selective_scan_states_size.argtypes = [i64] * 4 + [i32]
        lib.selective_scan_states_size.restype = sz
        lib.selective_scan_fwd_save.argtypes = [vp] * 11 + [sz] + [i64] * 4 + [i32, vp, sz, vp]
        lib.selective_scan_fwd_save.restype = i32
        lib.selective_scan_bwd_saved.argtypes = [vp] * 11 + [sz] + [vp] * 8 + [i64] * 4 + [i32, vp, sz, vp]
        lib.selective_scan_bwd_saved.restype = i32
        lib.selective_scan_bwd_ex.argtypes = [vp] * 11 + [ctypes.c_uint] + [vp] * 9 + [i64] * 4 + [i32, vp, sz, vp]
        lib.selective_scan_bwd_ex.restype = i32
        lib.sss_status_string.argtypes = [i32]
        lib.sss_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().sss_status_string(int(status)).decode()


# ---------------------------------------------------------------- raw-pointer entry points
def selective_scan_fwd_raw(x, delta, A, B, C, D_skip, z, h0, y, h_last, batch, seqlen, dim, dstate, io_dtype,
                           workspace, workspace_bytes, stream) -> int:
    """Direct call of the C function with integer pointers (0 = NULL)."""
    return load().selective_scan_fwd(x, delta, A, B, C, D_skip, z, h0, y, h_last, batch, seqlen, dim, dstate,
                                     io_dtype, workspace, workspace_bytes, stream)


def selective_scan_fwd_noalloc_raw(x, delta, A, B, C, D_skip, z, h0, y, h_last, batch, seqlen, dim, dstate, io_dtype,
                                   stream) -> int:
    """selective_scan_fwd_noalloc: no workspace (the library's per-GPU scratch array)."""
    return load().selective_scan_fwd_noalloc(x, delta, A, B, C, D_skip, z, h0, y, h_last, batch, seqlen, dim, dstate,
                                             io_dtype, stream)


def selective_scan_fwd_ex_raw(x, delta, A, B, C, D_skip, z, h0, y, h_last, delta_bias, flags, batch, seqlen, dim,
                              dstate, io_dtype, workspace, workspace_bytes, stream) -> int:
    return load().selective_scan_fwd_ex(x, delta, A, B, C, D_skip, z, h0, y, h_last, delta_bias, flags, batch, seqlen,
                                        dim, dstate, io_dtype, workspace, workspace_bytes, stream)


def selective_scan_bwd_raw(x, delta, A, B, C, D_skip, z, h0, dy, dh_last, dx, ddelta, dA, dB, dC, dD, dz, dh0, batch,
                           seqlen, dim, dstate, io_dtype, workspace, workspace_bytes, stream) -> int:
    return load().selective_scan_bwd(x, delta, A, B, C, D_skip, z, h0, dy, dh_last, dx, ddelta, dA, dB, dC, dD, dz, dh0,
                                     batch, seqlen, dim, dstate, io_dtype, workspace, workspace_bytes, stream)


def selective_scan_bwd_ex_raw(x, delta, A, B, C, D_skip, z, h0, dy, dh_last, delta_bias, flags, dx, ddelta, dA, dB,
                              dC, dD, dz, dh0, ddelta_bias, batch, seqlen, dim, dstate, io_dtype, workspace,
                              workspace_bytes, stream) -> int:
    return load().selective_scan_bwd_ex(x, delta, A, B, C, D_skip, z, h0, dy, dh_last, delta_bias, flags, dx, ddelta,
                                        dA, dB, dC, dD, dz, dh0, ddelta_bias, batch, seqlen, dim, dstate, io_dtype,
                                        workspace, workspace_bytes, stream)


def selective_scan_bwd_workspace_size(batch, seqlen, dim, dstate, device=0) -> int:
    return int(load().selective_scan_bwd_workspace_size(batch, seqlen, dim, dstate, device))


def selective_scan_states_size(batch, seqlen, dim, dstate, device=0) -> int:
    """Bytes of the segment entering states selective_scan_fwd_save keeps (0: nothing to keep)."""
    return int(load().selective_scan_states_size(batch, seqlen, dim, dstate, device))


def selective_scan_fwd_save_raw(x, delta, A, B, C, D_skip, z, h0, y, h_last, states, states_bytes, batch, seqlen, dim,
                                dstate, io_dtype, workspace, workspace_bytes, stream) -> int:
    return load().selective_scan_fwd_save(x, delta, A, B, C, D_skip, z, h0, y, h_last, states, states_bytes, batch,
                                          seqlen, dim, dstate, io_dtype, workspace, workspace_bytes, stream)


def selective_scan_bwd_saved_raw(x, delta, A, B, C, D_skip, z, h0, dy, dh_last, states, states_bytes, dx, ddelta, dA,
                                 dB, dC, dD, dz, dh0, batch, seqlen, dim, dstate, io_dtype, workspace, workspace_bytes,
                                 stream) -> int:
    return load().selective_scan_bwd_saved(x, delta, A, B, C, D_skip, z, h0, dy, dh_last, states, states_bytes, dx,
                                           ddelta, dA, dB, dC, dD, dz, dh0, batch, seqlen, dim, dstate, io_dtype,
                                           workspace, workspace_bytes, stream)


def _states_buffer(states, nbytes, dev):
    """(pointer, bytes) of a caller's saved-states buffer: a uint8 or float32 CUDA tensor of at
    least nbytes on dev; None only when nothing is kept (nbytes == 0)."""
    import torch
    if states is None:
        if nbytes > 0:
            raise ValueError(f"states: a buffer of {nbytes} bytes is needed (selective_scan_states_size)")
        return 0, 0
    if not isinstance(states, torch.Tensor) or states.dtype not in (torch.uint8, torch.float32):
        raise ValueError("states must be a uint8 or float32 torch tensor")
    if not states.is_contiguous():
        raise ValueError("states must be contiguous")
    if states.device != dev:
        raise ValueError(f"states is on {states.device}, the inputs on {dev}")
    have = states.numel() * states.element_size()
    if have < nbytes:
        raise ValueError(f"states holds {have} bytes, {nbytes} are needed")
    return states.data_ptr(), have


def selective_scan_bwd(x, delta, A, B, C, D=None, z=None, h0=None, *, dy, dh_last=None, want_dh0=True,
                       workspace=None, stream=None, states=None, delta_bias=None, delta_softplus=False):
    """Gradients of sum(dy * y) + sum(dh_last * h_last) of selective_scan_fwd (plain form).

    states: the buffer a selective_scan_fwd(..., states=...) call on the same x, delta, A, B,
    h0 filled (selective_scan_bwd_saved); None recomputes them (selective_scan_bwd).
    delta_bias (dim) float32 / delta_softplus: the delta front end of selective_scan_fwd_ex
    (selective_scan_bwd_ex); ddelta is then the gradient with respect to the stored delta.

    Returns a dict of float32 tensors: dx, ddelta, dA, dB, dC, and dD (with D), dz (with z),
    dh0 (if want_dh0), ddelta_bias (with delta_bias)."""
    import torch
    dev = x.device
    batch, seqlen, dim = x.shape
    dstate = A.shape[1]
    io = x.dtype
    io_code = _io_dtype(x)
    f32 = torch.float32
    for t, n, dt, sh in ((x, "x", io, (batch, seqlen, dim)), (delta, "delta", io, (batch, seqlen, dim)),
                         (z, "z", io, (batch, seqlen, dim)), (A, "A", f32, (dim, dstate)),
                         (B, "B", f32, (batch, seqlen, dstate)), (C, "C", f32, (batch, seqlen, dstate)),
                         (D, "D", f32, (dim,)), (h0, "h0", f32, (batch, dim, dstate)),
                         (dy, "dy", f32, (batch, seqlen, dim)), (dh_last, "dh_last", f32, (batch, dim, dstate)),
                         (delta_bias, "delta_bias", f32, (dim,))):
        _need(t, n, dt, sh, dev)
    front = delta_bias is not None or bool(delta_softplus)
    if front and states is not None:
        raise ValueError("the delta front end has no saved-states form (states=)")
    _on_device(dev, x=x, delta=delta, z=z, A=A, B=B, C=C, D=D, h0=h0, dy=dy, dh_last=dh_last, delta_bias=delta_bias)
    e = lambda *sh: torch.empty(sh, dtype=f32, device=dev)
    g = dict(dx=e(batch, seqlen, dim), ddelta=e(batch, seqlen, dim), dA=e(dim, dstate), dB=e(batch, seqlen, dstate),
             dC=e(batch, seqlen, dstate))
    g["dD"] = e(dim) if D is not None else None
    g["dz"] = e(batch, seqlen, dim) if z is not None else None
    g["dh0"] = e(batch, dim, dstate) if want_dh0 else None
    if delta_bias is not None:
        g["ddelta_bias"] = e(dim)
    wsb = selective_scan_bwd_workspace_size(batch, seqlen, dim, dstate, dev.index or 0)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    wsp, wsn = _workspace(workspace, dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    if front:
        rc = selective_scan_bwd_ex_raw(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                       _ptr(dy), _ptr(dh_last), _ptr(delta_bias),
                                       SSS_DELTA_SOFTPLUS if delta_softplus else 0, _ptr(g["dx"]), _ptr(g["ddelta"]),
                                       _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]),
                                       _ptr(g["dh0"]), _ptr(g.get("ddelta_bias")), batch, seqlen, dim, dstate, io_code,
                                       wsp, wsn, st)
        if rc != 0:
            raise SSSError(rc, "selective_scan_bwd_ex")
        return g
    if states is None:
        rc = selective_scan_bwd_raw(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                    _ptr(dy), _ptr(dh_last), _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
                                    _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]), batch,
                                    seqlen, dim, dstate, io_code, wsp, wsn, st)
        if rc != 0:
            raise SSSError(rc, "selective_scan_bwd")
        return g
    sp, sn = _states_buffer(states, selective_scan_states_size(batch, seqlen, dim, dstate, dev.index or 0), dev)
    rc = selective_scan_bwd_saved_raw(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                      _ptr(dy), _ptr(dh_last), sp, sn, _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
                                      _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]), batch,
                                      seqlen, dim, dstate, io_code, wsp, wsn, st)
    if rc != 0:
        raise SSSError(rc, "selective_scan_bwd_saved")
    return g


def causal_conv1d_fwd_raw(x, weight, bias, out, batch, seqlen, dim, width, io_dtype, apply_silu, stream) -> int:
    return load().causal_conv1d_fwd(x, weight, bias, out, batch, seqlen, dim, width, io_dtype, apply_silu, stream)


def causal_conv1d_fwd(x, weight, bias=None, *, silu=False, out=None, stream=None):
    """Causal depthwise convolution: out (batch, seqlen, dim) in x's dtype (float32 or
    bfloat16); weight (dim, width), bias (dim) float32."""
    import torch
    dev = x.device
    batch, seqlen, dim = x.shape
    width = weight.shape[1]
    io = x.dtype
    io_code = _io_dtype(x)
    _need(x, "x", io, (batch, seqlen, dim), dev)
    _need(weight, "weight", torch.float32, (dim, width), dev)
    _need(bias, "bias", torch.float32, (dim,), dev)
    o = out if out is not None else torch.empty((batch, seqlen, dim), dtype=io, device=dev)
    _need(o, "out", io, (batch, seqlen, dim), dev)
    _on_device(dev, x=x, weight=weight, bias=bias, out=o)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    rc = causal_conv1d_fwd_raw(_ptr(x), _ptr(weight), _ptr(bias), _ptr(o), batch, seqlen, dim, width, io_code,
                               int(bool(silu)), st)
    if rc != 0:
        raise SSSError(rc, "causal_conv1d_fwd")
    return o


def selective_state_update_raw(x, delta, A, B, C, D_skip, z, state, y, batch, dim, dstate, io_dtype, stream) -> int:
    return load().selective_state_update(x, delta, A, B, C, D_skip, z, state, y, batch, dim, dstate, io_dtype, stream)


def elementwise_scan_raw(x, A, B, C, h0, y, h_last, batch, seqlen, dim, workspace, workspace_bytes,
                         stream) -> int:
    return load().elementwise_scan(x, A, B, C, h0, y, h_last, batch, seqlen, dim, workspace, workspace_bytes,
                                   stream)


def selective_scan_fwd_ex_workspace_size(batch, seqlen, dim, dstate, flags=0, device=0) -> int:
    return int(load().selective_scan_fwd_ex_workspace_size(batch, seqlen, dim, dstate, flags, device))


def selective_scan_fwd_workspace_size(batch, seqlen, dim, dstate, device=0) -> int:
    return int(load().selective_scan_fwd_workspace_size(batch, seqlen, dim, dstate, device))


def elementwise_scan_workspace_size(batch, seqlen, dim, device=0) -> int:
    return int(load().elementwise_scan_workspace_size(batch, seqlen, dim, device))


# ---------------------------------------------------------------- torch-tensor entry points
def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _need(t, name, dtype, shape, device):
    """dtype, shape and contiguity of one tensor (its device is checked by _on_device once
    every tensor of the call has passed these): a mismatch raises before any device work."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(device, **tensors):
    """Every given tensor (None skipped) is on the call's GPU."""
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != device):
            raise ValueError(f"{name} must be on a GPU ({device}), got {t.device}")


def _io_dtype(x):
    """x/delta/z dtype code; anything but float32 and bfloat16 is rejected."""
    import torch
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"x must be float32 or bfloat16, got {x.dtype}")
    return SSS_BF16 if x.dtype == torch.bfloat16 else SSS_F32


def _workspace(ws, device):
    """(pointer, size in bytes) of a caller-given workspace, checked to be contiguous device
    memory on the call's device."""
    if ws is None:
        return 0, 0
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if not ws.is_cuda or ws.device != device:
        raise ValueError(f"workspace must be on {device}")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def selective_scan_fwd(x, delta, A, B, C, D=None, z=None, h0=None, *, return_last=True, out=None,
                       out_last=None, workspace=None, stream=None, delta_bias=None, delta_softplus=False,
                       exact_zoh=False, layout="bld", states=None):
    """y (batch, seqlen, dim) float32 [, h_last (batch, dim, dstate) float32].

    x, delta, z: float32 or bfloat16 (one dtype); A (dim, dstate), B, C (batch, seqlen,
    dstate), D (dim), h0 (batch, dim, dstate): float32.  All on one GPU, contiguous.
    delta_bias (dim) float32 / delta_softplus / exact_zoh select selective_scan_fwd_ex's
    options (step size softplus(delta + bias); exact zero-order-hold input term).
    layout="bdl": x, delta, z and y are (batch, dim, seqlen), B and C (batch, dstate, seqlen).
    """
    import torch
    if layout not in ("bld", "bdl"):
        raise ValueError(f"layout must be 'bld' or 'bdl', got {layout!r}")
    bdl = layout == "bdl"
    dev = x.device
    if bdl:
        batch, dim, seqlen = x.shape
    else:
        batch, seqlen, dim = x.shape
    dstate = A.shape[1]
    io = x.dtype
    io_code = _io_dtype(x)
    f32 = torch.float32
    io_shape = (batch, dim, seqlen) if bdl else (batch, seqlen, dim)
    bc_shape = (batch, dstate, seqlen) if bdl else (batch, seqlen, dstate)
    _need(x, "x", io, io_shape, dev)
    _need(delta, "delta", io, io_shape, dev)
    _need(z, "z", io, io_shape, dev)
    _need(A, "A", f32, (dim, dstate), dev)
    _need(B, "B", f32, bc_shape, dev)
    _need(C, "C", f32, bc_shape, dev)
    _need(D, "D", f32, (dim,), dev)
    _need(h0, "h0", f32, (batch, dim, dstate), dev)
    y = out if out is not None else torch.empty(io_shape, dtype=f32, device=dev)
    hl = out_last if out_last is not None else (
        torch.empty((batch, dim, dstate), dtype=f32, device=dev) if return_last else None)
    _need(y, "out", f32, io_shape, dev)
    _need(hl, "out_last", f32, (batch, dim, dstate), dev)
    flags = ((SSS_EXACT_ZOH if exact_zoh else 0) | (SSS_DELTA_SOFTPLUS if delta_softplus else 0)
             | (SSS_LAYOUT_BDL if bdl else 0))
    _need(delta_bias, "delta_bias", f32, (dim,), dev)
    _on_device(dev, x=x, delta=delta, z=z, A=A, B=B, C=C, D=D, h0=h0, out=y, out_last=hl, delta_bias=delta_bias)
    wsb = selective_scan_fwd_ex_workspace_size(batch, seqlen, dim, dstate, flags, dev.index or 0)
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    wsp, wsn = _workspace(workspace, dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    if states is not None:  # selective_scan_fwd_save: the plain form, keeping the segment entering states
        if flags != 0 or delta_bias is not None:
            raise ValueError("states: the forward that keeps its states is the plain form (no options)")
        sp, sn = _states_buffer(states, selective_scan_states_size(batch, seqlen, dim, dstate, dev.index or 0), dev)
        rc = selective_scan_fwd_save_raw(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                         _ptr(y), _ptr(hl), sp, sn, batch, seqlen, dim, dstate, io_code, wsp, wsn, st)
        if rc != 0:
            raise SSSError(rc, "selective_scan_fwd_save")
        return (y, hl) if return_last or out_last is not None else y
    rc = selective_scan_fwd_ex_raw(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                   _ptr(y), _ptr(hl), _ptr(delta_bias), flags, batch, seqlen, dim, dstate, io_code,
                                   wsp, wsn, st)
    if rc != 0:
        raise SSSError(rc, "selective_scan_fwd")
    return (y, hl) if return_last or out_last is not None else y


def selective_state_update(x, delta, A, B, C, D=None, z=None, *, state, out=None, stream=None):
    """One decode step: updates ``state`` (batch, dim, dstate) float32 in place and returns
    y (batch, dim) float32.  x, delta, z: (batch, dim) float32 or bfloat16 (one dtype);
    A (dim, dstate), B, C (batch, dstate), D (dim): float32."""
    import torch
    dev = x.device
    batch, dim = x.shape
    dstate = A.shape[1]
    io = x.dtype
    io_code = _io_dtype(x)
    f32 = torch.float32
    _need(x, "x", io, (batch, dim), dev)
    _need(delta, "delta", io, (batch, dim), dev)
    _need(z, "z", io, (batch, dim), dev)
    _need(A, "A", f32, (dim, dstate), dev)
    _need(B, "B", f32, (batch, dstate), dev)
    _need(C, "C", f32, (batch, dstate), dev)
    _need(D, "D", f32, (dim,), dev)
    _need(state, "state", f32, (batch, dim, dstate), dev)
    y = out if out is not None else torch.empty((batch, dim), dtype=f32, device=dev)
    _need(y, "out", f32, (batch, dim), dev)
    _on_device(dev, x=x, delta=delta, z=z, A=A, B=B, C=C, D=D, state=state, out=y)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    rc = selective_state_update_raw(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(state),
                                    _ptr(y), batch, dim, dstate, io_code, st)
    if rc != 0:
        raise SSSError(rc, "selective_state_update")
    return y


def elementwise_scan(x, A, B, C, h0=None, *, return_last=True, out=None, out_last=None, workspace=None,
                     stream=None):
    """y (batch, seqlen, dim) [, h_last (batch, dim)]; every tensor float32 on one GPU."""
    import torch
    dev = x.device
    batch, seqlen, dim = x.shape
    f32 = torch.float32
    for t, n in ((x, "x"), (A, "A"), (B, "B"), (C, "C")):
        _need(t, n, f32, (batch, seqlen, dim), dev)
    _need(h0, "h0", f32, (batch, dim), dev)
    y = out if out is not None else torch.empty((batch, seqlen, dim), dtype=f32, device=dev)
    hl = out_last if out_last is not None else (
        torch.empty((batch, dim), dtype=f32, device=dev) if return_last else None)
    _need(y, "out", f32, (batch, seqlen, dim), dev)
    _need(hl, "out_last", f32, (batch, dim), dev)
    _on_device(dev, x=x, A=A, B=B, C=C, h0=h0, out=y, out_last=hl)
    wsb = elementwise_scan_workspace_size(batch, seqlen, dim, dev.index or 0)
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    wsp, wsn = _workspace(workspace, dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    rc = elementwise_scan_raw(_ptr(x), _ptr(A), _ptr(B), _ptr(C), _ptr(h0), _ptr(y), _ptr(hl), batch, seqlen, dim,
                              wsp, wsn, st)
    if rc != 0:
        raise SSSError(rc, "elementwise_scan")
    return (y, hl) if return_last or out_last is not None else y
