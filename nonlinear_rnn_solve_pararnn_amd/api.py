"""Thin Python binding of libpararnn.so (include/pararnn.h).

Argument marshalling only: checks dtype, device, shape and contiguity,
allocates outputs and the workspace with torch (the caching allocator, so no
hipMalloc per call), passes raw device pointers and the current HIP stream to
the C ABI, and raises on a negative status.  Every step of the computation
runs in the library's HIP kernels; there is no fallback of any kind, and a
missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpararnn.so")

OP_LINSCAN_DIAG, OP_LINSCAN_BLK2, OP_GRU_FORWARD, OP_LSTM_FORWARD, OP_GRU_ADJOINT, \
    OP_LSTM_ADJOINT, OP_LINSCAN_BLK4, OP_LINSCAN_BLK8, OP_HGRU4_FORWARD, OP_HGRU8_FORWARD, \
    OP_HGRU4_BACKWARD, OP_HGRU8_BACKWARD = range(12)
CELL_GRU, CELL_LSTM = 0, 1

EXPORTS = ("pararnn_workspace_bytes", "rnn_linscan_diag", "rnn_linscan_blk2", "rnn_linscan_blk",
           "pararnn_gru_forward", "pararnn_lstm_forward", "pararnn_adjoint_backward",
           "pararnn_gru_sequential", "pararnn_lstm_sequential", "pararnn_status_string",
           "pararnn_gru_forward_noalloc", "pararnn_hgru_forward", "pararnn_hgru_backward")
NOALLOC_SCRATCH_BYTES = 64 << 20   # PARARNN_NOALLOC_SCRATCH_BYTES

_lib = None


class PararnnError(RuntimeError):
    pass


def load_library():
    """Load libpararnn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise PararnnError(
            "libpararnn.so not found at %s; build it with "
            "`python -m nonlinear_rnn_solve_pararnn_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sz = ctypes.c_size_t
    lib.pararnn_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
    lib.pararnn_workspace_bytes.restype = sz
    lib.rnn_linscan_diag.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, sz, vp]
    lib.rnn_linscan_diag.restype = ctypes.c_int
    lib.rnn_linscan_blk2.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, sz, vp]
    lib.rnn_linscan_blk2.restype = ctypes.c_int
    lib.rnn_linscan_blk.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, sz, vp]
    lib.rnn_linscan_blk.restype = ctypes.c_int
    lib.pararnn_gru_forward.argtypes = [i64, i64, i64] + [vp] * 9 + [
        ctypes.c_float, i32, vp, vp, vp, sz, vp]
    lib.pararnn_gru_forward.restype = ctypes.c_int
    lib.pararnn_lstm_forward.argtypes = [i64, i64, i64] + [vp] * 14 + [
        ctypes.c_float, i32, vp, vp, vp, sz, vp]
    lib.pararnn_lstm_forward.restype = ctypes.c_int
    lib.pararnn_hgru_forward.argtypes = [i32, i64, i64, i64] + [vp] * 9 + [
        ctypes.c_float, i32, vp, vp, vp, sz, vp]
    lib.pararnn_hgru_forward.restype = ctypes.c_int
    lib.pararnn_hgru_backward.argtypes = [i32, i64, i64, i64] + [vp] * 17 + [sz, vp]
    lib.pararnn_hgru_backward.restype = ctypes.c_int
    lib.pararnn_adjoint_backward.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                             vp, vp, vp, vp, vp, sz, vp]
    lib.pararnn_adjoint_backward.restype = ctypes.c_int
    lib.pararnn_gru_sequential.argtypes = [i64, i64, i64] + [vp] * 8 + [vp]
    lib.pararnn_gru_sequential.restype = ctypes.c_int
    lib.pararnn_lstm_sequential.argtypes = [i64, i64, i64] + [vp] * 12 + [vp]
    lib.pararnn_lstm_sequential.restype = ctypes.c_int
    lib.pararnn_gru_forward_noalloc.argtypes = [i64, i64, i64] + [vp] * 8 + [
        ctypes.c_float, i32, vp, vp, vp]
    lib.pararnn_gru_forward_noalloc.restype = ctypes.c_int
    lib.pararnn_status_string.argtypes = [ctypes.c_int]
    lib.pararnn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        msg = load_library().pararnn_status_string(status).decode()
        raise PararnnError("%s failed: status %d (%s)" % (what, status, msg))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, shape, name: str, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a HIP device" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def workspace_bytes(op: int, B: int, L: int, H: int, max_iter: int = 1) -> int:
    return int(load_library().pararnn_workspace_bytes(op, B, L, H, max_iter))


# One zero-filled workspace per (device, stream), grown on demand.  The
# library leaves a workspace ready for the next call of any entry point, so it
# is cleared only when it is first allocated.
_ws_cache = {}


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace of at least `nbytes` bytes (the library requires
    a zero-filled workspace on first use; later calls keep it valid)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def release_workspaces():
    """Drop the cached per-stream workspaces."""
    _ws_cache.clear()


def _workspace(op, B, L, H, device, max_iter=1, ws=None):
    n = workspace_bytes(op, B, L, H, max_iter)
    if n == 0:
        raise PararnnError("invalid sizes B=%d L=%d H=%d" % (B, L, H))
    if ws is not None:
        if ws.device != device or ws.numel() * ws.element_size() < n or ws.data_ptr() % 256:
            raise ValueError("workspace too small, misaligned or on the wrong device")
        return ws, ws.numel() * ws.element_size()
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < n:
        buf = new_workspace(n, device)
        _ws_cache[key] = buf
    return buf, buf.numel()


# ---------------------------------------------------------------- scans
def linscan_diag(a, b, h0=None, *, out=None, ws=None):
    """h_t = a_t * h_{t-1} + b_t over dim 1 of [B, L, H] tensors."""
    lib = load_library()
    B, L, H = a.shape
    dev = a.device
    _need(a, (B, L, H), "a")
    _need(b, (B, L, H), "b", dev)
    if h0 is not None:
        _need(h0, (B, H), "h0", dev)
    h = torch.empty_like(a) if out is None else out
    _need(h, (B, L, H), "out", dev)
    ws, n = _workspace(OP_LINSCAN_DIAG, B, L, H, dev, ws=ws)
    _check(lib.rnn_linscan_diag(B, L, H, _ptr(a), _ptr(b), _ptr(h0), _ptr(h), _ptr(ws), n,
                                _stream(dev)), "rnn_linscan_diag")
    return h


def linscan_blk2(A, b, h0=None, *, out=None, ws=None):
    """h_t = A_t @ h_{t-1} + b_t with A [B, L, H, 2, 2], b/h [B, L, H, 2]."""
    lib = load_library()
    B, L, H = b.shape[:3]
    dev = b.device
    _need(A, (B, L, H, 2, 2), "A", dev)
    _need(b, (B, L, H, 2), "b", dev)
    if h0 is not None:
        _need(h0, (B, H, 2), "h0", dev)
    h = torch.empty_like(b) if out is None else out
    _need(h, (B, L, H, 2), "out", dev)
    ws, n = _workspace(OP_LINSCAN_BLK2, B, L, H, dev, ws=ws)
    _check(lib.rnn_linscan_blk2(B, L, H, _ptr(A), _ptr(b), _ptr(h0), _ptr(h), _ptr(ws), n,
                                _stream(dev)), "rnn_linscan_blk2")
    return h


# ---------------------------------------------------------------- Newton forward
def linscan_blk(A, b, h0=None, *, out=None, ws=None):
    """k x k block scan h_t = A_t h_{t-1} + b_t (k = 2, 4 or 8); A [B, L, H, k, k],
    b [B, L, H, k]; returns h [B, L, H, k]."""
    lib = load_library()
    B, L, H, k = b.shape
    dev = b.device
    _need(A, (B, L, H, k, k), "A", dev)
    _need(b, (B, L, H, k), "b", dev)
    if h0 is not None:
        _need(h0, (B, H, k), "h0", dev)
    h = torch.empty_like(b) if out is None else out
    _need(h, (B, L, H, k), "out", dev)
    op = {2: OP_LINSCAN_BLK2, 4: OP_LINSCAN_BLK4, 8: OP_LINSCAN_BLK8}.get(k)
    if op is None:
        raise PararnnError("rnn_linscan_blk supports k = 2, 4 and 8, got %d" % k)
    ws, n = _workspace(op, B, L, H, dev, ws=ws)
    _check(lib.rnn_linscan_blk(k, B, L, H, _ptr(A), _ptr(b), _ptr(h0), _ptr(h), _ptr(ws), n,
                               _stream(dev)), "rnn_linscan_blk")
    return h


def gru_forward(pz, pr, pc, uz, ur, uc, h0=None, *, tol=1e-4, max_iter=32, out=None,
                info=None, trace=None, ws=None, init=None):
    """Newton solve of the diagonal GRU over [B, L, H] gate pre-projections.

    Returns h [B, L, H].  `init` [B, L, H] is Newton's initial iterate (a warm
    start; None starts from zero; it must not share memory with the output).
    `info` (int32[2] device tensor) receives {iterations, converged}; `trace`
    (float32[max_iter]) receives max|delta| per iteration."""
    lib = load_library()
    B, L, H = pz.shape
    dev = pz.device
    for t, n in ((pz, "pz"), (pr, "pr"), (pc, "pc")):
        _need(t, (B, L, H), n, dev)
    for t, n in ((uz, "uz"), (ur, "ur"), (uc, "uc")):
        _need(t, (H,), n, dev)
    if h0 is not None:
        _need(h0, (B, H), "h0", dev)
    if init is not None:
        _need(init, (B, L, H), "init", dev)
    h = torch.empty_like(pz) if out is None else out
    _need(h, (B, L, H), "out", dev)
    if info is not None and (info.dtype != torch.int32 or info.numel() < 2 or info.device != dev):
        raise ValueError("info must be an int32 device tensor with 2 elements")
    if trace is not None and (trace.dtype != torch.float32 or trace.numel() < max_iter or
                              trace.device != dev):
        raise ValueError("trace must be a float32 device tensor with max_iter elements")
    ws, n = _workspace(OP_GRU_FORWARD, B, L, H, dev, max_iter, ws)
    _check(lib.pararnn_gru_forward(B, L, H, _ptr(pz), _ptr(pr), _ptr(pc), _ptr(uz), _ptr(ur),
                                   _ptr(uc), _ptr(h0), _ptr(init), _ptr(h), float(tol),
                                   int(max_iter), _ptr(info), _ptr(trace), _ptr(ws), n,
                                   _stream(dev)),
           "pararnn_gru_forward")
    return h


def lstm_forward(pi, pf, po, pg, ui, uf, uo, ug, h0=None, c0=None, *, tol=1e-4, max_iter=32,
                 out_h=None, out_c=None, info=None, trace=None, ws=None, init_h=None,
                 init_c=None):
    """Newton solve of the diagonal LSTM; returns (h, c), each [B, L, H].
    `init_h`, `init_c` [B, L, H]: Newton's initial iterates (a warm start; a
    missing one is zero; neither may share memory with the outputs)."""
    lib = load_library()
    B, L, H = pi.shape
    dev = pi.device
    for t, n in ((pi, "pi"), (pf, "pf"), (po, "po"), (pg, "pg")):
        _need(t, (B, L, H), n, dev)
    for t, n in ((ui, "ui"), (uf, "uf"), (uo, "uo"), (ug, "ug")):
        _need(t, (H,), n, dev)
    if h0 is not None:
        _need(h0, (B, H), "h0", dev)
    if c0 is not None:
        _need(c0, (B, H), "c0", dev)
    if init_h is not None:
        _need(init_h, (B, L, H), "init_h", dev)
    if init_c is not None:
        _need(init_c, (B, L, H), "init_c", dev)
    h = torch.empty_like(pi) if out_h is None else out_h
    c = torch.empty_like(pi) if out_c is None else out_c
    _need(h, (B, L, H), "out_h", dev)
    _need(c, (B, L, H), "out_c", dev)
    if info is not None and (info.dtype != torch.int32 or info.numel() < 2 or info.device != dev):
        raise ValueError("info must be an int32 device tensor with 2 elements")
    if trace is not None and (trace.dtype != torch.float32 or trace.numel() < max_iter or
                              trace.device != dev):
        raise ValueError("trace must be a float32 device tensor with max_iter elements")
    ws, n = _workspace(OP_LSTM_FORWARD, B, L, H, dev, max_iter, ws)
    _check(lib.pararnn_lstm_forward(B, L, H, _ptr(pi), _ptr(pf), _ptr(po), _ptr(pg), _ptr(ui),
                                    _ptr(uf), _ptr(uo), _ptr(ug), _ptr(h0), _ptr(c0),
                                    _ptr(init_h), _ptr(init_c), _ptr(h), _ptr(c), float(tol),
                                    int(max_iter), _ptr(info), _ptr(trace), _ptr(ws), n,
                                    _stream(dev)), "pararnn_lstm_forward")
    return h, c


def hgru_forward(pz, pr, pc, Uz, Ur, Uc, h0=None, *, tol=1e-4, max_iter=32, out=None, info=None,
                 trace=None, ws=None, init=None):
    """Newton solve of the GRU with dense recurrence inside heads of k
    channels (k = 4 or 8): p [B, L, NH, k], U [NH, k, k], h0 [B, NH, k];
    returns h [B, L, NH, k].  `init` is Newton's initial iterate (a warm
    start; it must not share memory with the output); `info`, `trace` as for
    gru_forward."""
    lib = load_library()
    B, L, NH, k = pz.shape
    dev = pz.device
    for t, n in ((pz, "pz"), (pr, "pr"), (pc, "pc")):
        _need(t, (B, L, NH, k), n, dev)
    for t, n in ((Uz, "Uz"), (Ur, "Ur"), (Uc, "Uc")):
        _need(t, (NH, k, k), n, dev)
    if h0 is not None:
        _need(h0, (B, NH, k), "h0", dev)
    if init is not None:
        _need(init, (B, L, NH, k), "init", dev)
    op = {4: OP_HGRU4_FORWARD, 8: OP_HGRU8_FORWARD}.get(k)
    if op is None:
        raise PararnnError("pararnn_hgru_forward supports k = 4 and 8, got %d" % k)
    h = torch.empty_like(pz) if out is None else out
    _need(h, (B, L, NH, k), "out", dev)
    if info is not None and (info.dtype != torch.int32 or info.numel() < 2 or info.device != dev):
        raise ValueError("info must be an int32 device tensor with 2 elements")
    if trace is not None and (trace.dtype != torch.float32 or trace.numel() < max_iter or
                              trace.device != dev):
        raise ValueError("trace must be a float32 device tensor with max_iter elements")
    ws, n = _workspace(op, B, L, NH, dev, max_iter, ws)
    _check(lib.pararnn_hgru_forward(k, B, L, NH, _ptr(pz), _ptr(pr), _ptr(pc), _ptr(Uz), _ptr(Ur),
                                    _ptr(Uc), _ptr(h0), _ptr(init), _ptr(h), float(tol), int(max_iter),
                                    _ptr(info), _ptr(trace), _ptr(ws), n, _stream(dev)),
           "pararnn_hgru_forward")
    return h


def hgru_backward(pz, pr, pc, Uz, Ur, Uc, h0, h, grad_h, *, want_u=True, want_h0=True, ws=None, out=None):
    """Gradients of sum(grad_h * h) through the head-GRU solve h (the
    converged output of hgru_forward): returns (dpz, dpr, dpc, dUz, dUr, dUc,
    dh0), the U gradients None unless want_u, dh0 None unless want_h0.
    `out`: the seven output tensors to write instead (None entries for the
    gradients not wanted)."""
    lib = load_library()
    B, L, NH, k = pz.shape
    dev = pz.device
    for t, n in ((pz, "pz"), (pr, "pr"), (pc, "pc"), (h, "h"), (grad_h, "grad_h")):
        _need(t, (B, L, NH, k), n, dev)
    for t, n in ((Uz, "Uz"), (Ur, "Ur"), (Uc, "Uc")):
        _need(t, (NH, k, k), n, dev)
    if h0 is not None:
        _need(h0, (B, NH, k), "h0", dev)
    op = {4: OP_HGRU4_BACKWARD, 8: OP_HGRU8_BACKWARD}.get(k)
    if op is None:
        raise PararnnError("pararnn_hgru_backward supports k = 4 and 8, got %d" % k)
    if out is not None:
        gp, gU, gh0 = list(out[:3]), list(out[3:6]), out[6]
        for t, n in zip(gp, ("dpz", "dpr", "dpc")):
            _need(t, (B, L, NH, k), n, dev)
        for t, n in zip(gU, ("dUz", "dUr", "dUc")):
            if t is not None:
                _need(t, (NH, k, k), n, dev)
        if gh0 is not None:
            _need(gh0, (B, NH, k), "dh0", dev)
    else:
        gp = [torch.empty_like(pz) for _ in range(3)]
        gU = [torch.empty_like(Uz) for _ in range(3)] if want_u else [None] * 3
        gh0 = torch.empty(B, NH, k, device=dev) if want_h0 else None
    ws, n = _workspace(op, B, L, NH, dev, 1, ws)
    _check(lib.pararnn_hgru_backward(k, B, L, NH, _ptr(pz), _ptr(pr), _ptr(pc), _ptr(Uz), _ptr(Ur), _ptr(Uc),
                                     _ptr(h0), _ptr(h), _ptr(grad_h), _ptr(gp[0]), _ptr(gp[1]), _ptr(gp[2]),
                                     _ptr(gU[0]), _ptr(gU[1]), _ptr(gU[2]), _ptr(gh0), _ptr(ws), n, _stream(dev)),
           "pararnn_hgru_backward")
    return (*gp, *gU, gh0)


def gru_forward_noalloc(pz, pr, pc, uz, ur, uc, h0=None, *, tol=1e-4, max_iter=32, out=None,
                        info=None, trace=None):
    """gru_forward with the library's static scratch buffer as workspace
    (pararnn_gru_forward_noalloc): the call allocates nothing on the device
    when `out` is given."""
    lib = load_library()
    B, L, H = pz.shape
    dev = pz.device
    for t, n in ((pz, "pz"), (pr, "pr"), (pc, "pc")):
        _need(t, (B, L, H), n, dev)
    for t, n in ((uz, "uz"), (ur, "ur"), (uc, "uc")):
        _need(t, (H,), n, dev)
    if h0 is not None:
        _need(h0, (B, H), "h0", dev)
    h = torch.empty_like(pz) if out is None else out
    _need(h, (B, L, H), "out", dev)
    if info is not None and (info.dtype != torch.int32 or info.numel() < 2 or info.device != dev):
        raise ValueError("info must be an int32 device tensor with 2 elements")
    if trace is not None and (trace.dtype != torch.float32 or trace.numel() < max_iter or
                              trace.device != dev):
        raise ValueError("trace must be a float32 device tensor with max_iter elements")
    _check(lib.pararnn_gru_forward_noalloc(B, L, H, _ptr(pz), _ptr(pr), _ptr(pc), _ptr(uz), _ptr(ur),
                                           _ptr(uc), _ptr(h0), _ptr(h), float(tol), int(max_iter),
                                           _ptr(info), _ptr(trace), _stream(dev)),
           "pararnn_gru_forward_noalloc")
    return h


# ---------------------------------------------------------------- sequential
def gru_sequential(pz, pr, pc, uz, ur, uc, h0=None, *, out=None):
    """Sequential application of the GRU cell (one thread per channel, one
    cell per position); returns h [B, L, H]."""
    lib = load_library()
    B, L, H = pz.shape
    dev = pz.device
    for t, n in ((pz, "pz"), (pr, "pr"), (pc, "pc")):
        _need(t, (B, L, H), n, dev)
    for t, n in ((uz, "uz"), (ur, "ur"), (uc, "uc")):
        _need(t, (H,), n, dev)
    if h0 is not None:
        _need(h0, (B, H), "h0", dev)
    h = torch.empty_like(pz) if out is None else out
    _need(h, (B, L, H), "out", dev)
    _check(lib.pararnn_gru_sequential(B, L, H, _ptr(pz), _ptr(pr), _ptr(pc), _ptr(uz), _ptr(ur),
                                      _ptr(uc), _ptr(h0), _ptr(h), _stream(dev)),
           "pararnn_gru_sequential")
    return h


def lstm_sequential(pi, pf, po, pg, ui, uf, uo, ug, h0=None, c0=None, *, out_h=None, out_c=None):
    """Sequential application of the LSTM cell; returns (h, c), each [B, L, H]."""
    lib = load_library()
    B, L, H = pi.shape
    dev = pi.device
    for t, n in ((pi, "pi"), (pf, "pf"), (po, "po"), (pg, "pg")):
        _need(t, (B, L, H), n, dev)
    for t, n in ((ui, "ui"), (uf, "uf"), (uo, "uo"), (ug, "ug")):
        _need(t, (H,), n, dev)
    if h0 is not None:
        _need(h0, (B, H), "h0", dev)
    if c0 is not None:
        _need(c0, (B, H), "c0", dev)
    h = torch.empty_like(pi) if out_h is None else out_h
    c = torch.empty_like(pi) if out_c is None else out_c
    _need(h, (B, L, H), "out_h", dev)
    _need(c, (B, L, H), "out_c", dev)
    _check(lib.pararnn_lstm_sequential(B, L, H, _ptr(pi), _ptr(pf), _ptr(po), _ptr(pg), _ptr(ui),
                                       _ptr(uf), _ptr(uo), _ptr(ug), _ptr(h0), _ptr(c0), _ptr(h),
                                       _ptr(c), _stream(dev)), "pararnn_lstm_sequential")
    return h, c


# ---------------------------------------------------------------- adjoint
def adjoint_backward(cell: int, p: Sequence[torch.Tensor], u: Sequence[torch.Tensor],
                     h: torch.Tensor, grad_h: torch.Tensor, h0=None, *, c=None, c0=None,
                     grad_c=None, want_u=True, want_h0=True, want_c0=True, ws=None):
    """Reverse-time adjoint of the converged solve.  Returns a dict with
    'p' (list of [B, L, H]), 'u' (list of [H] or None), 'h0', 'c0'."""
    lib = load_library()
    ng = 3 if cell == CELL_GRU else 4
    if len(p) != ng or len(u) != ng:
        raise ValueError("expected %d gate tensors" % ng)
    B, L, H = h.shape
    dev = h.device
    for k, t in enumerate(p):
        _need(t, (B, L, H), "p[%d]" % k, dev)
    for k, t in enumerate(u):
        _need(t, (H,), "u[%d]" % k, dev)
    _need(h, (B, L, H), "h", dev)
    _need(grad_h, (B, L, H), "grad_h", dev)
    if h0 is not None:
        _need(h0, (B, H), "h0", dev)
    if cell == CELL_LSTM:
        _need(c, (B, L, H), "c", dev)
        if c0 is not None:
            _need(c0, (B, H), "c0", dev)
        if grad_c is not None:
            _need(grad_c, (B, L, H), "grad_c", dev)
    gp = [torch.empty_like(h) for _ in range(ng)]
    gu = [torch.empty(H, dtype=torch.float32, device=dev) for _ in range(ng)] if want_u else None
    gh0 = torch.empty(B, H, dtype=torch.float32, device=dev) if want_h0 else None
    gc0 = torch.empty(B, H, dtype=torch.float32, device=dev) if (want_c0 and cell == CELL_LSTM) else None
    op = OP_GRU_ADJOINT if cell == CELL_GRU else OP_LSTM_ADJOINT
    ws, n = _workspace(op, B, L, H, dev, ws=ws)
    P = (ctypes.c_void_p * ng)(*[t.data_ptr() for t in p])
    U = (ctypes.c_void_p * ng)(*[t.data_ptr() for t in u])
    GP = (ctypes.c_void_p * ng)(*[t.data_ptr() for t in gp])
    GU = (ctypes.c_void_p * ng)(*[t.data_ptr() for t in gu]) if gu is not None else None
    _check(lib.pararnn_adjoint_backward(cell, B, L, H, P, U, _ptr(h0), _ptr(c0), _ptr(h), _ptr(c),
                                        _ptr(grad_h), _ptr(grad_c), GP, GU, _ptr(gh0), _ptr(gc0),
                                        _ptr(ws), n, _stream(dev)), "pararnn_adjoint_backward")
    return {"p": gp, "u": gu, "h0": gh0, "c0": gc0}
