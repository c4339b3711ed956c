"""fp64 CPU oracle for the Newton / parallel-scan RNN path.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (the HIP library and its Python binding) never touches it, and the two
share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, sequential order; see the
header of that file for the passages each function follows).  This module
only builds it with gcc, loads it with ctypes and converts numpy arrays.

Functions take numpy arrays of any float dtype (fp32 inputs are up-cast to
fp64 exactly) and return fp64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    vp = ctypes.c_void_p
    lib.orc_linscan_diag.argtypes = [_I64, _I64, _I64, vp, vp, vp, vp]
    lib.orc_linscan_blk2.argtypes = [_I64, _I64, _I64, vp, vp, vp, vp]
    lib.orc_linscan_blk.argtypes = [_I64, _I64, _I64, _I64, vp, vp, vp, vp]
    lib.orc_gru_cell.argtypes = [ctypes.c_double] * 7 + [vp, vp, vp, vp]
    lib.orc_lstm_cell.argtypes = [ctypes.c_double] * 10 + [vp, vp, vp, vp, vp]
    lib.orc_gru_rollout.argtypes = [_I64, _I64, _I64] + [vp] * 8
    lib.orc_lstm_rollout.argtypes = [_I64, _I64, _I64] + [vp] * 12
    lib.orc_gru_newton.argtypes = [_I64, _I64, _I64] + [vp] * 8 + [
        ctypes.c_double, ctypes.c_int, vp, vp, vp]
    lib.orc_gru_newton.restype = ctypes.c_int
    lib.orc_lstm_newton.argtypes = [_I64, _I64, _I64] + [vp] * 12 + [
        ctypes.c_double, ctypes.c_int, vp, vp, vp, vp]
    lib.orc_lstm_newton.restype = ctypes.c_int
    lib.orc_gru_bptt.argtypes = [_I64, _I64, _I64] + [vp] * 16
    lib.orc_lstm_bptt.argtypes = [_I64, _I64, _I64] + [vp] * 24
    lib.orc_hgru_cell.argtypes = [ctypes.c_int] + [vp] * 10
    lib.orc_hgru_rollout.argtypes = [_I64, _I64, _I64, ctypes.c_int] + [vp] * 8
    lib.orc_hgru_newton.argtypes = [_I64, _I64, _I64, ctypes.c_int] + [vp] * 8 + [
        ctypes.c_double, ctypes.c_int, vp, vp, vp]
    lib.orc_hgru_newton.restype = ctypes.c_int
    lib.orc_hgru_bptt.argtypes = [_I64, _I64, _I64, ctypes.c_int] + [vp] * 16
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x), dtype=np.float64)


def _p(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(int(n))


# ----------------------------------------------------------------- cells
def gru_cell(h, pz, pr, pc, uz, ur, uc):
    """Scalar GRU cell: returns (f, J, dfdp[3], gates[z, r, c])."""
    lib = _load()
    f = np.zeros(1)
    J = np.zeros(1)
    dp = np.zeros(3)
    gt = np.zeros(3)
    lib.orc_gru_cell(float(h), float(pz), float(pr), float(pc), float(uz),
                     float(ur), float(uc), _p(f), _p(J), _p(dp), _p(gt))
    return f[0], J[0], dp, gt


def lstm_cell(cp, hp, pi, pf, po, pg, ui, uf, uo, ug):
    """Scalar LSTM cell: returns (c, h, J[2x2], dcdp[4], dhdp[4]) (gates i, f, o, g)."""
    lib = _load()
    c = np.zeros(1)
    h = np.zeros(1)
    J = np.zeros(4)
    dc = np.zeros(4)
    dh = np.zeros(4)
    lib.orc_lstm_cell(float(cp), float(hp), float(pi), float(pf), float(po),
                      float(pg), float(ui), float(uf), float(uo), float(ug),
                      _p(c), _p(h), _p(J), _p(dc), _p(dh))
    return c[0], h[0], J.reshape(2, 2), dc, dh


# ----------------------------------------------------------------- scans
def linscan_diag(a, b, h0=None):
    a, b, h0 = _f64(a), _f64(b), _f64(h0)
    B, L, H = a.shape
    h = np.empty_like(a)
    _load().orc_linscan_diag(B, L, H, _p(a), _p(b), _p(h0), _p(h))
    return h


def linscan_blk2(A, b, h0=None):
    A, b, h0 = _f64(A), _f64(b), _f64(h0)
    B, L, H = b.shape[:3]
    assert A.shape == (B, L, H, 2, 2) and b.shape == (B, L, H, 2)
    h = np.empty_like(b)
    _load().orc_linscan_blk2(B, L, H, _p(A), _p(b), _p(h0), _p(h))
    return h


def linscan_blk(A, b, h0=None):
    """k x k block recurrence h_t = A_t h_{t-1} + b_t; A [B,L,H,k,k], b [B,L,H,k]."""
    A, b, h0 = _f64(A), _f64(b), _f64(h0)
    B, L, H, k = b.shape
    assert A.shape == (B, L, H, k, k) and 1 <= k <= 64
    if h0 is not None:
        assert h0.shape == (B, H, k)
    h = np.empty_like(b)
    _load().orc_linscan_blk(k, B, L, H, _p(A), _p(b), _p(h0), _p(h))
    return h


# ----------------------------------------------------------------- rollouts
def gru_rollout(pz, pr, pc, uz, ur, uc, h0=None):
    pz, pr, pc = _f64(pz), _f64(pr), _f64(pc)
    uz, ur, uc, h0 = _f64(uz), _f64(ur), _f64(uc), _f64(h0)
    B, L, H = pz.shape
    h = np.empty_like(pz)
    _load().orc_gru_rollout(B, L, H, _p(pz), _p(pr), _p(pc), _p(uz), _p(ur),
                            _p(uc), _p(h0), _p(h))
    return h


def lstm_rollout(pi, pf, po, pg, ui, uf, uo, ug, h0=None, c0=None):
    ps = [_f64(x) for x in (pi, pf, po, pg)]
    us = [_f64(x) for x in (ui, uf, uo, ug)]
    h0, c0 = _f64(h0), _f64(c0)
    B, L, H = ps[0].shape
    h = np.empty_like(ps[0])
    c = np.empty_like(ps[0])
    _load().orc_lstm_rollout(B, L, H, *[_p(x) for x in ps], *[_p(x) for x in us],
                             _p(h0), _p(c0), _p(h), _p(c))
    return h, c


# ----------------------------------------------------------------- Newton
def gru_newton(pz, pr, pc, uz, ur, uc, h0=None, tol=1e-6, cap=64, init=None):
    """CPU Newton from s = 0, or from the iterate `init` [B, L, H].  Returns
    (s, iterations, converged, trace[iters])."""
    pz, pr, pc = _f64(pz), _f64(pr), _f64(pc)
    uz, ur, uc, h0 = _f64(uz), _f64(ur), _f64(uc), _f64(h0)
    init = _f64(init)
    B, L, H = pz.shape
    assert init is None or init.shape == (B, L, H)
    s = np.empty_like(pz)
    conv = np.zeros(1, np.int32)
    trace = np.zeros(max(cap, 1))
    it = _load().orc_gru_newton(B, L, H, _p(pz), _p(pr), _p(pc), _p(uz),
                                _p(ur), _p(uc), _p(h0), _p(init), float(tol), int(cap),
                                _p(s), conv.ctypes.data_as(ctypes.c_void_p),
                                _p(trace))
    return s, int(it), int(conv[0]), trace[:it].copy()


def lstm_newton(pi, pf, po, pg, ui, uf, uo, ug, h0=None, c0=None, tol=1e-4, cap=32,
                h_init=None, c_init=None):
    """CPU Newton on (c, h) from 0, or from the iterates h_init, c_init
    [B, L, H] (zero where None).  Returns (h, c, iterations, converged, trace)."""
    ps = [_f64(x) for x in (pi, pf, po, pg)]
    us = [_f64(x) for x in (ui, uf, uo, ug)]
    h0, c0 = _f64(h0), _f64(c0)
    h_init, c_init = _f64(h_init), _f64(c_init)
    B, L, H = ps[0].shape
    h = np.empty_like(ps[0])
    c = np.empty_like(ps[0])
    conv = np.zeros(1, np.int32)
    trace = np.zeros(max(cap, 1))
    it = _load().orc_lstm_newton(B, L, H, *[_p(x) for x in ps], *[_p(x) for x in us],
                                 _p(h0), _p(c0), _p(h_init), _p(c_init), float(tol), int(cap),
                                 _p(h), _p(c),
                                 conv.ctypes.data_as(ctypes.c_void_p), _p(trace))
    return h, c, int(it), int(conv[0]), trace[:it].copy()


# ----------------------------------------------------------------- BPTT
def gru_bptt(pz, pr, pc, uz, ur, uc, h, g, h0=None):
    """Gradients of sum(g*h) w.r.t. (pz, pr, pc), (uz, ur, uc) and h0."""
    pz, pr, pc = _f64(pz), _f64(pr), _f64(pc)
    uz, ur, uc, h0 = _f64(uz), _f64(ur), _f64(uc), _f64(h0)
    h, g = _f64(h), _f64(g)
    B, L, H = pz.shape
    dp = [np.empty_like(pz) for _ in range(3)]
    du = [np.empty(H) for _ in range(3)]
    dh0 = np.empty((B, H))
    _load().orc_gru_bptt(B, L, H, _p(pz), _p(pr), _p(pc), _p(uz), _p(ur),
                         _p(uc), _p(h0), _p(h), _p(g), *[_p(x) for x in dp],
                         *[_p(x) for x in du], _p(dh0))
    return dp, du, dh0


def lstm_bptt(pi, pf, po, pg, ui, uf, uo, ug, h, c, gh, gc=None, h0=None, c0=None):
    """Gradients of sum(gh*h) + sum(gc*c) w.r.t. p (i, f, o, g), u and (h0, c0)."""
    ps = [_f64(x) for x in (pi, pf, po, pg)]
    us = [_f64(x) for x in (ui, uf, uo, ug)]
    h0, c0 = _f64(h0), _f64(c0)
    h, c, gh, gc = _f64(h), _f64(c), _f64(gh), _f64(gc)
    B, L, H = ps[0].shape
    dp = [np.empty_like(ps[0]) for _ in range(4)]
    du = [np.empty(H) for _ in range(4)]
    dh0 = np.empty((B, H))
    dc0 = np.empty((B, H))
    _load().orc_lstm_bptt(B, L, H, *[_p(x) for x in ps], *[_p(x) for x in us],
                          _p(h0), _p(c0), _p(h), _p(c), _p(gh), _p(gc),
                          *[_p(x) for x in dp], *[_p(x) for x in du], _p(dh0), _p(dc0))
    return dp, du, dh0, dc0


# ----------------------------------------------------------------- head GRU
def hgru_cell(h, pz, pr, pc, Uz, Ur, Uc):
    """One step of the GRU with dense recurrence inside a head of k channels:
    vectors [k], matrices [k, k].  Returns (f [k], J [k, k], gates [4, k] =
    z, r, c, r*h)."""
    h, pz, pr, pc = _f64(h), _f64(pz), _f64(pr), _f64(pc)
    Uz, Ur, Uc = _f64(Uz), _f64(Ur), _f64(Uc)
    k = h.shape[0]
    f = np.zeros(k)
    J = np.zeros((k, k))
    gt = np.zeros((4, k))
    _load().orc_hgru_cell(k, _p(h), _p(pz), _p(pr), _p(pc), _p(Uz), _p(Ur), _p(Uc),
                          _p(f), _p(J), _p(gt))
    return f, J, gt


def hgru_rollout(pz, pr, pc, Uz, Ur, Uc, h0=None):
    """Sequential head GRU: p [B, L, NH, k], U [NH, k, k], h0 [B, NH, k]."""
    pz, pr, pc = _f64(pz), _f64(pr), _f64(pc)
    Uz, Ur, Uc, h0 = _f64(Uz), _f64(Ur), _f64(Uc), _f64(h0)
    B, L, NH, k = pz.shape
    assert k <= 8 and Uz.shape == (NH, k, k)
    h = np.empty_like(pz)
    _load().orc_hgru_rollout(B, L, NH, k, _p(pz), _p(pr), _p(pc), _p(Uz), _p(Ur), _p(Uc),
                             _p(h0), _p(h))
    return h


def hgru_newton(pz, pr, pc, Uz, Ur, Uc, h0=None, tol=1e-6, cap=64, init=None):
    """CPU Newton for the head GRU from s = 0 or from `init` (k x k block
    Jacobians).  Returns (s, iterations, converged, trace[iters])."""
    pz, pr, pc = _f64(pz), _f64(pr), _f64(pc)
    Uz, Ur, Uc, h0 = _f64(Uz), _f64(Ur), _f64(Uc), _f64(h0)
    init = _f64(init)
    B, L, NH, k = pz.shape
    s = np.empty_like(pz)
    conv = np.zeros(1, np.int32)
    trace = np.zeros(max(cap, 1))
    it = _load().orc_hgru_newton(B, L, NH, k, _p(pz), _p(pr), _p(pc), _p(Uz), _p(Ur), _p(Uc),
                                 _p(h0), _p(init), float(tol), int(cap), _p(s),
                                 conv.ctypes.data_as(ctypes.c_void_p), _p(trace))
    return s, int(it), int(conv[0]), trace[:it].copy()


def hgru_bptt(pz, pr, pc, Uz, Ur, Uc, h, g, h0=None):
    """Gradients of sum(g * h) through the head GRU rollout h.  Returns
    (dpz, dpr, dpc, dUz, dUr, dUc, dh0)."""
    pz, pr, pc = _f64(pz), _f64(pr), _f64(pc)
    Uz, Ur, Uc, h0 = _f64(Uz), _f64(Ur), _f64(Uc), _f64(h0)
    h, g = _f64(h), _f64(g)
    B, L, NH, k = pz.shape
    dp = [np.empty_like(pz) for _ in range(3)]
    dU = [np.empty_like(Uz) for _ in range(3)]
    dh0 = np.empty((B, NH, k))
    _load().orc_hgru_bptt(B, L, NH, k, _p(pz), _p(pr), _p(pc), _p(Uz), _p(Ur), _p(Uc),
                          _p(h0), _p(h), _p(g), *[_p(x) for x in dp], *[_p(x) for x in dU],
                          _p(dh0))
    return (*dp, *dU, dh0)
