"""Trainable diagonal GRU and LSTM layers on top of the Newton solve.

The recurrence is evaluated over the whole sequence at once by Newton's
method (ParaRNN page, TL;DR and Fig. 2; DEER summary page, first paragraph),
and its gradients come back through the converged solve by the reverse-time
adjoint scan (DEER summary page: forward plus gradients).  Both run in
libpararnn.so; the layers only add what sits on either side of them:

  - the input projections p_g = x W_g^T + b_g (one fp32 GEMM per gate, on the
    library GEMM of torch), whose outputs are the gate pre-projections the
    C ABI takes, and their gradients dL/dW_g, dL/db_g, dL/dx from dL/dp_g;
  - the diagonal recurrent weights u_g ([H] per gate, ParaRNN page, Fig. 2
    caption: diagonal recurrence for the GRU-style cell, 2x2 blocks for the
    LSTM-style one), whose gradients the adjoint returns directly.

The gradients are those of the sequence the solve converged to; they equal
backpropagation through the sequential rollout once Newton has converged
(with tol = 0 and the cap at L + 1 exactly, up to rounding).  `last_info`
holds the solve's {iterations, converged} as an int32 device tensor, so
reading it is the caller's choice of synchronisation point.

There is no CPU path: the solve raises unless its inputs are float32 tensors
on a HIP device.
"""
from __future__ import annotations

import math
from typing import Optional

import torch
import torch.nn.functional as F

from . import api


class GruSolve(torch.autograd.Function):
    """h = Newton solve of the diagonal GRU on gate pre-projections (pz, pr, pc),
    with the adjoint as its backward."""

    @staticmethod
    def forward(ctx, pz, pr, pc, uz, ur, uc, h0, tol, max_iter, info):
        h = api.gru_forward(pz, pr, pc, uz, ur, uc, h0, tol=tol, max_iter=max_iter, info=info)
        ctx.save_for_backward(pz, pr, pc, uz, ur, uc, h0, h)
        ctx.set_materialize_grads(False)
        return h

    @staticmethod
    def backward(ctx, gh):
        pz, pr, pc, uz, ur, uc, h0, h = ctx.saved_tensors
        need = ctx.needs_input_grad
        if gh is None:
            return (None,) * 10
        g = api.adjoint_backward(api.CELL_GRU, [pz, pr, pc], [uz, ur, uc], h, gh.contiguous(), h0,
                                 want_u=any(need[3:6]), want_h0=h0 is not None and need[6])
        gu = g["u"] if g["u"] is not None else [None] * 3
        return (*g["p"], *gu, g["h0"], None, None, None)


class LstmSolve(torch.autograd.Function):
    """(h, c) = Newton solve of the diagonal LSTM on gate pre-projections
    (pi, pf, po, pg), with the adjoint as its backward."""

    @staticmethod
    def forward(ctx, pi, pf, po, pg, ui, uf, uo, ug, h0, c0, tol, max_iter, info):
        h, c = api.lstm_forward(pi, pf, po, pg, ui, uf, uo, ug, h0, c0, tol=tol,
                                max_iter=max_iter, info=info)
        ctx.save_for_backward(pi, pf, po, pg, ui, uf, uo, ug, h0, c0, h, c)
        ctx.set_materialize_grads(False)
        return h, c

    @staticmethod
    def backward(ctx, gh, gc):
        pi, pf, po, pg, ui, uf, uo, ug, h0, c0, h, c = ctx.saved_tensors
        need = ctx.needs_input_grad
        if gh is None and gc is None:
            return (None,) * 13
        gh = torch.zeros_like(h) if gh is None else gh.contiguous()
        gc = None if gc is None else gc.contiguous()
        g = api.adjoint_backward(api.CELL_LSTM, [pi, pf, po, pg], [ui, uf, uo, ug], h, gh, h0,
                                 c=c, c0=c0, grad_c=gc, want_u=any(need[4:8]),
                                 want_h0=h0 is not None and need[8],
                                 want_c0=c0 is not None and need[9])
        gu = g["u"] if g["u"] is not None else [None] * 4
        return (*g["p"], *gu, g["h0"], g["c0"], None, None, None)


def _uniform_(t: torch.Tensor, k: float):
    with torch.no_grad():
        t.uniform_(-k, k)


class _DiagonalRnn(torch.nn.Module):
    NG = 0

    def __init__(self, input_size: int, hidden_size: int, *, bias: bool = True, tol: float = 1e-4,
                 max_iter: int = 32, device=None):
        super().__init__()
        if input_size < 1 or hidden_size < 1:
            raise ValueError("input_size and hidden_size must be positive")
        if not tol >= 0.0 or max_iter < 1:
            raise ValueError("tol must be >= 0 and max_iter >= 1")
        self.input_size, self.hidden_size = int(input_size), int(hidden_size)
        self.tol, self.max_iter = float(tol), int(max_iter)
        f32 = dict(dtype=torch.float32, device=device)
        # gate-major, so every gate's slice is a contiguous [H, D], [H] or [H]
        self.weight = torch.nn.Parameter(torch.empty(self.NG, hidden_size, input_size, **f32))
        self.bias = torch.nn.Parameter(torch.empty(self.NG, hidden_size, **f32)) if bias else None
        self.u = torch.nn.Parameter(torch.empty(self.NG, hidden_size, **f32))
        self.last_info: Optional[torch.Tensor] = None
        self.reset_parameters()

    def reset_parameters(self):
        # the classical recurrent layers' range, U(-1/sqrt(H), 1/sqrt(H))
        k = 1.0 / math.sqrt(self.hidden_size)
        _uniform_(self.weight, k)
        _uniform_(self.u, k)
        if self.bias is not None:
            _uniform_(self.bias, k)

    def project(self, x: torch.Tensor):
        """Gate pre-projections [B, L, H] (contiguous), one GEMM per gate."""
        if x.dim() != 3 or x.shape[-1] != self.input_size:
            raise ValueError("x must be [B, L, %d], got %s" % (self.input_size, tuple(x.shape)))
        return [F.linear(x, self.weight[g], None if self.bias is None else self.bias[g])
                for g in range(self.NG)]

    def _info(self, x):
        self.last_info = torch.zeros(2, dtype=torch.int32, device=x.device)
        return self.last_info

    def extra_repr(self):
        return "%d, %d, bias=%s, tol=%g, max_iter=%d" % (
            self.input_size, self.hidden_size, self.bias is not None, self.tol, self.max_iter)


class ParaGRU(_DiagonalRnn):
    """Diagonal GRU-style layer (ParaGRU; gates z, r, c):

        z = sigmoid(pz + uz*h), r = sigmoid(pr + ur*h),
        c = tanh(pc + uc*(r*h)), h' = (1 - z)*h + z*c,   p_g = x W_g^T + b_g.

    forward(x [B, L, D], h0 [B, H] or None) -> h [B, L, H]."""
    NG = 3

    def forward(self, x: torch.Tensor, h0: Optional[torch.Tensor] = None) -> torch.Tensor:
        pz, pr, pc = self.project(x)
        return GruSolve.apply(pz, pr, pc, self.u[0], self.u[1], self.u[2], h0, self.tol,
                              self.max_iter, self._info(x))


class ParaLSTM(_DiagonalRnn):
    """Diagonal LSTM-style layer (ParaLSTM; gates i, f, o, g, state (c, h)):

        i, f, o = sigmoid(p + u*h'), g = tanh(pg + ug*h'),
        c = f*c' + i*g, h = o*tanh(c),   p_g = x W_g^T + b_g.

    forward(x [B, L, D], h0, c0 [B, H] or None) -> (h, c), each [B, L, H]."""
    NG = 4

    def forward(self, x: torch.Tensor, h0: Optional[torch.Tensor] = None,
                c0: Optional[torch.Tensor] = None):
        pi, pf, po, pg = self.project(x)
        return LstmSolve.apply(pi, pf, po, pg, self.u[0], self.u[1], self.u[2], self.u[3], h0, c0,
                               self.tol, self.max_iter, self._info(x))
