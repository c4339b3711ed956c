"""Newton solve for user-defined cells with a diagonal Jacobian.

A cell is any function ``cell(h_prev, *inputs, *params) -> h`` written with
torch operations that acts channel by channel: output channel j depends on
channel j of ``h_prev`` only (and on anything in the inputs and parameters).
The whole sequence h_t = cell(h_{t-1}, x_t) is then solved by Newton's method
(ParaRNN page, TL;DR and abstract: Newton iterations on the whole-sequence
system; a framework for parallelising new nonlinear RNNs; DEER summary page,
method paragraph: the same for any differentiable recurrence, tolerance the
only extra hyper-parameter).  This is the modality in which the system is
assembled by the framework's tensor operations and only the parallel
reduction runs in a dedicated kernel (ParaRNN page, Fig. 5 caption): each
iteration evaluates the cell and its diagonal Jacobian with torch
(forward-mode differentiation with a tangent of ones gives the diagonal), and
solves the bi-diagonal linear system with the library's diagonal scan
(rnn_linscan_diag).  Cells with a built-in kernel (GRU, LSTM) are much
faster through pararnn_gru_forward / pararnn_lstm_forward.

Gradients come from the adjoint of the converged solve (DEER summary page:
forward plus gradients): lambda_t = g_t + J_{t+1} lambda_{t+1}, a reverse
diagonal scan, again on the library's kernel, then one vector-Jacobian
product of the cell for the inputs, parameters and h0.

Each iteration reads max|delta| on the host to decide whether to stop, so a
solve synchronises once per iteration.  There is no CPU path: the scans run
only on a HIP device.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence

import torch

from . import api


def _shift(s: torch.Tensor, h0: torch.Tensor) -> torch.Tensor:
    """States before each position: [h0, s_0, ..., s_{L-2}]."""
    return torch.cat([h0.unsqueeze(1), s[:, :-1]], dim=1)


def _cell_and_diag(cell, hp, inputs, params):
    """cell(hp, ...) and its diagonal Jacobian by hp (forward mode, tangent 1)."""
    f = lambda h: cell(h, *inputs, *params)  # noqa: E731
    return torch.func.jvp(f, (hp,), (torch.ones_like(hp),))


def _solve(cell, inputs, params, h0, tol, max_iter, info):
    s = torch.zeros_like(inputs[0])
    it, conv = 0, False
    with torch.no_grad():
        for k in range(1, max_iter + 1):
            F, J = _cell_and_diag(cell, _shift(s, h0), inputs, params)
            delta = api.linscan_diag(J.contiguous(), (F - s).contiguous())
            s += delta
            it = k
            e = torch.nan_to_num(delta.abs().max(), nan=float("inf")).item()
            if e <= tol:
                conv = True
                break
    if info is not None:
        info[0], info[1] = it, int(conv)
    return s


class _DiagonalSolve(torch.autograd.Function):
    @staticmethod
    def forward(ctx, cell, tol, max_iter, info, n_inputs, h0, *tensors):
        inputs, params = tensors[:n_inputs], tensors[n_inputs:]
        s = _solve(cell, inputs, params, h0, tol, max_iter, info)
        ctx.cell, ctx.n_inputs = cell, n_inputs
        ctx.save_for_backward(h0, s, *tensors)
        return s

    @staticmethod
    def backward(ctx, g):
        h0, s, *tensors = ctx.saved_tensors
        inputs, params = tensors[:ctx.n_inputs], tensors[ctx.n_inputs:]
        with torch.no_grad():
            _, J = _cell_and_diag(ctx.cell, _shift(s, h0), inputs, params)
            # lambda_t = g_t + J_{t+1} lambda_{t+1}: a diagonal scan in reversed time
            a = torch.cat([J[:, 1:], torch.zeros_like(J[:, :1])], dim=1)
            lam = api.linscan_diag(a.flip(1).contiguous(), g.flip(1).contiguous()).flip(1)
        # one vector-Jacobian product of the cell at the converged states
        with torch.enable_grad():
            h0_ = h0.detach().requires_grad_(ctx.needs_input_grad[5])
            ins = [x.detach().requires_grad_(True) for x in tensors]
            F = ctx.cell(_shift(s, h0_), *ins)
            wrt = [x for x in [h0_] + ins if x.requires_grad]
            grads = iter(torch.autograd.grad(F, wrt, grad_outputs=lam, allow_unused=True))
        gh0 = next(grads) if h0_.requires_grad else None
        gt = [next(grads) for _ in ins]
        gt = [torch.zeros_like(x) if gx is None else gx for x, gx in zip(tensors, gt)]
        return (None, None, None, None, None, gh0, *gt)


def newton_solve(cell: Callable[..., torch.Tensor], inputs: Sequence[torch.Tensor],
                 h0: Optional[torch.Tensor] = None, params: Sequence[torch.Tensor] = (), *,
                 tol: float = 1e-4, max_iter: int = 32,
                 info: Optional[list] = None) -> torch.Tensor:
    """Solve h_t = cell(h_{t-1}, *inputs_t, *params) over the whole sequence.

    inputs: tensors [B, L, H] (fp32, on a HIP device) passed to the cell
    position-wise; params: tensors the cell uses as they are (weights,
    broadcast against [B, L, H]); h0: [B, H] or None (zeros).  Newton starts
    from h = 0 and stops once max|delta| <= tol or after max_iter updates;
    `info`, if a list of two, receives [iterations, converged].  Returns h
    [B, L, H], differentiable with respect to inputs, params and h0 through
    the adjoint of the solve."""
    if not inputs:
        raise ValueError("at least one input sequence is needed")
    x0 = inputs[0]
    if x0.dim() != 3:
        raise ValueError("inputs must be [B, L, H]")
    if not tol >= 0.0 or max_iter < 1:
        raise ValueError("tol must be >= 0 and max_iter >= 1")
    B, L, H = x0.shape
    for x in inputs:
        if tuple(x.shape) != (B, L, H):
            raise ValueError("every input must be [B, L, H]")
    if h0 is None:
        h0 = torch.zeros(B, H, dtype=x0.dtype, device=x0.device)
    return _DiagonalSolve.apply(cell, float(tol), int(max_iter), info, len(inputs), h0,
                                *inputs, *params)
