"""Newton solve for user-defined cells whose Jacobian is diagonal over the
channels: one state value per channel (diagonal Jacobian) or two (2x2 blocks).

A cell is any function ``cell(s_prev, *inputs, *params) -> s`` written with
torch operations that acts channel by channel: the state of channel j depends
on the state of channel j only (and on anything in the inputs and
parameters).  With ``state_size=1`` states are [B, L, H]; with
``state_size=2`` they are [B, L, H, 2] (an LSTM-like cell with (c, h) per
channel).  The whole sequence s_t = cell(s_{t-1}, x_t) is then solved by
Newton's method (ParaRNN page, TL;DR and abstract: Newton iterations on the
whole-sequence system, diagonal and 2x2 block-diagonal Jacobians; a framework
for parallelising new nonlinear RNNs; DEER summary page, method paragraph:
the same for any differentiable recurrence, tolerance the only extra
hyper-parameter).  This is the modality in which the system is assembled by
the framework's tensor operations and only the parallel reduction runs in a
dedicated kernel (ParaRNN page, Fig. 5 caption): each iteration evaluates the
cell and its Jacobian blocks with torch (forward-mode differentiation, one
tangent per state component), and solves the block bi-diagonal linear system
with the library's diagonal or 2x2 scan (rnn_linscan_diag, rnn_linscan_blk2).
Cells with a built-in kernel (GRU, LSTM) are much faster through
pararnn_gru_forward / pararnn_lstm_forward.

Stopping: the convergence decision is taken on the device.  Each iteration
computes max|delta| there and clears a device flag once it is <= tol; every
later update is multiplied by that flag, so it changes nothing, and the
iteration count is summed on the device too.  The host copies the flag to
pinned memory without blocking and looks at it one iteration late: while it
waits for iteration k's flag, iteration k+1 is already queued, so the device
never idles on the host.  The solve enqueues at most one iteration past
convergence, whose update is discarded.

Gradients come from the adjoint of the converged solve (DEER summary page:
forward plus gradients): lambda_t = g_t + J_{t+1}^T lambda_{t+1}, a reverse
scan on the same kernels, then one vector-Jacobian product of the cell for
the inputs, parameters and the initial state.  There is no CPU path: the
scans run only on a HIP device.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence

import torch

from . import api


def _shift(s: torch.Tensor, h0: torch.Tensor) -> torch.Tensor:
    """States before each position: [h0, s_0, ..., s_{L-2}]."""
    return torch.cat([h0.unsqueeze(1), s[:, :-1]], dim=1)


def _cell_and_jacobian(cell, sp, inputs, params, k):
    """cell(sp, ...) and its Jacobian blocks by sp: [B, L, H] for one
    component, [B, L, H, 2, 2] (row i, column l = dF_i/ds_l) for two."""
    f = lambda s: cell(s, *inputs, *params)  # noqa: E731
    if k == 1:
        return torch.func.jvp(f, (sp,), (torch.ones_like(sp),))
    cols = []
    F = None
    for l in range(k):
        t = torch.zeros_like(sp)
        t[..., l] = 1.0
        F, c = torch.func.jvp(f, (sp,), (t,))
        cols.append(c)
    return F, torch.stack(cols, dim=-1)


def _scan(J, b, k):
    if k == 1:
        return api.linscan_diag(J.contiguous(), b.contiguous())
    return api.linscan_blk2(J.contiguous(), b.contiguous())


def _solve(cell, inputs, params, h0, tol, max_iter, info, k):
    B, L, H = inputs[0].shape
    shape = (B, L, H) if k == 1 else (B, L, H, k)
    s = torch.zeros(shape, dtype=inputs[0].dtype, device=inputs[0].device)
    dev = s.device
    active = torch.ones((), dtype=torch.float32, device=dev)   # 1 until converged
    its = torch.zeros((), dtype=torch.int32, device=dev)       # updates applied
    flags = torch.empty(max_iter, dtype=torch.float32, pin_memory=True)
    done = []
    with torch.no_grad():
        for n in range(max_iter):
            F, J = _cell_and_jacobian(cell, _shift(s, h0), inputs, params, k)
            delta = _scan(J, F - s, k)
            e = torch.nan_to_num(delta.abs().amax(), nan=float("inf"))
            s.add_(delta * active)
            its.add_(active.to(torch.int32))
            active.mul_((e > tol).to(torch.float32))
            flags[n].copy_(active, non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            done.append(ev)
            if n >= 1:
                done[n - 1].synchronize()
                if flags[n - 1].item() == 0.0:
                    break  # converged at iteration n; iteration n + 1 changed nothing
    if info is not None:
        info[0], info[1] = int(its.item()), int(active.item() == 0.0)
    return s


class _BlockDiagonalSolve(torch.autograd.Function):
    @staticmethod
    def forward(ctx, cell, tol, max_iter, info, k, n_inputs, h0, *tensors):
        inputs, params = tensors[:n_inputs], tensors[n_inputs:]
        s = _solve(cell, inputs, params, h0, tol, max_iter, info, k)
        ctx.cell, ctx.n_inputs, ctx.k = cell, n_inputs, k
        ctx.save_for_backward(h0, s, *tensors)
        return s

    @staticmethod
    def backward(ctx, g):
        h0, s, *tensors = ctx.saved_tensors
        inputs, params = tensors[:ctx.n_inputs], tensors[ctx.n_inputs:]
        k = ctx.k
        with torch.no_grad():
            _, J = _cell_and_jacobian(ctx.cell, _shift(s, h0), inputs, params, k)
            if k > 1:
                J = J.transpose(-1, -2)
            # lambda_t = g_t + J_{t+1}^T lambda_{t+1}: a scan in reversed time
            a = torch.cat([J[:, 1:], torch.zeros_like(J[:, :1])], dim=1)
            lam = _scan(a.flip(1), g.flip(1), k).flip(1)
        # one vector-Jacobian product of the cell at the converged states
        with torch.enable_grad():
            h0_ = h0.detach().requires_grad_(ctx.needs_input_grad[6])
            ins = [x.detach().requires_grad_(True) for x in tensors]
            F = ctx.cell(_shift(s, h0_), *ins)
            wrt = [x for x in [h0_] + ins if x.requires_grad]
            grads = iter(torch.autograd.grad(F, wrt, grad_outputs=lam, allow_unused=True))
        gh0 = next(grads) if h0_.requires_grad else None
        gt = [next(grads) for _ in ins]
        gt = [torch.zeros_like(x) if gx is None else gx for x, gx in zip(tensors, gt)]
        return (None, None, None, None, None, None, gh0, *gt)


def newton_solve(cell: Callable[..., torch.Tensor], inputs: Sequence[torch.Tensor],
                 h0: Optional[torch.Tensor] = None, params: Sequence[torch.Tensor] = (), *,
                 tol: float = 1e-4, max_iter: int = 32, info: Optional[list] = None,
                 state_size: int = 1) -> torch.Tensor:
    """Solve s_t = cell(s_{t-1}, *inputs_t, *params) over the whole sequence.

    inputs: tensors [B, L, H] (fp32, on a HIP device) passed to the cell
    position-wise; params: tensors the cell uses as they are (weights,
    broadcast against the state); state_size: 1 (states [B, L, H]) or 2
    (states [B, L, H, 2]); h0: [B, H] or [B, H, 2], or None (zeros).  Newton
    starts from s = 0 and stops once max|delta| <= tol or after max_iter
    updates; `info`, if a list of two, receives [iterations, converged].
    Returns the states, differentiable with respect to inputs, params and h0
    through the adjoint of the solve."""
    if not inputs:
        raise ValueError("at least one input sequence is needed")
    if state_size not in (1, 2):
        raise ValueError("state_size must be 1 or 2")
    x0 = inputs[0]
    if x0.device.type != "cuda":
        raise ValueError("newton_solve runs on a HIP device only; inputs are on %s" % x0.device)
    if x0.dim() != 3:
        raise ValueError("inputs must be [B, L, H]")
    if not tol >= 0.0 or max_iter < 1:
        raise ValueError("tol must be >= 0 and max_iter >= 1")
    B, L, H = x0.shape
    for x in inputs:
        if tuple(x.shape) != (B, L, H):
            raise ValueError("every input must be [B, L, H]")
    hshape = (B, H) if state_size == 1 else (B, H, state_size)
    if h0 is None:
        h0 = torch.zeros(hshape, dtype=x0.dtype, device=x0.device)
    elif tuple(h0.shape) != hshape:
        raise ValueError("h0 must be %s" % (hshape,))
    return _BlockDiagonalSolve.apply(cell, float(tol), int(max_iter), info, state_size,
                                     len(inputs), h0, *inputs, *params)
