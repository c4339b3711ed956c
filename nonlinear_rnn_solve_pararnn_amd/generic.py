"""Newton solve for user-defined cells whose Jacobian is block-diagonal over
the channels: one state value per channel (diagonal Jacobian), or k per
channel or head (k x k blocks, k = 2, 4 or 8).

A cell is any function ``cell(s_prev, *inputs, *params) -> s`` written with
torch operations whose state of channel (or head) j depends on the state of
j only (and on anything in the inputs and parameters).  With
``state_size=1`` states are [B, L, H]; with ``state_size=k`` they are
[B, L, H, k]: an LSTM-like cell with (c, h) per channel (k = 2), or a cell
with dense recurrence inside heads of k channels (head_gru_cell below, the
GRU with 8-channel heads of the DEER summary page's limitations paragraph).
The whole sequence s_t = cell(s_{t-1}, x_t) is then solved by Newton's
method (ParaRNN page, TL;DR and abstract: Newton iterations on the
whole-sequence system, diagonal and block-diagonal Jacobians; a framework for
parallelising new nonlinear RNNs; DEER summary page, method paragraph: the
same for any differentiable recurrence, tolerance the only extra
hyper-parameter).  This is the modality in which the system is assembled by
the framework's tensor operations and only the parallel reduction runs in a
dedicated kernel (ParaRNN page, Fig. 5 caption): each iteration evaluates the
cell and its Jacobian blocks with torch (forward-mode differentiation, one
tangent per state component), and solves the block bi-diagonal linear system
with the library's diagonal, 2x2 or k x k scan (rnn_linscan_diag,
rnn_linscan_blk2, rnn_linscan_blk).  Cells with a built-in kernel (GRU, LSTM)
are much faster through pararnn_gru_forward / pararnn_lstm_forward.

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
    if k == 2:
        return api.linscan_blk2(J.contiguous(), b.contiguous())
    return api.linscan_blk(J.contiguous(), b.contiguous())


STATE_SIZES = (1, 2, 4, 8)


def head_gru_cell(s, pz, pr, pc, Uz, Ur, Uc):
    """GRU with dense recurrence inside heads of k channels: the diagonal GRU
    cell with each weight vector replaced by one k x k matrix per head, acting
    on the state where the diagonal cell multiplies by u (a diagonal U gives
    the diagonal cell):
        z = sig(pz + Uz s), r = sig(pr + Ur s), c = tanh(pc + Uc (r*s)),
        s' = (1 - z)*s + z*c.
    s, p: [B, L, NH, k]; U: [NH, k, k] (U[n, i, l] takes component l into i).
    Its Jacobian blocks are dense k x k (DEER summary page, limitations
    paragraph); solve it with newton_solve(..., state_size=k)."""
    def mv(U, v):
        return torch.matmul(U, v.unsqueeze(-1)).squeeze(-1)
    z = torch.sigmoid(pz + mv(Uz, s))
    r = torch.sigmoid(pr + mv(Ur, s))
    c = torch.tanh(pc + mv(Uc, r * s))
    return (1 - z) * s + z * c


def _solve(cell, inputs, params, h0, tol, max_iter, info, k, init=None):
    B, L, H = inputs[0].shape[:3]
    shape = (B, L, H) if k == 1 else (B, L, H, k)
    if init is None:
        s = torch.zeros(shape, dtype=inputs[0].dtype, device=inputs[0].device)
    else:
        s = init.detach().clone()
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
    def forward(ctx, cell, tol, max_iter, info, k, n_inputs, init, h0, *tensors):
        inputs, params = tensors[:n_inputs], tensors[n_inputs:]
        s = _solve(cell, inputs, params, h0, tol, max_iter, info, k, init)
        ctx.cell, ctx.n_inputs, ctx.k = cell, n_inputs, k
        ctx.save_for_backward(h0, s, *tensors)
        return s

    @staticmethod
    def backward(ctx, g):
        h0, s, *tensors = ctx.saved_tensors
        gh0, gt = _adjoint(ctx.cell, ctx.k, ctx.n_inputs, h0, s, tensors, g, ctx.needs_input_grad[7])
        return (None, None, None, None, None, None, None, gh0, *gt)


def _adjoint(cell, k, n_inputs, h0, s, tensors, g, want_h0):
    """Gradients of <g, s> through the converged solve s: the adjoint
    lambda_t = g_t + J_{t+1}^T lambda_{t+1} (a scan in reversed time on the
    same kernels, transposed blocks), then one vector-Jacobian product of
    the cell for h0, the inputs and the parameters."""
    inputs, params = tensors[:n_inputs], tensors[n_inputs:]
    with torch.no_grad():
        _, J = _cell_and_jacobian(cell, _shift(s, h0), inputs, params, k)
        if k > 1:
            J = J.transpose(-1, -2)
        a = torch.cat([J[:, 1:], torch.zeros_like(J[:, :1])], dim=1)
        lam = _scan(a.flip(1), g.flip(1), k).flip(1)
    with torch.enable_grad():
        h0_ = h0.detach().requires_grad_(want_h0)
        ins = [x.detach().requires_grad_(True) for x in tensors]
        F = cell(_shift(s, h0_), *ins)
        wrt = [x for x in [h0_] + ins if x.requires_grad]
        grads = iter(torch.autograd.grad(F, wrt, grad_outputs=lam, allow_unused=True))
    gh0 = next(grads) if h0_.requires_grad else None
    gt = [next(grads) for _ in ins]
    gt = [torch.zeros_like(x) if gx is None else gx for x, gx in zip(tensors, gt)]
    return gh0, gt


class _HeadGruSolve(torch.autograd.Function):
    """Forward by the library's head-GRU Newton kernel (pararnn_hgru_forward),
    backward by its adjoint kernel (pararnn_hgru_backward)."""

    @staticmethod
    def forward(ctx, tol, max_iter, info, init, h0, pz, pr, pc, Uz, Ur, Uc):
        dev_info = torch.zeros(2, dtype=torch.int32, device=pz.device) if info is not None else None
        s = api.hgru_forward(pz.detach(), pr.detach(), pc.detach(), Uz.detach(), Ur.detach(), Uc.detach(),
                             h0.detach(), tol=tol, max_iter=max_iter, info=dev_info,
                             init=None if init is None else init.detach())
        if info is not None:
            info[0], info[1] = [int(v) for v in dev_info.tolist()]
        ctx.save_for_backward(h0, s, pz, pr, pc, Uz, Ur, Uc)
        ctx.k = pz.shape[-1]
        return s

    @staticmethod
    def backward(ctx, g):
        h0, s, pz, pr, pc, Uz, Ur, Uc = ctx.saved_tensors
        need = ctx.needs_input_grad
        dpz, dpr, dpc, dUz, dUr, dUc, dh0 = api.hgru_backward(
            pz.detach(), pr.detach(), pc.detach(), Uz.detach(), Ur.detach(), Uc.detach(), h0.detach(), s,
            g.contiguous(), want_u=any(need[8:11]), want_h0=need[4])
        return (None, None, None, None, dh0, dpz, dpr, dpc, dUz, dUr, dUc)


def head_gru_solve(pz: torch.Tensor, pr: torch.Tensor, pc: torch.Tensor, Uz: torch.Tensor,
                   Ur: torch.Tensor, Uc: torch.Tensor, h0: Optional[torch.Tensor] = None, *,
                   tol: float = 1e-4, max_iter: int = 32, info: Optional[list] = None,
                   init: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The GRU with dense recurrence inside heads of k channels (head_gru_cell,
    k = 4 or 8) solved by the library's Newton kernel (pararnn_hgru_forward:
    cell, k x k Jacobian rows and the block scan in one launch per
    iteration), differentiable with respect to p, U and h0 through the
    adjoint of the solve.  p [B, L, NH, k], U [NH, k, k], h0 [B, NH, k] or
    None; `init` a warm start; `info` receives [iterations, converged]."""
    B, L, NH, k = pz.shape
    if h0 is None:
        h0 = torch.zeros((B, NH, k), dtype=pz.dtype, device=pz.device)
    return _HeadGruSolve.apply(float(tol), int(max_iter), info, init, h0, pz, pr, pc, Uz, Ur, Uc)


def newton_solve(cell: Callable[..., torch.Tensor], inputs: Sequence[torch.Tensor],
                 h0: Optional[torch.Tensor] = None, params: Sequence[torch.Tensor] = (), *,
                 tol: float = 1e-4, max_iter: int = 32, info: Optional[list] = None,
                 state_size: int = 1, init: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Solve s_t = cell(s_{t-1}, *inputs_t, *params) over the whole sequence.

    inputs: tensors [B, L, H] or [B, L, H, state_size] (fp32, on a HIP
    device) passed to the cell position-wise; params: tensors the cell uses as
    they are (weights, broadcast against the state); state_size: 1 (states
    [B, L, H]) or k = 2, 4, 8 (states [B, L, H, k], k x k Jacobian blocks);
    h0: [B, H] or [B, H, k], or None (zeros).  Newton starts from s = 0, or
    from `init` (a warm start, shaped as the states; no gradient flows to
    it), and stops once max|delta| <= tol or after max_iter updates; `info`,
    if a list of two, receives [iterations, converged].  Returns the states,
    differentiable with respect to inputs, params and h0 through the adjoint
    of the solve."""
    if not inputs:
        raise ValueError("at least one input sequence is needed")
    if state_size not in STATE_SIZES:
        raise ValueError("state_size must be one of %s" % (STATE_SIZES,))
    x0 = inputs[0]
    if x0.device.type != "cuda":
        raise ValueError("newton_solve runs on a HIP device only; inputs are on %s" % x0.device)
    if x0.dim() not in (3, 4):
        raise ValueError("inputs must be [B, L, H] or [B, L, H, state_size]")
    if not tol >= 0.0 or max_iter < 1:
        raise ValueError("tol must be >= 0 and max_iter >= 1")
    B, L, H = x0.shape[:3]
    shapes = ((B, L, H), (B, L, H, state_size))
    for x in inputs:
        if tuple(x.shape) not in shapes:
            raise ValueError("every input must be [B, L, H] or [B, L, H, %d]" % state_size)
    hshape = (B, H) if state_size == 1 else (B, H, state_size)
    if h0 is None:
        h0 = torch.zeros(hshape, dtype=x0.dtype, device=x0.device)
    elif tuple(h0.shape) != hshape:
        raise ValueError("h0 must be %s" % (hshape,))
    sshape = (B, L, H) if state_size == 1 else (B, L, H, state_size)
    if init is not None and (tuple(init.shape) != sshape or init.device != x0.device):
        raise ValueError("init must be %s on %s" % (sshape, x0.device))
    return _BlockDiagonalSolve.apply(cell, float(tol), int(max_iter), info, state_size,
                                     len(inputs), init, h0, *inputs, *params)
