"""Library stand-ins used to pin the oracle (CPU, fp64).

The diagonal-recurrence GRU and LSTM cells are special cases of the classical
cells that torch.nn implements with dense recurrent weights.  Choosing the
input weights as (signed) identities and the recurrent weights as diagonal
matrices makes torch.nn.GRU / torch.nn.LSTM compute exactly the cells the
oracle implements, so the oracle can be checked against an implementation it
shares nothing with (including autograd for the Jacobians and gradients).

GRU mapping.  torch: r = s(x_r + W_hr h), z_t = s(x_z + W_hz h),
n = tanh(x_n + r*(W_hn h)), h' = (1 - z_t) n + z_t h.  Ours: z = s(pz + uz h),
h' = (1 - z) h + z c.  So z_t = 1 - z = s(-pz - uz h): feed x_z = -pz and use
W_hz = diag(-uz); x_r = pr, W_hr = diag(ur); x_n = pc, W_hn = diag(uc).

LSTM mapping.  torch gate order (i, f, g, o), identical equations: feed
x = (pi, pf, pg, po) and W_h* = diag(u*).
"""
from __future__ import annotations

import numpy as np
import torch


def _t(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def make_gru(H, uz, ur, uc):
    m = torch.nn.GRU(input_size=3 * H, hidden_size=H, batch_first=True,
                     bias=False, dtype=torch.float64)
    with torch.no_grad():
        m.weight_ih_l0.copy_(torch.eye(3 * H, dtype=torch.float64))
        whh = torch.zeros(3 * H, H, dtype=torch.float64)
        whh[0:H] = torch.diag(_t(ur))
        whh[H:2 * H] = torch.diag(-_t(uz))
        whh[2 * H:3 * H] = torch.diag(_t(uc))
        m.weight_hh_l0.copy_(whh)
    return m


def gru_x(pz, pr, pc):
    """Input sequence for make_gru: concat(pr, -pz, pc) on the feature axis."""
    return torch.cat([_t(pr), -_t(pz), _t(pc)], dim=-1)


def gru_rollout(pz, pr, pc, uz, ur, uc, h0=None):
    B, L, H = np.shape(pz)
    m = make_gru(H, uz, ur, uc)
    hx = None if h0 is None else _t(h0)[None]
    with torch.no_grad():
        y, _ = m(gru_x(pz, pr, pc), hx)
    return y.numpy()


def make_lstm_cell(H, ui, uf, uo, ug):
    m = torch.nn.LSTMCell(input_size=4 * H, hidden_size=H, bias=False,
                          dtype=torch.float64)
    with torch.no_grad():
        m.weight_ih.copy_(torch.eye(4 * H, dtype=torch.float64))
        whh = torch.zeros(4 * H, H, dtype=torch.float64)
        whh[0:H] = torch.diag(_t(ui))
        whh[H:2 * H] = torch.diag(_t(uf))
        whh[2 * H:3 * H] = torch.diag(_t(ug))
        whh[3 * H:4 * H] = torch.diag(_t(uo))
        m.weight_hh.copy_(whh)
    return m


def make_lstm(H, ui, uf, uo, ug):
    m = torch.nn.LSTM(input_size=4 * H, hidden_size=H, batch_first=True,
                      bias=False, dtype=torch.float64)
    cell = make_lstm_cell(H, ui, uf, uo, ug)
    with torch.no_grad():
        m.weight_ih_l0.copy_(cell.weight_ih)
        m.weight_hh_l0.copy_(cell.weight_hh)
    return m


def lstm_x(pi, pf, po, pg):
    return torch.cat([_t(pi), _t(pf), _t(pg), _t(po)], dim=-1)


def lstm_rollout(pi, pf, po, pg, ui, uf, uo, ug, h0=None, c0=None):
    """Per-step (h, c) via torch.nn.LSTMCell applied in a loop."""
    B, L, H = np.shape(pi)
    cell = make_lstm_cell(H, ui, uf, uo, ug)
    x = lstm_x(pi, pf, po, pg)
    h = torch.zeros(B, H, dtype=torch.float64) if h0 is None else _t(h0)
    c = torch.zeros(B, H, dtype=torch.float64) if c0 is None else _t(c0)
    hs, cs = [], []
    with torch.no_grad():
        for t in range(L):
            h, c = cell(x[:, t], (h, c))
            hs.append(h)
            cs.append(c)
    return torch.stack(hs, 1).numpy(), torch.stack(cs, 1).numpy()


def _blockdiag(U):
    """[NH, k, k] -> the [NH*k, NH*k] block-diagonal matrix."""
    return torch.block_diag(*[_t(u) for u in np.asarray(U)])


def make_hgru(NH, k, Uz, Ur, Uc):
    """torch.nn.GRU computing the GRU with dense recurrence inside heads of k
    channels, for a diagonal Uc: torch applies r after its recurrent matrix,
    r*(W_hn h), which equals Uc (r*h) only when Uc is diagonal.  Uz and Ur
    may be dense: W_hz = blockdiag(-Uz), W_hr = blockdiag(Ur)."""
    H = NH * k
    m = torch.nn.GRU(input_size=3 * H, hidden_size=H, batch_first=True,
                     bias=False, dtype=torch.float64)
    with torch.no_grad():
        m.weight_ih_l0.copy_(torch.eye(3 * H, dtype=torch.float64))
        whh = torch.zeros(3 * H, H, dtype=torch.float64)
        whh[0:H] = _blockdiag(Ur)
        whh[H:2 * H] = -_blockdiag(Uz)
        whh[2 * H:3 * H] = _blockdiag(Uc)
        m.weight_hh_l0.copy_(whh)
    return m
