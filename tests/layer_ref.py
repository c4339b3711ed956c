"""Reference for the trainable layers: the input projections and a sequential
rollout of the diagonal cells written with plain torch ops in fp64 on the CPU,
differentiated by torch autograd.  It shares nothing with the library (or
with the oracle), and is small enough for L of a few hundred.

Cells (ParaRNN page, Fig. 2 caption: diagonal recurrences):
  GRU   z = s(pz + uz h), r = s(pr + ur h), c = tanh(pc + uc (r h)),
        h' = (1 - z) h + z c
  LSTM  i, f, o = s(p + u h), g = tanh(pg + ug h), c' = f c + i g, h' = o tanh(c')
"""
import numpy as np
import torch

from nonlinear_rnn_solve_pararnn_amd import layers

NG = {"gru": 3, "lstm": 4}


def _seq(kind, p, u, h0, c0):
    B, L, H = p[0].shape
    h = h0
    c = c0
    hs, cs = [], []
    for t in range(L):
        if kind == "gru":
            z = torch.sigmoid(p[0][:, t] + u[0] * h)
            r = torch.sigmoid(p[1][:, t] + u[1] * h)
            cc = torch.tanh(p[2][:, t] + u[2] * (r * h))
            h = (1 - z) * h + z * cc
        else:
            i = torch.sigmoid(p[0][:, t] + u[0] * h)
            f = torch.sigmoid(p[1][:, t] + u[1] * h)
            o = torch.sigmoid(p[2][:, t] + u[2] * h)
            g = torch.tanh(p[3][:, t] + u[3] * h)
            c = f * c + i * g
            h = o * torch.tanh(c)
            cs.append(c)
        hs.append(h)
    return torch.stack(hs, 1), (torch.stack(cs, 1) if cs else None)


def reference(kind, d, with_h0=True, loss_on=("h", "c"), bias=True):
    """Outputs and gradients of loss = sum(gh*h) (+ sum(gc*c)) in fp64."""
    t = {k: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True) for k, v in d.items()}
    B, L, D = d["x"].shape
    H = d["u"].shape[1]
    p = [t["x"] @ t["weight"][g].T + (t["bias"][g] if bias else 0.0) for g in range(NG[kind])]
    h0 = t["h0"] if with_h0 else torch.zeros(B, H, dtype=torch.float64)
    c0 = t["c0"] if with_h0 else torch.zeros(B, H, dtype=torch.float64)
    h, c = _seq(kind, p, [t["u"][g] for g in range(NG[kind])], h0, c0)
    loss = 0.0
    if "h" in loss_on:
        loss = loss + (t["gh"] * h).sum()
    if kind == "lstm" and "c" in loss_on:
        loss = loss + (t["gc"] * c).sum()
    loss.backward()
    out = {"h": h.detach().numpy()}
    if c is not None:
        out["c"] = c.detach().numpy()
    for k in ("x", "weight", "bias", "u") if bias else ("x", "weight", "u"):
        out["d" + k] = t[k].grad.numpy()
    if with_h0:
        out["dh0"] = t["h0"].grad.numpy()
        if kind == "lstm":
            out["dc0"] = t["c0"].grad.numpy()
    return out


def run_layer(kind, d, device, with_h0=True, loss_on=("h", "c"), tol=1e-5, max_iter=32, bias=True):
    """The same through layers.ParaGRU / ParaLSTM on `device` (fp32)."""
    B, L, D = d["x"].shape
    H = d["u"].shape[1]
    cls = layers.ParaGRU if kind == "gru" else layers.ParaLSTM
    m = cls(D, H, bias=bias, tol=tol, max_iter=max_iter, device=device)
    keys = ("weight", "bias", "u") if bias else ("weight", "u")
    with torch.no_grad():
        for k in keys:
            getattr(m, k).copy_(torch.from_numpy(d[k]))
    x = torch.from_numpy(d["x"]).to(device).requires_grad_(True)
    h0 = torch.from_numpy(d["h0"]).to(device).requires_grad_(True) if with_h0 else None
    c0 = torch.from_numpy(d["c0"]).to(device).requires_grad_(True) if with_h0 else None
    gh = torch.from_numpy(d["gh"]).to(device)
    gc = torch.from_numpy(d["gc"]).to(device)
    if kind == "gru":
        h = m(x, h0)
        c = None
    else:
        h, c = m(x, h0, c0)
    loss = 0.0
    if "h" in loss_on:
        loss = loss + (gh * h).sum()
    if kind == "lstm" and "c" in loss_on:
        loss = loss + (gc * c).sum()
    loss.backward()
    out = {"h": h.detach().cpu().numpy(), "info": m.last_info.cpu().tolist()}
    if c is not None:
        out["c"] = c.detach().cpu().numpy()
    out["dx"] = x.grad.cpu().numpy()
    for k in keys:
        out["d" + k] = getattr(m, k).grad.cpu().numpy()
    if with_h0:
        out["dh0"] = h0.grad.cpu().numpy()
        if kind == "lstm":
            out["dc0"] = c0.grad.cpu().numpy()
    return out
