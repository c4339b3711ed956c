"""GPU parity of the Newton solve for user-defined diagonal cells (the
framework's tensor operations assemble the system, the library's diagonal
scan solves it): the GRU cell written with torch against the oracle (forward
and gradients) and against the built-in GRU kernel, and a cell with no
built-in kernel against torch autograd through a sequential fp64 loop."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_pararnn_amd import api, generic, synth
from tests.gpu_helpers import FWD_ATOL, GRAD_RTOL, dev, gru_args, host, max_abs, rel_inf, say

pytestmark = pytest.mark.gpu


def gru_cell(h, pz, pr, pc, uz, ur, uc):
    z = torch.sigmoid(pz + uz * h)
    r = torch.sigmoid(pr + ur * h)
    c = torch.tanh(pc + uc * (r * h))
    return (1 - z) * h + z * c


def leaky_cell(h, p, q, u):
    """h' = (1 - a) h + a tanh(p + u h), a = sigmoid(q): no built-in kernel."""
    a = torch.sigmoid(q)
    return (1 - a) * h + a * torch.tanh(p + u * h)


@pytest.mark.parametrize("B,L,H", [(2, 64, 4), (2, 700, 40), (1, 5000, 3), (3, 257, 70)])
def test_generic_gru_matches_oracle(orc, B, L, H):
    say("generic gru", B, L, H)
    d = synth.gru_inputs(B, L, H, seed=500 + H, h0=True, grad=True)
    p = [dev(d[k]).requires_grad_(True) for k in ("pz", "pr", "pc")]
    u = [dev(d[k]).requires_grad_(True) for k in ("uz", "ur", "uc")]
    h0 = dev(d["h0"]).requires_grad_(True)
    info = [0, 0]
    h = generic.newton_solve(gru_cell, p, h0, u, tol=1e-6, max_iter=64, info=info)
    href = orc.gru_rollout(*gru_args(d), h0=d["h0"])
    err = max_abs(host(h), href)
    (h * dev(d["g"])).sum().backward()
    dp, du, dh0 = orc.gru_bptt(*gru_args(d), href, d["g"], h0=d["h0"])
    errs = {"dp%d" % q: rel_inf(host(p[q].grad), dp[q]) for q in range(3)}
    errs.update({"du%d" % q: rel_inf(host(u[q].grad), du[q]) for q in range(3)})
    errs["dh0"] = rel_inf(host(h0.grad), dh0)
    say(info, err, errs)
    assert info[1] == 1 and err <= FWD_ATOL
    assert max(errs.values()) <= GRAD_RTOL, errs
    # the built-in kernel on the same inputs
    hk = api.gru_forward(*[x.detach() for x in p + u], h0.detach(), tol=1e-6, max_iter=64)
    assert float((hk - h.detach()).abs().max()) <= FWD_ATOL


def _leaky_reference(d):
    t = {k: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True) for k, v in d.items()}
    h = t["h0"]
    hs = []
    for s in range(t["p"].shape[1]):
        h = leaky_cell(h, t["p"][:, s], t["q"][:, s], t["u"])
        hs.append(h)
    hs = torch.stack(hs, 1)
    (hs * t["g"]).sum().backward()
    return hs.detach().numpy(), {k: t[k].grad.numpy() for k in ("p", "q", "u", "h0")}


@pytest.mark.parametrize("B,L,H", [(2, 300, 5), (2, 600, 64)])
def test_generic_custom_cell_matches_autograd_loop(B, L, H):
    say("generic leaky", B, L, H)
    rng = np.random.default_rng(510 + H)
    d = {"p": rng.standard_normal((B, L, H)).astype(np.float32),
         "q": rng.standard_normal((B, L, H)).astype(np.float32),
         "u": rng.uniform(-0.8, 0.8, H).astype(np.float32),
         "h0": rng.uniform(-0.9, 0.9, (B, H)).astype(np.float32),
         "g": rng.standard_normal((B, L, H)).astype(np.float32)}
    href, gref = _leaky_reference(d)
    t = {k: dev(v).requires_grad_(k != "g") for k, v in d.items()}
    info = [0, 0]
    h = generic.newton_solve(leaky_cell, [t["p"], t["q"]], t["h0"], [t["u"]], tol=1e-6,
                             max_iter=64, info=info)
    (h * t["g"]).sum().backward()
    err = max_abs(host(h), href)
    errs = {k: rel_inf(host(t[k].grad), gref[k]) for k in ("p", "q", "u", "h0")}
    say(info, err, errs)
    assert info[1] == 1 and err <= FWD_ATOL
    assert max(errs.values()) <= GRAD_RTOL, errs
