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


def lstm_cell(s, pi, pf, po, pg, ui, uf, uo, ug):
    """The LSTM-style cell on states (c, h) = s[..., 0], s[..., 1]."""
    cp, hp = s[..., 0], s[..., 1]
    i = torch.sigmoid(pi + ui * hp)
    f = torch.sigmoid(pf + uf * hp)
    o = torch.sigmoid(po + uo * hp)
    g = torch.tanh(pg + ug * hp)
    c = f * cp + i * g
    return torch.stack([c, o * torch.tanh(c)], dim=-1)


def pair_cell(s, p, q, u):
    """Two coupled states per channel with no built-in kernel:
    x' = tanh(p + u y) + 0.3 x,  y' = sigmoid(q) x' + 0.5 y (2x2 Jacobians)."""
    x, y = s[..., 0], s[..., 1]
    xn = torch.tanh(p + u * y) + 0.3 * x
    return torch.stack([xn, torch.sigmoid(q) * xn + 0.5 * y], dim=-1)


@pytest.mark.parametrize("B,L,H", [(2, 64, 4), (2, 700, 40), (1, 5000, 3)])
def test_generic_lstm_pairs_match_oracle(orc, B, L, H):
    """state_size=2: the LSTM cell written with torch, its 2x2 blocks solved by
    the 2x2 scan; forward and every gradient against the oracle."""
    from tests.gpu_helpers import lstm_args
    say("generic lstm", B, L, H)
    d = synth.lstm_inputs(B, L, H, seed=520 + H, h0=True, grad=True)
    p = [dev(d[k]).requires_grad_(True) for k in ("pi", "pf", "po", "pg")]
    u = [dev(d[k]).requires_grad_(True) for k in ("ui", "uf", "uo", "ug")]
    s0 = dev(np.stack([d["c0"], d["h0"]], axis=-1)).requires_grad_(True)
    info = [0, 0]
    s = generic.newton_solve(lstm_cell, p, s0, u, tol=1e-6, max_iter=64, info=info, state_size=2)
    href, cref = orc.lstm_rollout(*lstm_args(d), h0=d["h0"], c0=d["c0"])
    err = max(max_abs(host(s[..., 1]), href), max_abs(host(s[..., 0]), cref))
    g = dev(np.stack([d["gc"], d["gh"]], axis=-1))
    (s * g).sum().backward()
    dp, du, dh0, dc0 = orc.lstm_bptt(*lstm_args(d), href, cref, d["gh"], d["gc"], h0=d["h0"], c0=d["c0"])
    errs = {"dp%d" % q: rel_inf(host(p[q].grad), dp[q]) for q in range(4)}
    errs.update({"du%d" % q: rel_inf(host(u[q].grad), du[q]) for q in range(4)})
    errs["dc0"] = rel_inf(host(s0.grad[..., 0]), dc0)
    errs["dh0"] = rel_inf(host(s0.grad[..., 1]), dh0)
    say(info, err, errs)
    assert info[1] == 1 and err <= FWD_ATOL
    assert max(errs.values()) <= GRAD_RTOL, errs


@pytest.mark.parametrize("B,L,H", [(2, 300, 5), (2, 600, 64)])
def test_generic_pair_cell_matches_autograd_loop(B, L, H):
    say("generic pair", B, L, H)
    rng = np.random.default_rng(530 + H)
    d = {"p": rng.standard_normal((B, L, H)).astype(np.float32),
         "q": rng.standard_normal((B, L, H)).astype(np.float32),
         "u": rng.uniform(-0.8, 0.8, H).astype(np.float32),
         "h0": rng.uniform(-0.9, 0.9, (B, H, 2)).astype(np.float32),
         "g": rng.standard_normal((B, L, H, 2)).astype(np.float32)}
    t64 = {k: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True) for k, v in d.items()}
    st = t64["h0"]
    outs = []
    for i in range(L):
        st = pair_cell(st, t64["p"][:, i], t64["q"][:, i], t64["u"])
        outs.append(st)
    sref = torch.stack(outs, 1)
    (sref * t64["g"]).sum().backward()
    t = {k: dev(v).requires_grad_(k != "g") for k, v in d.items()}
    info = [0, 0]
    s = generic.newton_solve(pair_cell, [t["p"], t["q"]], t["h0"], [t["u"]], tol=1e-6,
                             max_iter=64, info=info, state_size=2)
    (s * t["g"]).sum().backward()
    err = max_abs(host(s), sref.detach().numpy())
    errs = {k: rel_inf(host(t[k].grad), t64[k].grad.numpy()) for k in ("p", "q", "u", "h0")}
    say(info, err, errs)
    assert info[1] == 1 and err <= FWD_ATOL
    assert max(errs.values()) <= GRAD_RTOL, errs


def test_generic_stops_on_the_device_one_iteration_late(orc):
    """The count reported equals the oracle's Newton count: the extra
    iteration the host enqueues before it sees the flag changes nothing."""
    d = synth.gru_inputs(2, 700, 40, seed=540, h0=True)
    t = [dev(x) for x in gru_args(d)]
    for tol, cap in ((1e-4, 32), (1e-6, 64), (0.0, 5)):
        info = [0, 0]
        h = generic.newton_solve(gru_cell, t[:3], dev(d["h0"]), t[3:], tol=tol, max_iter=cap, info=info)
        s, it, conv, _ = orc.gru_newton(*gru_args(d), h0=d["h0"], tol=tol, cap=cap)
        say(tol, cap, info, (it, conv))
        assert abs(info[0] - it) <= (1 if tol > 0 else 0) and info[1] == conv
        assert max_abs(host(h), s) <= (FWD_ATOL if tol > 0 else 1e-5)


# ---------------------------------------------------------------- k x k blocks
def _hgru(d):
    return [d[x] for x in ("pz", "pr", "pc", "Uz", "Ur", "Uc")]


@pytest.mark.parametrize("B,L,NH,k", [(2, 300, 3, 8), (2, 700, 5, 4), (1, 64, 1, 8), (2, 2000, 16, 8),
                                      (1, 3000, 2, 8)])
def test_generic_head_gru_matches_oracle(orc, B, L, NH, k):
    """The GRU with dense recurrence inside heads of k channels: k x k Jacobian
    blocks from torch, solved by the k x k scan; forward and every gradient
    (p, U, h0) against the oracle's rollout and backpropagation."""
    say("generic head gru", B, L, NH, k)
    d = synth.head_gru_inputs(B, L, NH, k, seed=550 + NH * k, h0=True, grad=True)
    p = [dev(d[x]).requires_grad_(True) for x in ("pz", "pr", "pc")]
    U = [dev(d[x]).requires_grad_(True) for x in ("Uz", "Ur", "Uc")]
    h0 = dev(d["h0"]).requires_grad_(True)
    info = [0, 0]
    h = generic.newton_solve(generic.head_gru_cell, p, h0, U, tol=1e-6, max_iter=64, info=info,
                             state_size=k)
    href = orc.hgru_rollout(*_hgru(d), h0=d["h0"])
    err = max_abs(host(h), href)
    (h * dev(d["g"])).sum().backward()
    ref = orc.hgru_bptt(*_hgru(d), href, d["g"], h0=d["h0"])
    got = [x.grad for x in p + U] + [h0.grad]
    names = ["dpz", "dpr", "dpc", "dUz", "dUr", "dUc", "dh0"]
    errs = {n: rel_inf(host(g), r) for n, g, r in zip(names, got, ref)}
    say(info, err, errs)
    assert info[1] == 1 and err <= FWD_ATOL
    assert max(errs.values()) <= GRAD_RTOL, errs


def test_generic_head_gru_iterates_equal_oracle_newton(orc):
    """tol = 0 and a cap of n: the n-th Newton iterate (k x k blocks) equals
    the oracle's."""
    d = synth.head_gru_inputs(2, 300, 3, 8, seed=560, h0=True)
    t = [dev(x) for x in _hgru(d)]
    for n in (1, 2, 3):
        info = [0, 0]
        s = generic.newton_solve(generic.head_gru_cell, t[:3], dev(d["h0"]), t[3:], tol=0.0,
                                 max_iter=n, info=info, state_size=8)
        ref, it, _, _ = orc.hgru_newton(*_hgru(d), h0=d["h0"], tol=0.0, cap=n)
        err = max_abs(host(s), ref)
        say(n, info, it, err)
        assert info[0] == n == it and err <= 1e-5
