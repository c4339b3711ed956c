"""GPU parity of warm-started Newton: the forwards take an initial iterate
instead of zero (GRU on every path, LSTM on every path, the generic solver
with k x k blocks).  Two properties pin it against the oracle's Newton from
the same iterate: the iterates themselves (tol 0, cap n), and a start at a
converged solution returning after one iteration with the rollout."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_pararnn_amd import api, generic, synth
from tests.gpu_helpers import FWD_ATOL, dev, gru_args, host, lstm_args, max_abs, say

pytestmark = pytest.mark.gpu

# path, (B, L, H): channel lanes over several chunks, time lanes over many
GRU_CASES = [("fused", (2, 300, 40)), ("fused", (1, 512, 20)), ("chain", (2, 300, 40)),
             ("local", (2, 300, 40)), ("step", (2, 300, 40)), ("chain", (2, 5000, 1)),
             ("step", (2, 5000, 1)), ("chain", (3, 700, 70))]
LSTM_CASES = [("chain", (2, 300, 40)), ("local", (2, 300, 40)), ("step", (2, 300, 40)),
              ("chain", (2, 3000, 3)), ("step", (2, 3000, 3))]


def _info():
    return torch.zeros(2, dtype=torch.int32, device="cuda:0")


@pytest.mark.parametrize("path,shape", GRU_CASES)
def test_gru_warm_iterates_equal_oracle(orc, monkeypatch, path, shape):
    """From the oracle's second iterate (in fp32), n more GPU iterations equal
    the oracle's n iterations from that same start."""
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    B, L, H = shape
    say("gru warm iterates", path, shape)
    d = synth.gru_inputs(B, L, H, seed=600 + L + H, h0=True)
    a = gru_args(d)
    s2, _, _, _ = orc.gru_newton(*a, h0=d["h0"], tol=0.0, cap=2)
    init = s2.astype(np.float32)
    ins = [dev(x) for x in a]
    for n in (1, 2):
        info = _info()
        h = api.gru_forward(*ins, dev(d["h0"]), tol=0.0, max_iter=n, info=info, init=dev(init))
        ref, it, _, _ = orc.gru_newton(*a, h0=d["h0"], tol=0.0, cap=n, init=init)
        err = max_abs(host(h), ref)
        say(n, host(info), err)
        assert host(info)[0] == n == it and err <= FWD_ATOL


@pytest.mark.parametrize("path,shape", GRU_CASES)
def test_gru_converged_warm_start_takes_one_iteration(orc, monkeypatch, path, shape):
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    B, L, H = shape
    d = synth.gru_inputs(B, L, H, seed=610 + L + H, h0=True)
    ins = [dev(x) for x in gru_args(d)]
    h_star = api.gru_forward(*ins, dev(d["h0"]), tol=1e-6, max_iter=64)
    info = _info()
    h = api.gru_forward(*ins, dev(d["h0"]), tol=1e-5, max_iter=32, info=info, init=h_star)
    err = max_abs(host(h), orc.gru_rollout(*gru_args(d), h0=d["h0"]))
    say(path, shape, host(info), err)
    assert host(info).tolist() == [1, 1] and err <= FWD_ATOL


@pytest.mark.parametrize("path,shape", LSTM_CASES)
def test_lstm_warm_iterates_equal_oracle(orc, monkeypatch, path, shape):
    """Both initial iterates, and h alone (c from zero)."""
    monkeypatch.setenv("PARARNN_LSTM_PATH", path)
    B, L, H = shape
    say("lstm warm iterates", path, shape)
    d = synth.lstm_inputs(B, L, H, seed=620 + L + H, h0=True)
    a = lstm_args(d)
    h2, c2, _, _, _ = orc.lstm_newton(*a, h0=d["h0"], c0=d["c0"], tol=0.0, cap=2)
    hi, ci = h2.astype(np.float32), c2.astype(np.float32)
    ins = [dev(x) for x in a]
    for n, with_c in ((1, True), (2, True), (2, False)):
        info = _info()
        h, c = api.lstm_forward(*ins, dev(d["h0"]), dev(d["c0"]), tol=0.0, max_iter=n, info=info,
                                init_h=dev(hi), init_c=dev(ci) if with_c else None)
        rh, rc, it, _, _ = orc.lstm_newton(*a, h0=d["h0"], c0=d["c0"], tol=0.0, cap=n, h_init=hi,
                                           c_init=ci if with_c else None)
        err = max(max_abs(host(h), rh), max_abs(host(c), rc))
        say(n, with_c, host(info), err)
        assert host(info)[0] == n == it and err <= FWD_ATOL


@pytest.mark.parametrize("path,shape", LSTM_CASES)
def test_lstm_converged_warm_start_takes_one_iteration(orc, monkeypatch, path, shape):
    monkeypatch.setenv("PARARNN_LSTM_PATH", path)
    B, L, H = shape
    d = synth.lstm_inputs(B, L, H, seed=630 + L + H, h0=True)
    ins = [dev(x) for x in lstm_args(d)]
    h_star, c_star = api.lstm_forward(*ins, dev(d["h0"]), dev(d["c0"]), tol=1e-6, max_iter=64)
    info = _info()
    h, c = api.lstm_forward(*ins, dev(d["h0"]), dev(d["c0"]), tol=1e-5, max_iter=32, info=info,
                            init_h=h_star, init_c=c_star)
    rh, rc = orc.lstm_rollout(*lstm_args(d), h0=d["h0"], c0=d["c0"])
    err = max(max_abs(host(h), rh), max_abs(host(c), rc))
    say(path, shape, host(info), err)
    assert host(info).tolist() == [1, 1] and err <= FWD_ATOL


def test_warm_start_rejects_an_initial_iterate_sharing_the_output():
    d = synth.gru_inputs(1, 64, 8, seed=640)
    ins = [dev(x) for x in gru_args(d)]
    out = torch.empty(1, 64, 8, device="cuda:0")
    with pytest.raises(api.PararnnError):
        api.gru_forward(*ins, None, out=out, init=out)


def test_generic_head_gru_warm_start(orc):
    """The generic solver from an initial iterate (k x k blocks): iterates
    equal the oracle's Newton from the same start, and a converged start
    returns after one iteration."""
    d = synth.head_gru_inputs(2, 300, 3, 8, seed=650, h0=True)
    a = [d[x] for x in ("pz", "pr", "pc", "Uz", "Ur", "Uc")]
    t = [dev(x) for x in a]
    s2, _, _, _ = orc.hgru_newton(*a, h0=d["h0"], tol=0.0, cap=2)
    init = s2.astype(np.float32)
    for n in (1, 2):
        info = [0, 0]
        s = generic.newton_solve(generic.head_gru_cell, t[:3], dev(d["h0"]), t[3:], tol=0.0,
                                 max_iter=n, info=info, state_size=8, init=dev(init))
        ref, it, _, _ = orc.hgru_newton(*a, h0=d["h0"], tol=0.0, cap=n, init=init)
        assert info[0] == n == it and max_abs(host(s), ref) <= FWD_ATOL
    ref = orc.hgru_rollout(*a, h0=d["h0"])
    info = [0, 0]
    s = generic.newton_solve(generic.head_gru_cell, t[:3], dev(d["h0"]), t[3:], tol=1e-5,
                             max_iter=32, info=info, state_size=8, init=dev(ref.astype(np.float32)))
    assert info == [1, 1] and max_abs(host(s), ref) <= FWD_ATOL
