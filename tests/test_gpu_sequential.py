"""GPU parity of the sequential application (one thread per channel, one cell
per position) against the oracle's fp64 rollout, and agreement with the
Newton forwards, which converge to the same sequence."""
import pytest
import torch

from nonlinear_rnn_solve_pararnn_amd import api, synth
from tests.gpu_helpers import FWD_ATOL, dev, gru_args, lstm_args, max_abs, say

pytestmark = pytest.mark.gpu

# B*H not a multiple of 64, L not a multiple of the 16-position load blocks,
# L = 1, H = 1 (time-contiguous rows) and a wide shape
SHAPES = [(1, 1, 1), (1, 64, 4), (2, 33, 5), (3, 257, 70), (2, 5000, 1), (2, 100, 130),
          (1, 16, 64), (4, 17, 64)]


@pytest.mark.parametrize("B,L,H", SHAPES)
def test_gru_sequential_matches_rollout(orc, B, L, H):
    say("gru seq", B, L, H)
    d = synth.gru_inputs(B, L, H, seed=170 + H, h0=True)
    ins = [dev(x) for x in gru_args(d)]
    h = api.gru_sequential(*ins, dev(d["h0"]))
    err = max_abs(h.cpu().numpy(), orc.gru_rollout(*gru_args(d), h0=d["h0"]))
    say(err)
    assert err <= FWD_ATOL
    h0less = api.gru_sequential(*ins)
    assert max_abs(h0less.cpu().numpy(), orc.gru_rollout(*gru_args(d))) <= FWD_ATOL


@pytest.mark.parametrize("B,L,H", SHAPES)
def test_lstm_sequential_matches_rollout(orc, B, L, H):
    say("lstm seq", B, L, H)
    d = synth.lstm_inputs(B, L, H, seed=180 + H, h0=True)
    ins = [dev(x) for x in lstm_args(d)]
    h, c = api.lstm_sequential(*ins, dev(d["h0"]), dev(d["c0"]))
    hr, cr = orc.lstm_rollout(*lstm_args(d), h0=d["h0"], c0=d["c0"])
    errs = (max_abs(h.cpu().numpy(), hr), max_abs(c.cpu().numpy(), cr))
    say(errs)
    assert max(errs) <= FWD_ATOL


def test_sequential_equals_converged_newton():
    """Newton from zero converges to the sequence the rollout computes."""
    d = synth.gru_inputs(4, 3000, 96, seed=190)
    ins = [dev(x) for x in gru_args(d)]
    hs = api.gru_sequential(*ins)
    hn = api.gru_forward(*ins, tol=1e-6, max_iter=64)
    assert float((hs - hn).abs().max()) <= FWD_ATOL
    d = synth.lstm_inputs(2, 1500, 64, seed=191)
    ins = [dev(x) for x in lstm_args(d)]
    hs, cs = api.lstm_sequential(*ins)
    hn, cn = api.lstm_forward(*ins, tol=1e-6, max_iter=64)
    assert max(float((hs - hn).abs().max()), float((cs - cn).abs().max())) <= FWD_ATOL


def test_sequential_rejects_bad_arguments():
    d = synth.gru_inputs(1, 8, 4, seed=192)
    ins = [dev(x) for x in gru_args(d)]
    with pytest.raises(ValueError):
        api.gru_sequential(*ins, torch.zeros(2, 4, device="cuda"))  # h0 of the wrong shape
