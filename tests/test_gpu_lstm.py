"""GPU parity of the LSTM Newton forward (2x2 block Jacobians) against the
fp64 oracle, on the chained path (each chunk on chip for all iterations) and
on the per-iteration path."""
import pytest
import torch

from nonlinear_rnn_solve_pararnn_amd import api, synth
from tests.gpu_helpers import FWD_ATOL, ITER_ATOL, dev, host, lstm_args, max_abs, say

pytestmark = pytest.mark.gpu


# "chain" and "local" force the two forms of the chained kernel (chunks chained
# across workgroups; workgroups owning whole chains, channel lanes only).
@pytest.fixture(params=["chain", "local", "step"], autouse=True)
def lstm_path(request, monkeypatch):
    monkeypatch.setenv("PARARNN_LSTM_PATH", request.param)
    return request.param


def _run(d, tol, cap, with_init=True):
    ins = [dev(x) for x in lstm_args(d)]
    info = torch.zeros(2, dtype=torch.int32, device="cuda:0")
    h0 = dev(d["h0"]) if with_init else None
    c0 = dev(d["c0"]) if with_init else None
    h, c = api.lstm_forward(*ins, h0, c0, tol=tol, max_iter=cap, info=info)
    return host(h), host(c), host(info)


def test_iterates_match_oracle_newton(orc):
    d = synth.lstm_inputs(1, 64, 4, seed=70, h0=True)
    for k in range(1, 7):
        h, c, info = _run(d, 0.0, k)
        hr, cr, it, conv, _ = orc.lstm_newton(*lstm_args(d), h0=d["h0"], c0=d["c0"], tol=0.0, cap=k)
        assert list(info) == [k, 0]
        assert max_abs(h, hr) <= ITER_ATOL and max_abs(c, cr) <= ITER_ATOL, k


# H = 31 is the widest time-lane layout, H = 32 the narrowest channel-lane one.
@pytest.mark.parametrize("B,L,H", [(1, 1, 1), (2, 100, 3), (3, 257, 70), (2, 3000, 1), (2, 700, 33),
                                   (2, 9000, 1), (2, 300, 31), (2, 300, 32)])
def test_shapes_match_rollout(orc, B, L, H):
    say("lstm", B, L, H)
    d = synth.lstm_inputs(B, L, H, seed=71 + H, h0=True)
    h, c, info = _run(d, 1e-5, 32)
    hr, cr = orc.lstm_rollout(*lstm_args(d), h0=d["h0"], c0=d["c0"])
    assert info[1] == 1
    assert max_abs(h, hr) <= FWD_ATOL and max_abs(c, cr) <= FWD_ATOL


def test_non_convergence_and_nan_reported():
    d = synth.lstm_inputs(2, 200, 40, seed=75, h0=True)
    _, _, info = _run(d, 0.0, 1)
    assert list(info) == [1, 0]
    d["pi"][1, 50, 3] = float("nan")
    _, _, info = _run(d, 1e-4, 6)
    assert list(info) == [6, 0]


# Positions past the end of the sequence (ragged last chunks) and channels past
# H (ragged channel blocks) must not change when Newton stops: the count is
# that of Newton over the whole sequence (R4), within one of the oracle's
# where the last update is within rounding of tol (R5).
@pytest.mark.parametrize("B,L,H", [(2, 700, 33), (3, 257, 70), (2, 3001, 1)])
def test_ragged_stop_matches_oracle_count(orc, B, L, H):
    d = synth.lstm_inputs(B, L, H, seed=76 + H, h0=True)
    h, c, info = _run(d, 1e-4, 32)
    hr, cr, it, conv, _ = orc.lstm_newton(*lstm_args(d), h0=d["h0"], c0=d["c0"], tol=1e-4, cap=32)
    say("lstm ragged", B, L, H, "gpu", list(info), "oracle", it, conv)
    assert info[1] == 1 and conv == 1
    assert abs(int(info[0]) - int(it)) <= 1
    assert max_abs(h, hr) <= FWD_ATOL and max_abs(c, cr) <= FWD_ATOL


def test_u0_converges_in_three_updates(orc):
    d = synth.lstm_inputs(2, 500, 40, seed=72, zero_u=True)
    h, c, info = _run(d, 1e-6, 10, with_init=False)
    hr, cr = orc.lstm_rollout(*lstm_args(d))
    assert info[1] == 1 and info[0] <= 3
    assert max_abs(h, hr) <= FWD_ATOL and max_abs(c, cr) <= FWD_ATOL


def test_workload_full(orc):
    """B=8, L=2048, H=2048, p~N(0,1), u~U(-0.5,0.5), tol 1e-4, cap 32."""
    say("lstm full workload")
    d = synth.workload_inputs("c3_lstm")
    h, c, info = _run(d, 1e-4, 32, with_init=False)
    hr, cr = orc.lstm_rollout(*lstm_args(d))
    eh, ec = max_abs(h, hr), max_abs(c, cr)
    say("iters", info, "err h", eh, "err c", ec)
    assert info[1] == 1 and eh <= FWD_ATOL and ec <= FWD_ATOL


@pytest.mark.parametrize("B,L,H", [(2, 700, 40), (1, 9000, 2)])
def test_iterates_across_chunks(orc, B, L, H):
    """Several chunks per channel: with tol = 0 the k-th result equals the
    oracle's k-th global Newton iterate on both paths."""
    d = synth.lstm_inputs(B, L, H, seed=73, h0=True)
    for k in (1, 2, 4):
        h, c, info = _run(d, 0.0, k)
        hr, cr, it, conv, _ = orc.lstm_newton(*lstm_args(d), h0=d["h0"], c0=d["c0"], tol=0.0, cap=k)
        assert list(info) == [k, 0]
        assert max_abs(h, hr) <= ITER_ATOL and max_abs(c, cr) <= ITER_ATOL, k


def test_large_cap(orc):
    d = synth.lstm_inputs(2, 700, 40, seed=74, h0=True)
    h, c, info = _run(d, 1e-5, 200)
    hr, cr = orc.lstm_rollout(*lstm_args(d), h0=d["h0"], c0=d["c0"])
    assert info[1] == 1 and max_abs(h, hr) <= FWD_ATOL and max_abs(c, cr) <= FWD_ATOL
