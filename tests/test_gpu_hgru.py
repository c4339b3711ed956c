"""GPU parity of the Newton forward of the GRU with dense recurrence inside
heads of k channels (pararnn_hgru_forward: k x k Jacobian blocks, one launch
per iteration on the lane-group scan) against the oracle: single iterates
(tol 0, cap n), the converged solve against the rollout, warm starts,
non-convergence and NaN, the measured workload, and gradients through
generic.head_gru_solve (the library's forward, the adjoint of the solve)."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_pararnn_amd import api, generic, synth
from tests.gpu_helpers import FWD_ATOL, GRAD_RTOL, ITER_ATOL, dev, host, max_abs, rel_inf, say

pytestmark = pytest.mark.gpu


def _args(d):
    return [d[x] for x in ("pz", "pr", "pc", "Uz", "Ur", "Uc")]


def _run(d, tol, cap, init=None, trace=False, ws=None):
    t = [dev(x) for x in _args(d)]
    info = torch.zeros(2, dtype=torch.int32, device="cuda:0")
    tr = torch.zeros(cap, dtype=torch.float32, device="cuda:0") if trace else None
    h = api.hgru_forward(*t, dev(d["h0"]), tol=tol, max_iter=cap, info=info, trace=tr, ws=ws,
                         init=None if init is None else dev(init))
    out = (host(h), host(info).tolist())
    return out + ((host(tr),) if trace else ())


# (B, L, NH, k): heads fewer than a wave holds (8 for k = 8, 16 for k = 4),
# ragged head blocks, ragged chunks, several chunks, one head over a long L
SHAPES = [(2, 300, 3, 8), (2, 97, 13, 8), (1, 64, 1, 8), (1, 700, 8, 8), (3, 257, 9, 4),
          (2, 1000, 20, 4), (1, 3000, 1, 8)]


@pytest.mark.parametrize("B,L,NH,k", SHAPES)
def test_hgru_iterates_equal_oracle_newton(orc, B, L, NH, k):
    say("hgru iterates", B, L, NH, k)
    d = synth.head_gru_inputs(B, L, NH, k, seed=700 + L + NH * k, h0=True)
    for n in (1, 2, 3):
        h, info = _run(d, 0.0, n)
        ref, it, _, _ = orc.hgru_newton(*_args(d), h0=d["h0"], tol=0.0, cap=n)
        err = max_abs(h, ref)
        say(n, info, err)
        assert info == [n, 0] and err <= ITER_ATOL


@pytest.mark.parametrize("B,L,NH,k", SHAPES)
def test_hgru_converges_to_the_rollout(orc, B, L, NH, k):
    d = synth.head_gru_inputs(B, L, NH, k, seed=710 + L + NH * k, h0=True)
    h, info, tr = _run(d, 1e-6, 64, trace=True)
    ref = orc.hgru_rollout(*_args(d), h0=d["h0"])
    _, it, conv, otr = orc.hgru_newton(*_args(d), h0=d["h0"], tol=1e-6, cap=64)
    err = max_abs(h, ref)
    say(B, L, NH, k, info, (it, conv), err, tr[:info[0]])
    assert info[1] == 1 and abs(info[0] - it) <= 1 and err <= FWD_ATOL
    # the reported max|delta| of the first iterations is the oracle's
    for e, oe in list(zip(tr, otr))[:2]:
        assert abs(e - oe) <= 1e-4 * max(1.0, oe)


def test_hgru_full_workload(orc):
    """B=16, L=2048, 64 heads of 8 channels, tol 1e-4, cap 32: every element
    against the oracle's rollout."""
    d = synth.workload_inputs("x_hgru8_fwd")
    h, info = _run(d, 1e-4, 32)
    err = max_abs(h, orc.hgru_rollout(*_args(d), h0=d["h0"]))
    say("hgru full", info, err)
    assert info[1] == 1 and err <= FWD_ATOL


def test_hgru_warm_start(orc):
    d = synth.head_gru_inputs(2, 700, 6, 8, seed=720, h0=True)
    s2, _, _, _ = orc.hgru_newton(*_args(d), h0=d["h0"], tol=0.0, cap=2)
    init = s2.astype(np.float32)
    for n in (1, 2):
        h, info = _run(d, 0.0, n, init=init)
        ref, _, _, _ = orc.hgru_newton(*_args(d), h0=d["h0"], tol=0.0, cap=n, init=init)
        assert info == [n, 0] and max_abs(h, ref) <= ITER_ATOL
    ref = orc.hgru_rollout(*_args(d), h0=d["h0"])
    h, info = _run(d, 1e-5, 32, init=ref.astype(np.float32))
    assert info == [1, 1] and max_abs(h, ref) <= FWD_ATOL


def test_hgru_non_convergence_and_nan_reported():
    d = synth.head_gru_inputs(2, 200, 5, 8, seed=730)
    _, info = _run(d, 0.0, 1)
    assert info == [1, 0]
    d["pz"][1, 50, 3, 2] = np.nan
    _, info = _run(d, 1e-4, 6)
    assert info == [6, 0]


def test_hgru_shares_a_workspace_across_shapes(orc):
    """One workspace for calls of different shapes and both k (launch tags
    keep their records apart)."""
    shapes = [(2, 700, 6, 8), (1, 300, 20, 4), (2, 700, 6, 8)]
    need = max(api.workspace_bytes(api.OP_HGRU8_FORWARD if k == 8 else api.OP_HGRU4_FORWARD, B, L, NH, 16)
               for B, L, NH, k in shapes)
    ws = api.new_workspace(need, torch.device("cuda:0"))
    for r, (B, L, NH, k) in enumerate(shapes):
        d = synth.head_gru_inputs(B, L, NH, k, seed=740 + r, h0=True)
        h, info = _run(d, 1e-6, 16, ws=ws)
        assert info[1] == 1 and max_abs(h, orc.hgru_rollout(*_args(d), h0=d["h0"])) <= FWD_ATOL


def test_hgru_rejects_bad_arguments():
    d = synth.head_gru_inputs(1, 64, 2, 8, seed=750)
    t = [dev(x) for x in _args(d)]
    out = torch.empty(1, 64, 2, 8, device="cuda:0")
    with pytest.raises(api.PararnnError):
        api.hgru_forward(*t, None, out=out, init=out)  # initial iterate overlaps the output
    p3 = torch.zeros(1, 64, 2, 3, device="cuda:0")
    U3 = torch.zeros(2, 3, 3, device="cuda:0")
    with pytest.raises(api.PararnnError):
        api.hgru_forward(p3, p3, p3, U3, U3, U3)  # k = 3


@pytest.mark.parametrize("B,L,NH,k", [(2, 300, 3, 8), (2, 1000, 20, 4)])
def test_head_gru_solve_gradients_match_oracle(orc, B, L, NH, k):
    """generic.head_gru_solve: the library's forward, gradients for p, U and
    h0 through the adjoint of the solve, against the oracle's rollout and
    backpropagation through time."""
    d = synth.head_gru_inputs(B, L, NH, k, seed=760 + NH, h0=True, grad=True)
    p = [dev(d[x]).requires_grad_(True) for x in ("pz", "pr", "pc")]
    U = [dev(d[x]).requires_grad_(True) for x in ("Uz", "Ur", "Uc")]
    h0 = dev(d["h0"]).requires_grad_(True)
    info = [0, 0]
    h = generic.head_gru_solve(*p, *U, h0, tol=1e-6, max_iter=64, info=info)
    href = orc.hgru_rollout(*_args(d), h0=d["h0"])
    (h * dev(d["g"])).sum().backward()
    ref = orc.hgru_bptt(*_args(d), href, d["g"], h0=d["h0"])
    got = [x.grad for x in p + U] + [h0.grad]
    errs = {n: rel_inf(host(gv), rv) for n, gv, rv in zip(["dpz", "dpr", "dpc", "dUz", "dUr", "dUc", "dh0"], got, ref)}
    err = max_abs(host(h), href)
    say(info, err, errs)
    assert info[1] == 1 and err <= FWD_ATOL
    assert max(errs.values()) <= GRAD_RTOL, errs
