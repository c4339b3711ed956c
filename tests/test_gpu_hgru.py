"""GPU parity of the Newton forward of the GRU with dense recurrence inside
heads of k channels (pararnn_hgru_forward: k x k Jacobian blocks, one launch
per iteration on the lane-group scan) against the oracle: single iterates
(tol 0, cap n), the converged solve against the rollout, warm starts,
non-convergence and NaN, the measured workload; the adjoint kernel
(pararnn_hgru_backward) against the oracle's backpropagation through time,
and gradients through generic.head_gru_solve (both kernels under autograd)."""
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


@pytest.mark.parametrize("B,L,NH,k", SHAPES + [(1, 1, 1, 8), (2, 5, 3, 4)])
@pytest.mark.parametrize("with_h0", [False, True])
def test_hgru_backward_matches_oracle_bptt(orc, B, L, NH, k, with_h0):
    """The adjoint kernel against the oracle's backpropagation through time,
    both at the oracle's rollout: dp, dU and dh0 at GRAD_RTOL each."""
    say("hgru_backward", B, L, NH, k, with_h0)
    d = synth.head_gru_inputs(B, L, NH, k, seed=800 + 7 * NH + L % 97, h0=with_h0, grad=True)
    h = orc.hgru_rollout(*_args(d), h0=d["h0"]).astype(np.float32)
    ref = orc.hgru_bptt(*_args(d), h, d["g"], h0=d["h0"])
    got = api.hgru_backward(*[dev(x) for x in _args(d)], dev(d["h0"]) if with_h0 else None, dev(h),
                            dev(d["g"]))
    names = ["dpz", "dpr", "dpc", "dUz", "dUr", "dUc", "dh0"]
    errs = {n: rel_inf(host(gv), rv) for n, gv, rv in zip(names, got, ref)}
    say(errs)
    assert max(errs.values()) <= GRAD_RTOL, errs


def test_hgru_backward_full_workload(orc):
    """B=16, L=2048, 64 heads of 8 channels (the forward's measured
    workload) at the converged forward's states, every gradient against the
    oracle's backpropagation through time at those states."""
    say("hgru_backward full workload")
    d = synth.head_gru_inputs(16, 2048, 64, 8, seed=830, grad=True)
    t = [dev(x) for x in _args(d)]
    h = api.hgru_forward(*t, None, tol=1e-4, max_iter=32)
    hh = host(h)
    ref = orc.hgru_bptt(*_args(d), hh, d["g"])
    got = api.hgru_backward(*t, None, h, dev(d["g"]))
    names = ["dpz", "dpr", "dpc", "dUz", "dUr", "dUc", "dh0"]
    errs = {n: rel_inf(host(gv), rv) for n, gv, rv in zip(names, got, ref)}
    say(errs)
    assert max(errs.values()) <= GRAD_RTOL, errs


def test_hgru_backward_options_and_reuse(orc):
    """Without dL/dU and dL/dh0 the other gradients are unchanged; the
    gradients may overwrite the inputs p; one workspace serves two shapes and
    both k in a row (the partials of the first call are not read by the
    second)."""
    d = synth.head_gru_inputs(2, 300, 5, 8, seed=840, h0=True, grad=True)
    h = orc.hgru_rollout(*_args(d), h0=d["h0"]).astype(np.float32)
    ref = orc.hgru_bptt(*_args(d), h, d["g"], h0=d["h0"])
    ws = api.new_workspace(max(api.workspace_bytes(api.OP_HGRU8_BACKWARD, 2, 300, 5),
                               api.workspace_bytes(api.OP_HGRU4_BACKWARD, 3, 200, 7)), torch.device("cuda:0"))
    full = api.hgru_backward(*[dev(x) for x in _args(d)], dev(d["h0"]), dev(h), dev(d["g"]), ws=ws)
    part = api.hgru_backward(*[dev(x) for x in _args(d)], dev(d["h0"]), dev(h), dev(d["g"]),
                             want_u=False, want_h0=False, ws=ws)
    assert part[3] is None and part[6] is None
    for a, b in zip(full[:3], part[:3]):
        assert torch.equal(a, b)
    d4 = synth.head_gru_inputs(3, 200, 7, 4, seed=841, grad=True)
    h4 = orc.hgru_rollout(*_args(d4)).astype(np.float32)
    ref4 = orc.hgru_bptt(*_args(d4), h4, d4["g"])
    got4 = api.hgru_backward(*[dev(x) for x in _args(d4)], None, dev(h4), dev(d4["g"]), ws=ws)
    assert max(rel_inf(host(a), b) for a, b in zip(got4, ref4)) <= GRAD_RTOL
    # the gradients written over the inputs p (each element is read before it is written)
    t = [dev(x) for x in _args(d)]
    h0_d, h_d, g_d = dev(d["h0"]), dev(h), dev(d["g"])  # held: the call takes raw pointers
    lib = api.load_library()
    gU = [torch.empty_like(t[3]) for _ in range(3)]
    gh0 = torch.empty(2, 5, 8, device="cuda:0")
    n = api.workspace_bytes(api.OP_HGRU8_BACKWARD, 2, 300, 5)
    st = lib.pararnn_hgru_backward(8, 2, 300, 5, *[api._ptr(x) for x in t], api._ptr(h0_d),
                                   api._ptr(h_d), api._ptr(g_d), *[api._ptr(x) for x in t[:3]],
                                   *[api._ptr(x) for x in gU], api._ptr(gh0), api._ptr(ws), n,
                                   api._stream(torch.device("cuda:0")))
    assert st == 0
    errs = [rel_inf(host(a), b) for a, b in zip(t[:3] + gU + [gh0], ref)]
    assert max(errs) <= GRAD_RTOL, errs


def test_hgru_backward_rejects_bad_arguments():
    d = synth.head_gru_inputs(1, 64, 2, 8, seed=850, grad=True)
    t = [dev(x) for x in _args(d)]
    h = torch.zeros(1, 64, 2, 8, device="cuda:0")
    g = dev(d["g"])
    lib = api.load_library()
    ws = api.new_workspace(api.workspace_bytes(api.OP_HGRU8_BACKWARD, 1, 64, 2), torch.device("cuda:0"))
    n = ws.numel()
    s = api._stream(torch.device("cuda:0"))

    def call(k=8, gp=None, wsb=n):
        gp = gp or [torch.empty_like(t[0]) for _ in range(3)]
        return lib.pararnn_hgru_backward(k, 1, 64, 2, *[api._ptr(x) for x in t], None, api._ptr(h), api._ptr(g),
                                         *[api._ptr(x) for x in gp], None, None, None, None, api._ptr(ws), wsb, s)
    assert call() == 0
    assert call(gp=[h, torch.empty_like(h), torch.empty_like(h)]) != 0  # a gradient over h
    assert call(k=3) != 0
    assert call(k=0) != 0
    assert call(wsb=n - 256) != 0  # workspace too small
