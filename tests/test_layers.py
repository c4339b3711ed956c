"""Trainable layers on the CPU: the autograd wiring (projection GEMMs, the
solve's backward returning dL/dp, dL/du, dL/dh0, dL/dc0 in the right slots)
checked against torch autograd through a sequential fp64 rollout
(tests/layer_ref.py).  The library's solve and adjoint are replaced here by
the oracle's rollout and backpropagation through time, so only the layer code
is under test; the GPU parity of the real path is in test_gpu_layers.py."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_pararnn_amd import api, layers, synth
from tests.gpu_helpers import FWD_ATOL, GRAD_RTOL, max_abs, rel_inf
from tests.layer_ref import reference, run_layer


def _np(t):
    return None if t is None else t.detach().numpy()


@pytest.fixture
def oracle_solve(orc, monkeypatch):
    def gru_forward(pz, pr, pc, uz, ur, uc, h0=None, *, tol, max_iter, info=None, **kw):
        h = orc.gru_rollout(*[_np(t) for t in (pz, pr, pc, uz, ur, uc)], h0=_np(h0))
        if info is not None:
            info.copy_(torch.tensor([1, 1], dtype=torch.int32))
        return torch.from_numpy(h.astype(np.float32))

    def lstm_forward(pi, pf, po, pg, ui, uf, uo, ug, h0=None, c0=None, *, tol, max_iter,
                     info=None, **kw):
        h, c = orc.lstm_rollout(*[_np(t) for t in (pi, pf, po, pg, ui, uf, uo, ug)],
                                h0=_np(h0), c0=_np(c0))
        if info is not None:
            info.copy_(torch.tensor([1, 1], dtype=torch.int32))
        return torch.from_numpy(h.astype(np.float32)), torch.from_numpy(c.astype(np.float32))

    def adjoint_backward(cell, p, u, h, grad_h, h0=None, *, c=None, c0=None, grad_c=None,
                         want_u=True, want_h0=True, want_c0=True, ws=None):
        f32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32))
        if cell == api.CELL_GRU:
            dp, du, dh0 = orc.gru_bptt(*[_np(t) for t in p], *[_np(t) for t in u], _np(h),
                                       _np(grad_h), h0=_np(h0))
            dc0 = None
        else:
            dp, du, dh0, dc0 = orc.lstm_bptt(*[_np(t) for t in p], *[_np(t) for t in u], _np(h),
                                             _np(c), _np(grad_h), _np(grad_c), h0=_np(h0),
                                             c0=_np(c0))
        return {"p": [f32(x) for x in dp], "u": [f32(x) for x in du] if want_u else None,
                "h0": f32(dh0) if want_h0 else None,
                "c0": f32(dc0) if (want_c0 and dc0 is not None) else None}

    monkeypatch.setattr(api, "gru_forward", gru_forward)
    monkeypatch.setattr(api, "lstm_forward", lstm_forward)
    monkeypatch.setattr(api, "adjoint_backward", adjoint_backward)


def _compare(got, ref):
    for k in ("h", "c"):
        if k in ref:
            assert max_abs(got[k], ref[k]) <= FWD_ATOL, k
    errs = {k: rel_inf(got[k], ref[k]) for k in ref if k.startswith("d")}
    assert set(errs) == {k for k in got if k.startswith("d")}
    assert max(errs.values()) <= GRAD_RTOL, errs


@pytest.mark.parametrize("kind", ["gru", "lstm"])
@pytest.mark.parametrize("with_h0", [True, False])
def test_layer_gradients_match_autograd_rollout(oracle_solve, kind, with_h0):
    d = synth.layer_inputs(2, 37, 5, 6, 3 if kind == "gru" else 4, seed=140)
    _compare(run_layer(kind, d, "cpu", with_h0=with_h0), reference(kind, d, with_h0=with_h0))


def test_layer_without_bias(oracle_solve):
    d = synth.layer_inputs(2, 25, 3, 4, 4, seed=142)
    _compare(run_layer("lstm", d, "cpu", bias=False), reference("lstm", d, bias=False))


@pytest.mark.parametrize("loss_on", [("h",), ("c",)])
def test_lstm_loss_on_one_output(oracle_solve, loss_on):
    d = synth.layer_inputs(2, 20, 4, 3, 4, seed=141)
    _compare(run_layer("lstm", d, "cpu", loss_on=loss_on), reference("lstm", d, loss_on=loss_on))


def test_layer_shapes_and_arguments():
    m = layers.ParaGRU(7, 5)
    assert tuple(m.weight.shape) == (3, 5, 7) and tuple(m.u.shape) == (3, 5)
    assert tuple(layers.ParaLSTM(7, 5, bias=False).weight.shape) == (4, 5, 7)
    assert layers.ParaLSTM(7, 5, bias=False).bias is None
    with pytest.raises(ValueError):
        layers.ParaGRU(0, 5)
    with pytest.raises(ValueError):
        layers.ParaGRU(3, 5, tol=-1.0)
    with pytest.raises(ValueError):
        m(torch.zeros(2, 4, 6))  # wrong feature size


def test_layer_has_no_cpu_path():
    """Without the stand-ins the solve runs only in the HIP library, which
    rejects host tensors."""
    m = layers.ParaGRU(3, 4)
    with pytest.raises((ValueError, api.PararnnError)):
        m(torch.zeros(1, 5, 3))


def test_generic_solve_has_no_cpu_path():
    """The generic Newton solve assembles with torch but solves with the HIP
    scan, which rejects host tensors."""
    from nonlinear_rnn_solve_pararnn_amd import generic
    x = torch.zeros(1, 5, 3)
    with pytest.raises((ValueError, api.PararnnError)):
        generic.newton_solve(lambda h, p: torch.tanh(p + h), [x])
