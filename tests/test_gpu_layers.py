"""GPU parity of the trainable layers: the Newton solve and its adjoint in
libpararnn.so, plus the projection GEMMs, against torch autograd through a
sequential fp64 rollout on the CPU (tests/layer_ref.py).  Shapes cover the
fused kernel (L <= 512), the chained kernel with channel lanes (H >= 32) and
with time lanes (H < 32)."""
import pytest

from nonlinear_rnn_solve_pararnn_amd import synth
from tests.gpu_helpers import DEV, FWD_ATOL, GRAD_RTOL, max_abs, rel_inf, say
from tests.layer_ref import reference, run_layer

pytestmark = pytest.mark.gpu

SHAPES = [(2, 37, 5, 6), (2, 300, 8, 64), (1, 700, 6, 40), (2, 900, 4, 3)]


def _check(kind, got, ref):
    fwd = {k: max_abs(got[k], ref[k]) for k in ("h", "c") if k in ref}
    errs = {k: rel_inf(got[k], ref[k]) for k in ref if k.startswith("d")}
    say(kind, got["info"], fwd, errs)
    assert got["info"][1] == 1
    assert max(fwd.values()) <= FWD_ATOL, fwd
    assert max(errs.values()) <= GRAD_RTOL, errs


@pytest.mark.parametrize("kind", ["gru", "lstm"])
@pytest.mark.parametrize("B,L,D,H", SHAPES)
def test_layer_matches_autograd_rollout(kind, B, L, D, H):
    say("layer", kind, B, L, D, H)
    d = synth.layer_inputs(B, L, D, H, 3 if kind == "gru" else 4, seed=150 + H)
    _check(kind, run_layer(kind, d, DEV), reference(kind, d))


@pytest.mark.parametrize("kind", ["gru", "lstm"])
def test_layer_without_initial_state(kind):
    d = synth.layer_inputs(2, 200, 5, 33, 3 if kind == "gru" else 4, seed=160)
    _check(kind, run_layer(kind, d, DEV, with_h0=False), reference(kind, d, with_h0=False))


@pytest.mark.parametrize("loss_on", [("h",), ("c",)])
def test_lstm_layer_loss_on_one_output(loss_on):
    d = synth.layer_inputs(2, 150, 4, 40, 4, seed=161)
    _check("lstm", run_layer("lstm", d, DEV, loss_on=loss_on), reference("lstm", d, loss_on=loss_on))


def test_layer_without_bias_on_the_per_iteration_path():
    """bias=False, and a cap above the chained kernel's limit (per-iteration
    launches) with L > 512."""
    d = synth.layer_inputs(2, 700, 5, 40, 3, seed=162)
    got = run_layer("gru", d, DEV, max_iter=100, bias=False)
    assert "dbias" not in got
    _check("gru", got, reference("gru", d, bias=False))


def test_layer_inference_without_grad():
    import torch
    from nonlinear_rnn_solve_pararnn_amd import layers
    m = layers.ParaLSTM(4, 33, device=DEV)
    x = torch.randn(2, 50, 4, device=DEV)
    with torch.no_grad():
        h, c = m(x)
    assert not h.requires_grad and h.shape == (2, 50, 33) and c.shape == (2, 50, 33)
    assert m.last_info.cpu().tolist()[1] == 1
