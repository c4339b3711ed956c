"""GPU parity of the GRU Newton forward (the fused on-chip path, the chained
path that keeps every chunk on chip for all iterations, and the
per-iteration path) against the fp64 oracle: the sequential rollout, and the
oracle's own Newton iterates."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_pararnn_amd import api, synth
from tests.gpu_helpers import (FWD_ATOL, ITER_ATOL, dev, gru_args, host, max_abs, say)

pytestmark = pytest.mark.gpu
# "chain" and "local" force the two forms of the chained kernel (chunks chained
# across workgroups; workgroups owning whole chains, channel lanes only).
PATHS = ["fused", "chain", "local", "step"]


def _run(d, tol, cap, with_h0=True, trace=False):
    ins = [dev(x) for x in gru_args(d)]
    info = torch.zeros(2, dtype=torch.int32, device="cuda:0")
    tr = torch.zeros(cap, dtype=torch.float32, device="cuda:0") if trace else None
    h = api.gru_forward(*ins, dev(d["h0"]) if with_h0 else None, tol=tol, max_iter=cap,
                        info=info, trace=tr)
    out = host(h), host(info)
    return out + ((host(tr),) if trace else ())


@pytest.mark.parametrize("path", PATHS)
def test_tiny_workload_matches_rollout(orc, monkeypatch, path):
    """B=1, L=64, H=4, tol 1e-6, cap 64 (= L, the guaranteed bound)."""
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    d = synth.workload_inputs("c0_gru_tiny")
    h, info = _run(d, 1e-6, 64)
    ref = orc.gru_rollout(*gru_args(d), h0=d["h0"])
    say(path, "iters", info, "err", max_abs(h, ref))
    assert max_abs(h, ref) <= FWD_ATOL
    _, it, conv, _ = orc.gru_newton(*gru_args(d), h0=d["h0"], tol=1e-6, cap=64)
    assert info[1] == 1 and abs(int(info[0]) - it) <= 1


@pytest.mark.parametrize("path", PATHS)
def test_iterates_match_oracle_newton(orc, monkeypatch, path):
    """cap = k, tol = 0: the k-th GPU iterate equals the oracle's k-th Newton
    iterate (pins the zero start, the delta form and the time indexing)."""
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    d = synth.workload_inputs("c0_gru_tiny")
    for k in range(1, 7):
        h, info = _run(d, 0.0, k)
        s, it, conv, _ = orc.gru_newton(*gru_args(d), h0=d["h0"], tol=0.0, cap=k)
        assert info[0] == k and info[1] == 0
        assert max_abs(h, s) <= ITER_ATOL, k


@pytest.mark.parametrize("path", PATHS)
def test_L_iterations_reproduce_rollout(orc, monkeypatch, path):
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    d = synth.gru_inputs(2, 64, 5, seed=31, h0=True)
    h, info = _run(d, 0.0, 64)
    assert max_abs(h, orc.gru_rollout(*gru_args(d), h0=d["h0"])) <= FWD_ATOL


# H = 31 is the widest time-lane layout, H = 32 the narrowest channel-lane one.
SHAPES = [(1, 1, 1), (2, 100, 70), (3, 37, 5), (2, 512, 20), (1, 33, 16), (4, 300, 130), (2, 300, 31),
          (2, 300, 32)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("B,L,H", SHAPES)
def test_shapes_match_rollout(orc, monkeypatch, path, B, L, H):
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    say("gru", path, B, L, H)
    d = synth.gru_inputs(B, L, H, seed=40 + L + H, h0=True)
    h, info = _run(d, 1e-5, 64)
    assert info[1] == 1
    assert max_abs(h, orc.gru_rollout(*gru_args(d), h0=d["h0"])) <= FWD_ATOL


@pytest.mark.parametrize("path", ["chain", "local", "step"])
@pytest.mark.parametrize("B,L,H", [(2, 513, 20), (1, 5000, 3), (2, 700, 100), (3, 20000, 1),
                                   (1, 12, 1), (2, 4098, 1), (2, 8192, 1), (2, 3000, 200)])
def test_long_sequences(orc, monkeypatch, path, B, L, H):
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    say("gru long", path, B, L, H)
    d = synth.gru_inputs(B, L, H, seed=50 + H, h0=True)
    h, info = _run(d, 1e-5, 32)
    assert info[1] == 1
    assert max_abs(h, orc.gru_rollout(*gru_args(d), h0=d["h0"])) <= FWD_ATOL


def test_fused_workload_full(orc):
    """B=16, L=512, H=4096, p = 0.5 N(0,1), tol 1e-4, cap 32: every output checked."""
    say("gru fused full workload")
    d = synth.workload_inputs("c2_gru_fused")
    h, info = _run(d, 1e-4, 32, with_h0=False)
    ref = orc.gru_rollout(*gru_args(d))
    err = max_abs(h, ref)
    say("iters", info, "err", err)
    assert info[1] == 1 and err <= FWD_ATOL


@pytest.mark.parametrize("path", ["chain", "step"])
def test_long_workload_forward_full(orc, monkeypatch, path):
    """B=16, L=1,048,576, H=1, tol 1e-4, cap 32: every output checked, on the
    chained kernel and on the per-iteration launches."""
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    say("gru long workload", path)
    d = synth.workload_inputs("c4_gru_long_fwd_adj")
    h, info = _run(d, 1e-4, 32, with_h0=False)
    ref = orc.gru_rollout(*gru_args(d))
    err = max_abs(h, ref)
    say("iters", info, "err", err)
    assert info[1] == 1 and err <= FWD_ATOL


@pytest.mark.parametrize("path", PATHS)
def test_u0_equals_linear_scan(monkeypatch, path):
    """u = 0 makes the cell affine in h: the result must equal the exported
    diagonal scan with a = 1 - sigmoid(pz), b = sigmoid(pz) tanh(pc)."""
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    d = synth.gru_inputs(2, 400, 40, seed=60, zero_u=True)
    h, info = _run(d, 1e-6, 10, with_h0=False)
    z = 1.0 / (1.0 + np.exp(-d["pz"].astype(np.float64)))
    a = (1.0 - z).astype(np.float32)
    b = (z * np.tanh(d["pc"].astype(np.float64))).astype(np.float32)
    hs = host(api.linscan_diag(dev(a), dev(b)))
    assert max_abs(h, hs) <= 1e-5
    assert info[0] <= 2 and info[1] == 1


@pytest.mark.parametrize("path", PATHS)
def test_non_convergence_and_nan_reported(monkeypatch, path):
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    d = synth.gru_inputs(2, 200, 20, seed=61)
    _, info = _run(d, 0.0, 1)
    assert list(info) == [1, 0]
    d["pz"][1, 50, 3] = np.nan
    _, info = _run(d, 1e-4, 6)
    assert list(info) == [6, 0]


@pytest.mark.parametrize("path", PATHS)
def test_trace_shows_quadratic_convergence(monkeypatch, path):
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    d = synth.gru_inputs(4, 256, 64, seed=62)
    h, info, tr = _run(d, 0.0, 8, trace=True)
    tr = [float(x) for x in tr]
    say(path, "trace", tr)
    # once below 1e-2 the next error is at most ~C e^2 (until fp32 rounding)
    for e, en in zip(tr, tr[1:]):
        if 1e-5 < e < 1e-2:
            assert en <= 10 * e * e + 1e-6


def test_invalid_arguments_raise():
    d = synth.gru_inputs(1, 10, 4, seed=63)
    ins = [dev(x) for x in gru_args(d)]
    with pytest.raises(api.PararnnError):
        api.gru_forward(*ins, tol=-1.0)
    with pytest.raises(api.PararnnError):
        api.gru_forward(*ins, tol=float("nan"))
    with pytest.raises(api.PararnnError):
        api.gru_forward(*ins, max_iter=0)


@pytest.mark.parametrize("path,B,L,H", [("step", 16, 20000, 1), ("step", 4, 3000, 256),
                                        ("chain", 16, 20000, 1), ("chain", 4, 3000, 256),
                                        ("fused", 16, 512, 1024)])
def test_trace_equals_oracle_newton_trace(orc, monkeypatch, path, B, L, H):
    """max|delta| of each iteration, reduced over thousands of workgroups on
    every XCD, equals the oracle's global max (a lost update would show)."""
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    d = synth.gru_inputs(B, L, H, seed=64)
    cap = 3
    h, info, tr = _run(d, 0.0, cap, with_h0=False, trace=True)
    _, it, conv, otr = orc.gru_newton(*gru_args(d), tol=0.0, cap=cap)
    say(path, "gpu trace", list(tr), "oracle", list(otr))
    for k in range(cap):
        assert abs(float(tr[k]) - otr[k]) <= 1e-4 * otr[k] + 1e-6, (k, tr, otr)


def test_fused_full_tiles_with_h0_and_iterates(orc):
    """Full 16-channel tiles of 512 positions (the unmasked kernel) with a
    non-zero h0, and their first iterates against the oracle's Newton iterates."""
    d = synth.gru_inputs(8, 512, 2048, seed=65, h0=True)
    h, info = _run(d, 1e-5, 32)
    assert info[1] == 1
    assert max_abs(h, orc.gru_rollout(*gru_args(d), h0=d["h0"])) <= FWD_ATOL
    for k in (1, 2, 3):
        h, info = _run(d, 0.0, k)
        s, it, conv, _ = orc.gru_newton(*gru_args(d), h0=d["h0"], tol=0.0, cap=k)
        assert list(info) == [k, 0]
        assert max_abs(h, s) <= ITER_ATOL, k


@pytest.mark.parametrize("path", ["chain", "local"])
@pytest.mark.parametrize("B,L,H", [(2, 1000, 40), (2, 20000, 1)])
def test_chain_iterates_across_chunks(orc, monkeypatch, path, B, L, H):
    """Chained path over several chunks (channel lanes: 64-position chunks;
    time lanes: 12288): with tol = 0 no chunk stops early, so the k-th result
    equals the oracle's k-th global Newton iterate."""
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    d = synth.gru_inputs(B, L, H, seed=66, h0=True)
    for k in (1, 2, 3, 5):
        h, info = _run(d, 0.0, k)
        s, it, conv, _ = orc.gru_newton(*gru_args(d), h0=d["h0"], tol=0.0, cap=k)
        say("chain", B, L, H, k, info, max_abs(h, s))
        assert list(info) == [k, 0]
        assert max_abs(h, s) <= ITER_ATOL, k


def test_large_cap_takes_per_iteration_path(orc, monkeypatch):
    """A cap above the chained kernel's limit (its workspace holds every
    iteration's records) runs the per-iteration launches, with the same result."""
    monkeypatch.setenv("PARARNN_GRU_PATH", "chain")
    d = synth.gru_inputs(2, 2000, 40, seed=67, h0=True)
    h, info = _run(d, 1e-5, 200)
    assert info[1] == 1
    assert max_abs(h, orc.gru_rollout(*gru_args(d), h0=d["h0"])) <= FWD_ATOL


@pytest.mark.parametrize("path", ["fused", "chain", "local", "step"])
def test_cap_beyond_sequence_length(orc, monkeypatch, path):
    """A cap far above L is taken as L + 1 (exact after L updates, confirmed by
    the next): same result and count as the oracle, trace zero past the cap."""
    monkeypatch.setenv("PARARNN_GRU_PATH", path)
    d = synth.gru_inputs(2, 20, 5, seed=68, h0=True)
    h, info, tr = _run(d, 0.0, 1000, trace=True)
    s, it, conv, _ = orc.gru_newton(*gru_args(d), h0=d["h0"], tol=0.0, cap=21)
    assert max_abs(h, orc.gru_rollout(*gru_args(d), h0=d["h0"])) <= FWD_ATOL
    assert int(info[0]) <= 21
    assert float(abs(tr[21:]).max()) == 0.0
