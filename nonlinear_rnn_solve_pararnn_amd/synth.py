"""Seeded synthetic inputs for the five workloads and for ad-hoc test shapes.

This module only draws random numbers: it holds none of the method's
arithmetic, so both the fp64 oracle and the GPU path can take their inputs
from it without sharing any computation.

Every draw uses ``numpy.random.Generator(PCG64(seed))``, is made in fp64 in the
order listed, each tensor in C order, and is then rounded to fp32.  The oracle
up-casts those same fp32 values back to fp64, so both sides see identical
inputs.

The pages (ParaRNN, Fig. 2 and Fig. 5 captions; DEER summary, results
paragraph) measure on trained cells and evaluation datasets that are not
available; freshly-initialised-like draws stand in for them:
gate pre-projections ~ N(0,1) (or 0.5*N(0,1)), diagonal recurrent weights
u ~ U(-0.5, 0.5), and zero initial state.

Layout of every sequence tensor is [B, L, H] (channel index fastest).
"""
from __future__ import annotations

import numpy as np

# Workload table: name -> description used by bench.py and the tests.
WORKLOADS = {
    "c0_gru_tiny": dict(kind="gru", B=1, L=64, H=4, tol=1e-6, cap=64),
    "c1_linscan": dict(kind="linscan_diag", B=16, L=4096, H=1024),
    "c2_gru_fused": dict(kind="gru", B=16, L=512, H=4096, tol=1e-4, cap=32),
    "c3_lstm": dict(kind="lstm", B=8, L=2048, H=2048, tol=1e-4, cap=32),
    "c4_gru_long_fwd_adj": dict(kind="gru_adjoint", B=16, L=1048576, H=1,
                                tol=1e-4, cap=32),
    # the exported 2x2 block scan at the diagonal scan's element count / 2
    "x_linscan_blk2": dict(kind="linscan_blk2", B=16, L=4096, H=512),
    # the LSTM adjoint at the LSTM forward's shape, with upstream gradients on h and c
    "x_lstm_adjoint": dict(kind="lstm_adjoint", B=8, L=2048, H=2048, tol=1e-4, cap=32),
    # the per-iteration Newton path (one launch per iteration) on the inputs of
    # the LSTM forward and of the long GRU forward
    "x_lstm_step": dict(kind="lstm", B=8, L=2048, H=2048, tol=1e-4, cap=32, same_as="c3_lstm"),
    "x_gru_long_step": dict(kind="gru", B=16, L=1048576, H=1, tol=1e-4, cap=32,
                            same_as="c4_gru_long_fwd_adj"),
    # sequential application (one thread per channel) on the inputs of the
    # fused GRU forward, the LSTM forward and the long GRU forward
    # the long GRU forward alone (chained kernel), for its ratio to sequential application
    "x_gru_long_fwd": dict(kind="gru", B=16, L=1048576, H=1, tol=1e-4, cap=32,
                           same_as="c4_gru_long_fwd_adj"),
    "x_gru_seq": dict(kind="gru", B=16, L=512, H=4096, same_as="c2_gru_fused"),
    "x_lstm_seq": dict(kind="lstm", B=8, L=2048, H=2048, same_as="c3_lstm"),
    "x_gru_long_seq": dict(kind="gru", B=16, L=1048576, H=1, same_as="c4_gru_long_fwd_adj"),
    # the 4x4 block scan at the diagonal scan's byte count (96 B per block position)
    "x_linscan_blk4": dict(kind="linscan_blk", B=16, L=2048, H=256, k=4),
    # 8x8 blocks: heads of 8 channels with dense recurrence inside a head,
    # 64 heads (512 channels), 320 B per block position
    "x_linscan_blk8": dict(kind="linscan_blk", B=16, L=2048, H=64, k=8),
    # Newton forward of the GRU with dense recurrence inside heads of 8
    # channels (8x8 Jacobian blocks), 64 heads (512 channels)
    "x_hgru8_fwd": dict(kind="hgru", B=16, L=2048, H=64, k=8, tol=1e-4, cap=32),
    # its gradients: the adjoint at the converged forward's states, with
    # upstream gradients ~ N(0,1)
    "x_hgru8_bwd": dict(kind="hgru", B=16, L=2048, H=64, k=8, tol=1e-4, cap=32),
}
WORKLOAD_ORDER = list(WORKLOADS)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape, scale=1.0):
    x = rng.standard_normal(size=shape)
    if scale != 1.0:
        x = x * scale
    return x.astype(np.float32)


def _uniform(rng, shape, lo, hi):
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def gru_inputs(B, L, H, seed, pscale=1.0, ulo=-0.5, uhi=0.5, h0=False,
               grad=False, zero_u=False):
    """GRU draws: pz, pr, pc ~ pscale*N(0,1) [B,L,H]; uz, ur, uc ~ U(ulo,uhi) [H];
    then optionally h0 ~ U(-0.9,0.9) [B,H] and the upstream gradient g ~ N(0,1)."""
    rng = _rng(seed)
    out = {}
    for k in ("pz", "pr", "pc"):
        out[k] = _normal(rng, (B, L, H), pscale)
    for k in ("uz", "ur", "uc"):
        out[k] = _uniform(rng, (H,), ulo, uhi)
        if zero_u:
            out[k][:] = 0.0
    out["h0"] = _uniform(rng, (B, H), -0.9, 0.9) if h0 else np.zeros((B, H), np.float32)
    if grad:
        out["g"] = _normal(rng, (B, L, H))
    return out


def head_gru_inputs(B, L, NH, k, seed, h0=False, grad=False):
    """Draws for the GRU with dense recurrence inside heads of k channels:
    pz, pr, pc ~ N(0,1) [B,L,NH,k]; Uz, Ur, Uc [NH,k,k] with diagonal
    U(-0.5,0.5) (the diagonal cell's u) and off-diagonal U(-0.3,0.3)/sqrt(k);
    then optionally h0 ~ U(-0.9,0.9) [B,NH,k] and g ~ N(0,1) [B,L,NH,k]."""
    rng = _rng(seed)
    out = {}
    for key in ("pz", "pr", "pc"):
        out[key] = _normal(rng, (B, L, NH, k))
    for key in ("Uz", "Ur", "Uc"):
        off = _uniform(rng, (NH, k, k), -0.3, 0.3) / np.float32(np.sqrt(k))
        diag = _uniform(rng, (NH, k), -0.5, 0.5)
        idx = np.arange(k)
        off[:, idx, idx] = diag
        out[key] = off.astype(np.float32)
    out["h0"] = _uniform(rng, (B, NH, k), -0.9, 0.9) if h0 else np.zeros((B, NH, k), np.float32)
    if grad:
        out["g"] = _normal(rng, (B, L, NH, k))
    return out


def lstm_inputs(B, L, H, seed, pscale=1.0, ulo=-0.5, uhi=0.5, h0=False,
                grad=False, zero_u=False):
    """LSTM draws: pi, pf, po, pg ~ pscale*N(0,1) [B,L,H]; ui, uf, uo, ug ~ U(ulo,uhi);
    then optionally h0, c0 ~ U(-0.9,0.9) [B,H] and upstream gradients gh, gc ~ N(0,1)."""
    rng = _rng(seed)
    out = {}
    for k in ("pi", "pf", "po", "pg"):
        out[k] = _normal(rng, (B, L, H), pscale)
    for k in ("ui", "uf", "uo", "ug"):
        out[k] = _uniform(rng, (H,), ulo, uhi)
        if zero_u:
            out[k][:] = 0.0
    if h0:
        out["h0"] = _uniform(rng, (B, H), -0.9, 0.9)
        out["c0"] = _uniform(rng, (B, H), -0.9, 0.9)
    else:
        out["h0"] = np.zeros((B, H), np.float32)
        out["c0"] = np.zeros((B, H), np.float32)
    if grad:
        out["gh"] = _normal(rng, (B, L, H))
        out["gc"] = _normal(rng, (B, L, H))
    return out


def layer_inputs(B, L, D, H, ngates, seed):
    """Trainable-layer draws: x ~ N(0,1) [B,L,D]; weight ~ U(-1/sqrt(D), 1/sqrt(D))
    [ngates,H,D]; bias ~ U(-0.5,0.5) [ngates,H]; u ~ U(-0.5,0.5) [ngates,H];
    h0, c0 ~ U(-0.9,0.9) [B,H]; upstream gradients gh, gc ~ N(0,1) [B,L,H]."""
    rng = _rng(seed)
    k = 1.0 / np.sqrt(D)
    out = {"x": _normal(rng, (B, L, D)),
           "weight": _uniform(rng, (ngates, H, D), -k, k),
           "bias": _uniform(rng, (ngates, H), -0.5, 0.5),
           "u": _uniform(rng, (ngates, H), -0.5, 0.5),
           "h0": _uniform(rng, (B, H), -0.9, 0.9),
           "c0": _uniform(rng, (B, H), -0.9, 0.9),
           "gh": _normal(rng, (B, L, H)),
           "gc": _normal(rng, (B, L, H))}
    return out


def linscan_diag_inputs(B, L, H, seed, alo=0.5, ahi=1.0, h0=False):
    """Diagonal linear recurrence draws: a ~ U(alo,ahi), b ~ N(0,1) [B,L,H];
    optionally h0 ~ N(0,1) [B,H]."""
    rng = _rng(seed)
    a = _uniform(rng, (B, L, H), alo, ahi)
    b = _normal(rng, (B, L, H))
    hz = _normal(rng, (B, H)) if h0 else np.zeros((B, H), np.float32)
    return {"a": a, "b": b, "h0": hz}


def linscan_blk2_inputs(B, L, H, seed, scale=0.6, h0=False):
    """2x2 block linear recurrence draws: A ~ U(-scale,scale) [B,L,H,2,2]
    (row-major a00,a01,a10,a11), b ~ N(0,1) [B,L,H,2]; optionally h0 ~ N(0,1) [B,H,2].
    With scale 0.6 every block has spectral norm below 1.2 and the products stay
    bounded in practice over long sequences."""
    rng = _rng(seed)
    A = _uniform(rng, (B, L, H, 2, 2), -scale, scale)
    b = _normal(rng, (B, L, H, 2))
    hz = _normal(rng, (B, H, 2)) if h0 else np.zeros((B, H, 2), np.float32)
    return {"A": A, "b": b, "h0": hz}


def linscan_blk_inputs(B, L, H, k, seed, h0=False):
    """k x k block linear recurrence draws: A ~ U(-s,s) [B,L,H,k,k] with
    s = 0.6*sqrt(2/k) (row-major), b ~ N(0,1) [B,L,H,k]; optionally h0 ~ N(0,1)
    [B,H,k].  With that s a random block shrinks a vector by about half per
    step on average, as the 2x2 draws do, so long products stay bounded."""
    rng = _rng(seed)
    s = 0.6 * np.sqrt(2.0 / k)
    A = _uniform(rng, (B, L, H, k, k), -s, s)
    b = _normal(rng, (B, L, H, k))
    hz = _normal(rng, (B, H, k)) if h0 else np.zeros((B, H, k), np.float32)
    return {"A": A, "b": b, "h0": hz}


def workload_inputs(name: str) -> dict:
    """Inputs of one named workload, seed 1000 + its index in WORKLOAD_ORDER
    (a workload with `same_as` takes that workload's inputs)."""
    w = WORKLOADS[name]
    if "same_as" in w:
        return workload_inputs(w["same_as"])
    seed = 1000 + WORKLOAD_ORDER.index(name)
    B, L, H = w["B"], w["L"], w["H"]
    if name == "c0_gru_tiny":
        return gru_inputs(B, L, H, seed)
    if name == "c1_linscan":
        return linscan_diag_inputs(B, L, H, seed)
    if name == "c2_gru_fused":
        return gru_inputs(B, L, H, seed, pscale=0.5)
    if name == "c3_lstm":
        return lstm_inputs(B, L, H, seed)
    if name == "c4_gru_long_fwd_adj":
        return gru_inputs(B, L, H, seed, grad=True)
    if name == "x_linscan_blk2":
        return linscan_blk2_inputs(B, L, H, seed)
    if name == "x_lstm_adjoint":
        return lstm_inputs(B, L, H, seed, grad=True)
    if name in ("x_linscan_blk4", "x_linscan_blk8"):
        return linscan_blk_inputs(B, L, H, w["k"], seed)
    if name == "x_hgru8_fwd":
        return head_gru_inputs(B, L, H, w["k"], seed)
    if name == "x_hgru8_bwd":
        return head_gru_inputs(B, L, H, w["k"], seed, grad=True)
    raise KeyError(name)
