"""Shared helpers of the GPU parity tests.

Tolerances (fp32 GPU vs fp64 oracle):
  FWD_ATOL  max abs error of forward states (h, c) and of the linear scans;
  GRAD_RTOL ||g_gpu - g_ref||_inf / ||g_ref||_inf per gradient tensor.
"""
import sys

import numpy as np
import torch

FWD_ATOL = 1e-4
GRAD_RTOL = 1e-3
ITER_ATOL = 1e-5   # single Newton iterates at the tiny workload

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    d = np.abs(a - b)
    if np.isnan(d).any():
        return float("inf")
    return float(d.max())


def rel_inf(g, r):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = max(float(np.abs(r).max()), 1e-30)
    d = np.abs(g - r)
    if np.isnan(d).any():
        return float("inf")
    return float(d.max()) / den


def gru_args(d):
    return [d[k] for k in ("pz", "pr", "pc", "uz", "ur", "uc")]


def lstm_args(d):
    return [d[k] for k in ("pi", "pf", "po", "pg", "ui", "uf", "uo", "ug")]
