#!/usr/bin/env python3
"""Benchmark of the Newton / parallel-scan RNN path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the path on one batch of synthetic inputs that already
reside in HBM.  The headline workload (default) is the diagonal linear
recurrence h_t = a_t h_{t-1} + b_t at B=16, L=4096, H=1024 (a ~ U(0.5,1),
b ~ N(0,1), h0 = 0): the parallel reduction that every Newton iteration
runs (ParaRNN page, Fig. 2 left), and for a linear recurrence the whole
solve.  The other workloads are measured in the same run and reported under
"workloads", each with its own roofline: the fully fused GRU Newton forward
at B=16, L=512, H=4096 (ParaRNN page, Fig. 2 right and Fig. 5 at L = 2^9),
the LSTM Newton forward at B=8, L=2048, H=2048 and the long-sequence GRU
forward plus adjoint at B=16, L=2^20, H=1 (the DEER summary's V100 shape),
then the 2x2 and 4x4 block scans, the LSTM adjoint, the per-iteration
Newton path, and sequential application (one thread per channel) of the
same cells on the same inputs, whose ratio to each Newton forward is
reported as speedup_vs_sequential.

Printed: one JSON line with the metric, the throughput (state elements per
second = B*L*H / wall time per step), the roofline of the dominant kernel
(its duration taken with HIP events on the stream it runs on) and the fp64
CPU oracle timed on this host as a baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Newton-solved state elements/sec (B·L·H) and achieved HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0

# Algorithmic bytes per state element (inputs read once, outputs written once).
ALG_BYTES = {
    "c1_linscan": 12,            # a, b in; h out
    "c2_gru_fused": 16,          # pz, pr, pc in; h out
    "c3_lstm": 24,               # pi, pf, po, pg in; h, c out
    "c4_gru_long_fwd_adj": 48,   # fwd: 3 p in, h out; adjoint: g, 3 p, h in, 3 dp out
    "x_linscan_blk2": 32,        # A (2x2) and b (2) in; h (2) out, per (batch, position, channel)
    "x_lstm_adjoint": 48,        # gh, gc, 4 p, h, c in; 4 dp out
    "x_lstm_step": 24,           # as c3_lstm: the whole solve's inputs once, outputs once
    "x_gru_long_step": 16,       # 3 p in; h out (the forward of c4 alone)
    "x_gru_long_fwd": 16,        # 3 p in; h out (the forward of c4 alone)
    "x_gru_seq": 16,             # 3 p in; h out
    "x_lstm_seq": 24,            # 4 p in; h, c out
    "x_gru_long_seq": 16,        # 3 p in; h out
    "x_linscan_blk4": 96,        # A (4x4) and b (4) in; h (4) out, per (batch, position, channel)
}
DOMINANT = {
    "c1_linscan": "diag_pf_kernel<16,16,2> (chunked scan, next tile prefetched)",
    "c2_gru_fused": "gru_fused_kernel<16>",
    "c3_lstm": "newton_local_kernel<LstmChain> (one launch for every iteration; each workgroup owns whole chains)",
    "c4_gru_long_fwd_adj": "newton_chain_kernel<GruChain> + chunk_scan_kernel<GruAdjOp> (whole step)",
    "x_linscan_blk2": "chunk_scan_kernel<LinBlk2Op>",
    "x_lstm_adjoint": "chunk_scan_kernel<LstmAdjOp> + reduce_u_kernel (whole step)",
    "x_lstm_step": "chunk_scan_kernel<LstmStepOp> (one launch per iteration up to the cap; "
                   "launches after convergence exit at once)",
    "x_gru_long_step": "chunk_scan_kernel<GruStepOp> (one launch per iteration up to the cap; "
                       "launches after convergence exit at once)",
    "x_gru_long_fwd": "newton_chain_kernel<GruChain> (time lanes, one launch for every iteration)",
    "x_gru_seq": "gru_rollout_kernel (sequential application, one thread per channel)",
    "x_lstm_seq": "lstm_rollout_kernel (sequential application, one thread per channel)",
    "x_gru_long_seq": "gru_rollout_kernel (sequential application, one thread per channel)",
    "x_linscan_blk4": "chunk_scan_kernel<LinBlkOp<4>>",
}
# HBM bytes per launch of the dominant kernel from rocprofv3 counter runs
# (FETCH_SIZE x 2.000 and WRITE_SIZE x 1.000, the factors a plain 1 GiB device
# copy gives for these counters), valid only for the kernel sources they were
# taken on: the sha256 prefix of those sources is checked at run time and the
# figure is dropped (null) once any of them has changed.
TRAFFIC = {
    "c1_linscan": {"bytes": 551421952 + 289021952,
                   "sources": ["common.hpp", "plan.hpp", "launch.hpp", "scan_core.hpp", "linscan.hip"],
                   "sha256": "3c1d79cf3f80249c"},
    "c2_gru_fused": {"bytes": 419277619 + 152519270,
                     "sources": ["common.hpp", "cells.hpp", "plan.hpp", "launch.hpp", "gru_fused.hip"],
                     "sha256": "17fe61c95e651689"},
}
DESCRIBE = {
    "c1_linscan": "linear diagonal recurrence h_t = a_t h_{t-1} + b_t, B=16 L=4096 H=1024, "
                  "a~U(0.5,1), b~N(0,1), h0=0",
    "c2_gru_fused": "diagonal GRU Newton forward, B=16 L=512 H=4096, p=0.5N(0,1), "
                    "u~U(-0.5,0.5), h0=0, tol 1e-4, cap 32 (fused on-chip kernel)",
    "c3_lstm": "diagonal LSTM Newton forward (2x2 block Jacobians), B=8 L=2048 H=2048, "
               "p~N(0,1), u~U(-0.5,0.5), h0=c0=0, tol 1e-4, cap 32",
    "c4_gru_long_fwd_adj": "diagonal GRU Newton forward + reverse adjoint, B=16 L=1048576 H=1, "
                           "p~N(0,1), u~U(-0.5,0.5), g~N(0,1), h0=0, tol 1e-4, cap 32",
    "x_linscan_blk2": "2x2 block linear recurrence h_t = A_t h_{t-1} + b_t, B=16 L=4096 H=512, "
                      "A~U(-0.6,0.6), b~N(0,1), h0=0",
    "x_lstm_adjoint": "diagonal LSTM reverse adjoint at the converged forward, B=8 L=2048 H=2048, "
                      "p~N(0,1), u~U(-0.5,0.5), gh, gc~N(0,1), h0=c0=0",
    "x_lstm_step": "the LSTM Newton forward of c3_lstm on the per-iteration path "
                   "(PARARNN_LSTM_PATH=step)",
    "x_gru_long_step": "the GRU Newton forward of c4_gru_long_fwd_adj on the per-iteration path "
                       "(PARARNN_GRU_PATH=step)",
    "x_gru_long_fwd": "the GRU Newton forward of c4_gru_long_fwd_adj alone (chained kernel)",
    "x_gru_seq": "sequential application of the GRU cell on the inputs of c2_gru_fused "
                 "(B*H = 65536 threads, 512 positions each)",
    "x_lstm_seq": "sequential application of the LSTM cell on the inputs of c3_lstm "
                  "(B*H = 16384 threads, 2048 positions each)",
    "x_gru_long_seq": "sequential application of the GRU cell on the inputs of c4_gru_long_fwd_adj "
                      "(B*H = 16 threads, 2^20 positions each)",
    "x_linscan_blk4": "4x4 block linear recurrence h_t = A_t h_{t-1} + b_t, B=16 L=2048 H=256, "
                      "A~U(-0.42,0.42), b~N(0,1), h0=0",
}


# Sequential-application workload on the same inputs as a Newton forward.
SEQUENTIAL_OF = {"c2_gru_fused": "x_gru_seq", "c3_lstm": "x_lstm_seq",
                 "x_lstm_step": "x_lstm_seq", "x_gru_long_step": "x_gru_long_seq",
                 "x_gru_long_fwd": "x_gru_long_seq"}


def measured_traffic(name):
    """Counter-derived HBM bytes per launch, or None if not taken on the
    current kernel sources."""
    import hashlib
    t = TRAFFIC.get(name)
    if t is None:
        return None
    m = hashlib.sha256()
    for f in t["sources"]:
        with open(os.path.join(ROOT, "nonlinear_rnn_solve_pararnn_amd", "csrc", f), "rb") as fh:
            m.update(fh.read())
    return t["bytes"] if m.hexdigest()[:16] == t["sha256"] else None


def roofline(name, elements, kernel_ms):
    """HBM roofline of the workload's dominant kernel: algorithmic bytes (inputs
    read once, outputs written once) over its event-timed duration."""
    alg = ALG_BYTES[name] * elements
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(name),
            "kernel": DOMINANT[name], "alg_bytes_per_launch": alg,
            "kernel_us": kernel_ms * 1e3}


# Arithmetic roofs of the Newton kernels that iterate on chip.  VALU issue
# slots per element and Newton iteration, from rocprofv3 counters of one
# dispatch (SQ_INSTS_VALU and SQ_INSTS_VALU_TRANS_F32 count wave instructions;
# times 64 lanes, over elements x iterations): plain instructions count one
# slot, transcendentals (exp2, reciprocal) four, since they issue at a
# quarter of the rate.  The fp32 vector peak of 157.3 TFLOP/s is 78.6 T
# lane-operations per second of FMA issue.
#  - fused GRU, B=16 L=512 H=4096, 4 iterations: 80,297,984 VALU and
#    12,615,680 transcendental wave instructions = 38.29 and 6.02 per element
#    and iteration (the gfx950 assembly of the loop gives 33.8 and 6; the rest
#    is per-iteration work outside the cell loop);
#  - LSTM whole chains, B=8 L=2048 H=2048, 4 iterations: 180,076,284 and
#    20,975,616 = 85.87 and 10.00.
ALU_SLOTS_PER_ELEMENT_ITER = {
    "c2_gru_fused": (38.29 - 6.02) + 6.02 * 4,
    "c3_lstm": (85.87 - 10.00) + 10.00 * 4,
}
PEAK_VALU_TOPS = 78.6


def alu_roofline(name, elements, iterations, kernel_ms):
    per = ALU_SLOTS_PER_ELEMENT_ITER[name]
    slots = per * elements * iterations
    achieved = slots / (kernel_ms * 1e-3) / 1e12
    return {"bound": "alu", "achieved": achieved, "peak": PEAK_VALU_TOPS,
            "unit": "T VALU issue slots/s", "frac": achieved / PEAK_VALU_TOPS,
            "model": "%.1f slots per element and Newton iteration (transcendentals count 4), "
                     "%d iterations (the most any tile took)" % (per, iterations)}


def _torch_gru_cell(h, pz, pr, pc, uz, ur, uc):
    import torch
    z = torch.sigmoid(pz + uz * h)
    r = torch.sigmoid(pr + ur * h)
    c = torch.tanh(pc + uc * (r * h))
    return (1 - z) * h + z * c


def modalities(dev, steps, warmup):
    """The GRU at B=16, L=512, H=4096 (the fused workload's inputs) through
    every way this library can evaluate it (ParaRNN page, Fig. 2 and Fig. 5:
    sequential application, tensor-op assembly with a dedicated reduction
    kernel, one fused pass per iteration, the fully fused solver), and the
    residual max|delta| per Newton iteration from a zero start at several
    sequence lengths (Fig. 4, on synthetic inputs)."""
    import torch

    from nonlinear_rnn_solve_pararnn_amd import api, generic, synth
    w = synth.WORKLOADS["c2_gru_fused"]
    host = synth.workload_inputs("c2_gru_fused")
    t = {k: torch.from_numpy(v).to(dev) for k, v in host.items()}
    p = [t["pz"], t["pr"], t["pc"]]
    u = [t["uz"], t["ur"], t["uc"]]
    tol, cap = w["tol"], w["cap"]

    def per_iteration():
        os.environ["PARARNN_GRU_PATH"] = "step"
        try:
            return api.gru_forward(*p, *u, tol=tol, max_iter=cap)
        finally:
            del os.environ["PARARNN_GRU_PATH"]

    ways = {
        "sequential application (one thread per channel)": lambda: api.gru_sequential(*p, *u),
        "torch assembly + HIP diagonal scan (generic.newton_solve)":
            lambda: generic.newton_solve(_torch_gru_cell, p, None, u, tol=tol, max_iter=cap),
        "one fused pass per Newton iteration (chunk_scan_kernel<GruStepOp>)": per_iteration,
        "fully fused Newton (gru_fused_kernel)": lambda: api.gru_forward(*p, *u, tol=tol, max_iter=cap),
    }
    ref = api.gru_sequential(*p, *u)
    out = {"workload": "GRU B=16 L=512 H=4096, pz, pr, pc = 0.5 N(0,1), u ~ U(-0.5,0.5), "
                       "h0 = 0, tol 1e-4, cap 32", "ms_per_call": {}, "max_abs_vs_sequential": {}}
    for name, fn in ways.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            h = fn()
        torch.cuda.synchronize()
        out["ms_per_call"][name] = (time.perf_counter() - t0) / steps * 1e3
        out["max_abs_vs_sequential"][name] = float((h - ref).abs().max())
    # residual per iteration from h = 0 at fixed B*H, tol = 0 (no early stop)
    traces = {}
    for L in (64, 512, 4096, 32768):
        d = synth.gru_inputs(8, L, 256, seed=700 + L)
        a = [torch.from_numpy(d[k]).to(dev) for k in ("pz", "pr", "pc", "uz", "ur", "uc")]
        tr = torch.zeros(12, device=dev)
        api.gru_forward(*a, tol=0.0, max_iter=12, trace=tr)
        traces["L=%d" % L] = [float(x) for x in tr.cpu()]
    out["residual_per_iteration"] = {"shape": "B=8 H=256, p ~ N(0,1), u ~ U(-0.5,0.5), h = 0 start, "
                                              "max|delta| of iterations 1..12", "traces": traces}
    return out


def device_copy(dev, reps=10):
    """Bandwidth of a plain 1 GiB device-to-device copy (torch copy_, read +
    write), timed with HIP events: a reference point for the HBM figures
    (kernels with streamed loads go past it)."""
    import torch
    n = 1 << 28
    a = torch.ones(n, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * 4 * n / (ms * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return {"value": gbs, "unit": "GB/s", "frac_of_peak": gbs / PEAK_HBM_GBS,
            "what": "torch copy_ of 1 GiB fp32 (1 GiB read + 1 GiB written), %d copies, HIP events" % reps}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Workload:
    """Inputs on the GPU plus a step() that runs the path once."""

    def __init__(self, name, dev):
        import torch

        from nonlinear_rnn_solve_pararnn_amd import api, synth
        self.name = name
        self.w = synth.WORKLOADS[name]
        self.host = synth.workload_inputs(name)
        self.dev = dev
        t = {k: torch.from_numpy(v).to(dev) for k, v in self.host.items()}
        self.t = t
        B, L, H = self.w["B"], self.w["L"], self.w["H"]
        self.B, self.L, self.H = B, L, H
        self.elements = B * L * H
        self.info = torch.zeros(2, dtype=torch.int32, device=dev)
        if name == "c1_linscan":
            self.out = torch.empty(B, L, H, device=dev)
            self.ws = api.new_workspace(api.workspace_bytes(api.OP_LINSCAN_DIAG, B, L, H), dev)
            self._step = lambda: api.linscan_diag(t["a"], t["b"], None, out=self.out, ws=self.ws)
        elif name == "x_linscan_blk2":
            self.out = torch.empty(B, L, H, 2, device=dev)
            self.ws = api.new_workspace(api.workspace_bytes(api.OP_LINSCAN_BLK2, B, L, H), dev)
            self._step = lambda: api.linscan_blk2(t["A"], t["b"], None, out=self.out, ws=self.ws)
        elif name == "x_linscan_blk4":
            self.out = torch.empty(B, L, H, 4, device=dev)
            self.ws = api.new_workspace(api.workspace_bytes(api.OP_LINSCAN_BLK4, B, L, H), dev)
            self._step = lambda: api.linscan_blk(t["A"], t["b"], None, out=self.out, ws=self.ws)
        elif name == "x_lstm_adjoint":
            p = [t[k] for k in ("pi", "pf", "po", "pg")]
            u = [t[k] for k in ("ui", "uf", "uo", "ug")]
            h, c = api.lstm_forward(*p, *u, None, None, tol=self.w["tol"], max_iter=self.w["cap"])
            self.out = h
            self.ws = api.new_workspace(api.workspace_bytes(api.OP_LSTM_ADJOINT, B, L, H), dev)
            self._step = lambda: api.adjoint_backward(api.CELL_LSTM, p, u, h, t["gh"], None, c=c,
                                                      grad_c=t["gc"], ws=self.ws)
        elif name == "c2_gru_fused":
            self.out = torch.empty(B, L, H, device=dev)
            cap = self.w["cap"]
            self.ws = api.new_workspace(api.workspace_bytes(api.OP_GRU_FORWARD, B, L, H, cap), dev)
            args = [t[k] for k in ("pz", "pr", "pc", "uz", "ur", "uc")]
            # no info/trace in the timed call: the step is exactly one kernel launch
            self._step = lambda: api.gru_forward(*args, None, tol=self.w["tol"], max_iter=cap,
                                                 out=self.out, ws=self.ws)
            self._probe = lambda: api.gru_forward(*args, None, tol=self.w["tol"], max_iter=cap,
                                                  out=self.out, ws=self.ws, info=self.info)
        elif name == "c3_lstm":
            self.out = torch.empty(B, L, H, device=dev)
            self.out_c = torch.empty(B, L, H, device=dev)
            cap = self.w["cap"]
            self.ws = api.new_workspace(api.workspace_bytes(api.OP_LSTM_FORWARD, B, L, H, cap), dev)
            args = [t[k] for k in ("pi", "pf", "po", "pg", "ui", "uf", "uo", "ug")]
            self._step = lambda: api.lstm_forward(*args, None, None, tol=self.w["tol"],
                                                  max_iter=cap, out_h=self.out, out_c=self.out_c,
                                                  info=self.info, ws=self.ws)
        elif name in ("x_lstm_step", "x_gru_long_step"):
            lstm = name == "x_lstm_step"
            cap = self.w["cap"]
            self.out = torch.empty(B, L, H, device=dev)
            self.out_c = torch.empty(B, L, H, device=dev) if lstm else None
            op = api.OP_LSTM_FORWARD if lstm else api.OP_GRU_FORWARD
            keys = ("pi", "pf", "po", "pg", "ui", "uf", "uo", "ug") if lstm else \
                ("pz", "pr", "pc", "uz", "ur", "uc")
            args = [t[k] for k in keys]
            var = "PARARNN_LSTM_PATH" if lstm else "PARARNN_GRU_PATH"
            # the workspace of the path the calls take (the query reads the override too)
            os.environ[var] = "step"
            try:
                self.ws = api.new_workspace(api.workspace_bytes(op, B, L, H, cap), dev)
            finally:
                del os.environ[var]

            def step():
                # the library reads the path override at each call
                os.environ[var] = "step"
                try:
                    if lstm:
                        return api.lstm_forward(*args, None, None, tol=self.w["tol"], max_iter=cap,
                                                out_h=self.out, out_c=self.out_c, info=self.info,
                                                ws=self.ws)
                    return api.gru_forward(*args, None, tol=self.w["tol"], max_iter=cap,
                                           out=self.out, info=self.info, ws=self.ws)
                finally:
                    del os.environ[var]
            self._step = step
        elif name == "x_gru_long_fwd":
            self.out = torch.empty(B, L, H, device=dev)
            cap = self.w["cap"]
            self.ws = api.new_workspace(api.workspace_bytes(api.OP_GRU_FORWARD, B, L, H, cap), dev)
            args = [t[k] for k in ("pz", "pr", "pc", "uz", "ur", "uc")]
            self._step = lambda: api.gru_forward(*args, None, tol=self.w["tol"], max_iter=cap,
                                                 out=self.out, info=self.info, ws=self.ws)
        elif name in ("x_gru_seq", "x_gru_long_seq"):
            self.out = torch.empty(B, L, H, device=dev)
            args = [t[k] for k in ("pz", "pr", "pc", "uz", "ur", "uc")]
            self._step = lambda: api.gru_sequential(*args, None, out=self.out)
        elif name == "x_lstm_seq":
            self.out = torch.empty(B, L, H, device=dev)
            self.out_c = torch.empty(B, L, H, device=dev)
            args = [t[k] for k in ("pi", "pf", "po", "pg", "ui", "uf", "uo", "ug")]
            self._step = lambda: api.lstm_sequential(*args, None, None, out_h=self.out,
                                                     out_c=self.out_c)
        elif name == "c4_gru_long_fwd_adj":
            self.out = torch.empty(B, L, H, device=dev)
            cap = self.w["cap"]
            self.ws = api.new_workspace(max(api.workspace_bytes(api.OP_GRU_FORWARD, B, L, H, cap),
                                            api.workspace_bytes(api.OP_GRU_ADJOINT, B, L, H)), dev)
            args = [t[k] for k in ("pz", "pr", "pc", "uz", "ur", "uc")]

            def step():
                h = api.gru_forward(*args, None, tol=self.w["tol"], max_iter=cap, out=self.out,
                                    info=self.info, ws=self.ws)
                return api.adjoint_backward(api.CELL_GRU, args[:3], args[3:], h, t["g"], None,
                                            ws=self.ws)
            self._step = step
        else:
            raise KeyError(name)

    def step(self):
        return self._step()

    def iterations(self):
        import torch
        if hasattr(self, "_probe"):
            self._probe()
        else:
            self._step()
        torch.cuda.synchronize()
        return [int(x) for x in self.info.cpu().tolist()]


def time_workload(wl, steps, warmup):
    """Returns (ms per step from the wall clock around K steps, ms per step
    from a HIP event pair around the same K steps on the launch stream)."""
    import torch
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        wl.step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, e0.elapsed_time(e1) / steps


def cpu_baseline(name, host):
    """The fp64 oracle's sequential rollout (the definition of the result) on
    this host, timed over the full workload or a bounded sample of it."""
    import numpy as np

    import oracle
    from nonlinear_rnn_solve_pararnn_amd import synth
    oracle.build(force=False)
    threads = oracle.num_threads()
    name = synth.WORKLOADS[name].get("same_as", name)
    if name in ("c2_gru_fused", "c4_gru_long_fwd_adj", "c0_gru_tiny"):
        args = [host[k].astype(np.float64) for k in ("pz", "pr", "pc", "uz", "ur", "uc")]
        fn = lambda: oracle.gru_rollout(*args)
        n = args[0].size
        what = "fp64 sequential GRU rollout (oracle.gru_rollout) over the full workload"
    elif name == "c3_lstm":
        args = [host[k].astype(np.float64) for k in ("pi", "pf", "po", "pg", "ui", "uf", "uo", "ug")]
        fn = lambda: oracle.lstm_rollout(*args)
        n = args[0].size
        what = "fp64 sequential LSTM rollout (oracle.lstm_rollout) over the full workload"
    elif name == "x_lstm_adjoint":
        keys = ("pi", "pf", "po", "pg", "ui", "uf", "uo", "ug")
        args = [host[k].astype(np.float64) for k in keys]
        h, c = oracle.lstm_rollout(*args)
        gh, gc = host["gh"].astype(np.float64), host["gc"].astype(np.float64)
        fn = lambda: oracle.lstm_bptt(*args, h, c, gh, gc)
        n = args[0].size
        what = "fp64 LSTM backpropagation through time (oracle.lstm_bptt) over the full workload"
    elif name == "x_linscan_blk2":
        args = [host["A"].astype(np.float64), host["b"].astype(np.float64)]
        fn = lambda: oracle.linscan_blk2(*args)
        n = args[1].size // 2
        what = "fp64 serial 2x2 block recurrence (oracle.linscan_blk2) over the full workload"
    else:
        args = [host["a"].astype(np.float64), host["b"].astype(np.float64)]
        fn = lambda: oracle.linscan_diag(*args)
        n = args[0].size
        what = "fp64 serial linear recurrence (oracle.linscan_diag) over the full workload"
    def timed(limit_s, max_reps):
        reps, t = 0, 0.0
        t0 = time.perf_counter()
        while t < limit_s and reps < max_reps:
            fn()
            reps += 1
            t = time.perf_counter() - t0
        return reps, t

    fn()  # page-in
    reps, t = timed(10.0, 400)
    out = {"value": n * reps / t, "unit": "elements/s", "cores": threads, "kind": "oracle",
           "sample": "%s, %d repetition(s), %.2f s" % (what, reps, t)}
    # the same on one core (channels are independent, so the threaded figure
    # is this one times the parallel efficiency)
    oracle.set_num_threads(1)
    try:
        reps1, t1 = timed(4.0, 400)
    finally:
        oracle.set_num_threads(threads)
    out["single_thread"] = {"value": n * reps1 / t1, "cores": 1,
                            "sample": "%d repetition(s), %.2f s" % (reps1, t1)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c1_linscan",
                    choices=list(ALG_BYTES))
    ap.add_argument("--only", action="store_true",
                    help="measure only the chosen workload (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--modalities", action="store_true",
                    help="only the modality comparison and residual traces (one JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(each GPU would run the same kernels on its own batch/channel shard); "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")

    if args.modalities:
        print(json.dumps(modalities(dev, args.steps, args.warmup)), flush=True)
        return

    if args.copy_calibration:
        n = 1 << 28  # 1 GiB of fp32
        a = torch.ones(n, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.warmup + args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: %d launches of a %d-byte device copy" % (args.warmup + args.steps, 4 * n))
        return

    names = [args.workload] if args.only else \
        [args.workload] + [n for n in ALG_BYTES if n != args.workload]
    results = {}
    for name in names:
        log("workload", name)
        wl = Workload(name, dev)
        iters = wl.iterations() if name in ("c2_gru_fused", "c3_lstm", "c4_gru_long_fwd_adj",
                                            "x_lstm_step", "x_gru_long_step",
                                            "x_gru_long_fwd") else None
        wall_ms, ev_ms = time_workload(wl, args.steps, args.warmup)
        results[name] = {
            "elements": wl.elements,
            "elements_per_s": wl.elements / (wall_ms * 1e-3),
            "ms_per_step": wall_ms,
            "event_ms_per_step": ev_ms,
            "newton_iterations": iters,
            "describe": DESCRIBE[name],
            "roofline": roofline(name, wl.elements, ev_ms),
        }
        if name in ALU_SLOTS_PER_ELEMENT_ITER and iters:
            results[name]["roofline_alu"] = alu_roofline(name, wl.elements, iters[0], ev_ms)
        log(json.dumps({name: results[name]}))
        del wl
        torch.cuda.empty_cache()

    # Newton forwards against sequential application of the same cell on the
    # same inputs (the comparison the pages quote their speedups for)
    for newton, seq in SEQUENTIAL_OF.items():
        if newton in results and seq in results:
            results[newton]["speedup_vs_sequential"] = (results[seq]["event_ms_per_step"] /
                                                        results[newton]["event_ms_per_step"])

    head = results[args.workload]
    from nonlinear_rnn_solve_pararnn_amd import synth
    w = synth.WORKLOADS[args.workload]
    out = {
        "metric": METRIC,
        "value": head["elements_per_s"],
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload + ": " + DESCRIBE[args.workload],
                   "B": w["B"], "L": w["L"], "H": w["H"], "parallelism": "single GPU"},
        "newton_iterations": head["newton_iterations"],
        "roofline": head["roofline"],
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(args.workload, synth.workload_inputs(args.workload))
    else:
        out["cpu_baseline"] = None
    if not args.only:
        out["device_copy"] = device_copy(dev)
    if len(results) > 1:
        out["workloads"] = {k: v for k, v in results.items() if k != args.workload}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
