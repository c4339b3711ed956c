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
    "x_linscan_blk4": 96,        # A (4x4) and b (4) in; h (4) out, per (batch, position, block)
    "x_linscan_blk8": 320,       # A (8x8) and b (8) in; h (8) out, per (batch, position, block)
    "x_hgru8_fwd": 128,          # pz, pr, pc (8 each) in; h (8) out, per (batch, position, head): the whole solve
    "x_hgru8_bwd": 256,          # pz, pr, pc, h, g (8 each) in; dpz, dpr, dpc (8 each) out, per (batch, position, head)
}
DOMINANT = {
    "c1_linscan": "scan_pf_kernel<LinDiagOp,16,16,2> (chunked scan, next tile prefetched)",
    "c2_gru_fused": "gru_fused_kernel<16>",
    "c3_lstm": "newton_local_kernel<LstmChain> (one launch for every iteration; each workgroup owns whole chains)",
    "c4_gru_long_fwd_adj": "newton_chain_kernel<GruChain> + chunk_scan_kernel<GruAdjOp> (whole step)",
    "x_linscan_blk2": "scan_pf_kernel<LinBlk2Op,8,12,1> (chunked scan, next tile prefetched)",
    "x_lstm_adjoint": "chunk_scan_kernel<LstmAdjOp> + reduce_u_kernel (whole step)",
    "x_lstm_step": "chunk_scan_kernel<LstmStepOp> (one launch per iteration up to the cap; "
                   "launches after convergence exit at once)",
    "x_gru_long_step": "chunk_scan_kernel<GruStepOp> (one launch per iteration up to the cap; "
                       "launches after convergence exit at once)",
    "x_gru_long_fwd": "newton_chain_kernel<GruChain> (time lanes, one launch for every iteration)",
    "x_gru_seq": "gru_rollout_kernel (sequential application, one thread per channel)",
    "x_lstm_seq": "lstm_rollout_kernel (sequential application, one thread per channel)",
    "x_gru_long_seq": "gru_rollout_kernel (sequential application, one thread per channel)",
    "x_linscan_blk4": "lg::scan_kernel<LinRowOp<4>,8,8,1> (each block's rows on a group of 4 lanes)",
    "x_linscan_blk8": "lg::scan_kernel<LinRowOp<8>,4,7,3> (each block's rows on a group of 8 lanes)",
    "x_hgru8_bwd": "lg::scan_kernel<HgruAdjOp<8>,4,8,1> + hgru_u_reduce_kernel (whole step: the reverse-time "
                   "scan of the transposed blocks with dL/dp, and the dL/dU reduction)",
    "x_hgru8_fwd": "lg::scan_kernel<HgruStepOp<8>,4,6,3> (one launch per Newton iteration up to the cap; "
                   "launches after convergence exit at once)",
}
# HBM bytes per launch of the dominant kernel from rocprofv3 counter runs
# (FETCH_SIZE x 2.000 and WRITE_SIZE x 1.000, the factors a plain 1 GiB device
# copy gives for these counters), valid only for the kernel sources they were
# taken on: the sha256 prefix of those sources is checked at run time and the
# figure is dropped (null) once any of them has changed.
TRAFFIC = {
    "c1_linscan": {"bytes": 551225435 + 289021984,
        "sources": ["common.hpp", "tags.hpp", "plan.hpp", "launch.hpp", "scan_core.hpp", "linscan.hip"],
        "sha256": "3eb66f7d7ef182f5"},
    "c2_gru_fused": {"bytes": 418677664 + 151870328,
        "sources": ["common.hpp", "tags.hpp", "cells.hpp", "plan.hpp", "launch.hpp", "gru_fused.hip"],
        "sha256": "21b6cb6480f857e0"},
    "c3_lstm": {"bytes": 537166576 + 268441296,
        "sources": ["common.hpp", "tags.hpp", "cells.hpp", "plan.hpp", "launch.hpp",
                    "scan_core.hpp", "newton_chain.hip"],
        "sha256": "284394b7d1def984"},
    "c4_gru_long_fwd_adj": {"bytes": 544031216 + 269397744,
        "sources": ["common.hpp", "tags.hpp", "cells.hpp", "plan.hpp", "launch.hpp", "scan_core.hpp",
                    "newton_chain.hip", "adjoint.hip"],
        "sha256": "79354152ed395f4d"},
    "x_linscan_blk2": {"bytes": 829594368 + 345952325,
        "sources": ["common.hpp", "tags.hpp", "plan.hpp", "launch.hpp", "scan_core.hpp", "linscan.hip"],
        "sha256": "3eb66f7d7ef182f5"},
    "x_linscan_blk4": {"bytes": 695824622 + 159006752,
        "sources": ["common.hpp", "tags.hpp", "plan.hpp", "launch.hpp", "lanegroup.hpp", "blkrow.hip"],
        "sha256": "5eb5a788fbd16856"},
    "x_linscan_blk8": {"bytes": 678415744 + 115343392,
        "sources": ["common.hpp", "tags.hpp", "plan.hpp", "launch.hpp", "lanegroup.hpp", "blkrow.hip"],
        "sha256": "5eb5a788fbd16856"},
    "x_lstm_adjoint": {"bytes": 1127551689 + 597172256,
        "sources": ["common.hpp", "tags.hpp", "cells.hpp", "plan.hpp", "launch.hpp",
                    "scan_core.hpp", "adjoint.hip"],
        "sha256": "7621327f970f43b0"},
    "x_gru_long_fwd": {"bytes": 204860880 + 67792476,
        "sources": ["common.hpp", "tags.hpp", "cells.hpp", "plan.hpp", "launch.hpp",
                    "scan_core.hpp", "newton_chain.hip"],
        "sha256": "284394b7d1def984"},
    "x_hgru8_bwd": {"bytes": 444734336 + 296485664,
        "sources": ["common.hpp", "tags.hpp", "plan.hpp", "launch.hpp", "lanegroup.hpp",
                    "newton_iter.hpp", "hgru.hip"],
        "sha256": "a543f5d6c4fc4522"},
    "x_gru_seq": {"bytes": 402868864 + 134217728,
        "sources": ["common.hpp", "tags.hpp", "cells.hpp", "plan.hpp", "launch.hpp", "rollout.hip"],
        "sha256": "f3430fb8a98878ef"},
    "x_lstm_seq": {"bytes": 537126857 + 268435456,
        "sources": ["common.hpp", "tags.hpp", "cells.hpp", "plan.hpp", "launch.hpp", "rollout.hip"],
        "sha256": "f3430fb8a98878ef"},
    # per step: the launches of the iterations that ran (the launches after
    # convergence read and write almost nothing)
    "x_hgru8_fwd": {"bytes": 1417230800 + 504173056,
        "sources": ["common.hpp", "tags.hpp", "plan.hpp", "launch.hpp", "lanegroup.hpp",
                    "newton_iter.hpp", "hgru.hip"],
        "sha256": "a543f5d6c4fc4522"},
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
    "x_linscan_blk8": "8x8 block linear recurrence h_t = A_t h_{t-1} + b_t (heads of 8 channels), "
                      "B=16 L=2048 H=64 heads, A~U(-0.3,0.3), b~N(0,1), h0=0",
    "x_hgru8_bwd": "gradients of the GRU with dense recurrence inside heads of 8 channels (the adjoint: "
                   "reverse-time scan of the transposed 8x8 blocks, dL/dp, dL/dU, dL/dh0) at the converged "
                   "forward of x_hgru8_fwd's inputs, B=16 L=2048 H=64 heads, upstream g~N(0,1)",
    "x_hgru8_fwd": "Newton forward of the GRU with dense recurrence inside heads of 8 channels (8x8 "
                   "Jacobian blocks), B=16 L=2048 H=64 heads, p~N(0,1), U: diagonal U(-0.5,0.5), "
                   "off-diagonal U(-0.3,0.3)/sqrt(8), h0=0, tol 1e-4, cap 32",
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


# Arithmetic roofs of the Newton kernels that iterate on chip, from rocprofv3
# counters of one dispatch, times 64 lanes, over elements x iterations.
#
# Primary basis (published peak): SQ_INSTS_VALU and SQ_INSTS_VALU_TRANS_F32
# count wave instructions; plain instructions count one slot and
# transcendentals (exp2, reciprocal) four, against the fp32 vector peak of
# 157.3 TFLOP/s = 78.6 T lane-operations per second.  The measured
# multiply-add rate of this build is reported beside it (alu_calibration).
#  - fused GRU, B=16 L=512 H=4096, 4 iterations: 36.34 VALU and 6.02
#    transcendental wave instructions per element and iteration (the gfx950
#    assembly of the loop gives 31.8 and 6; the rest is per-iteration work
#    outside the cell loop);
#  - LSTM whole chains, B=8 L=2048 H=2048, 4 iterations: 74.89 and 10.00;
#  - long GRU forward (chained, time lanes), B=16 L=2^20 H=1, 3 iterations:
#    41.42 and 6.08;
#  - GRU with 8x8 heads, B=16 L=2048 NH=64, per launch of one iteration:
#    327.70 and 6.07.
ALU_SLOTS_PER_ELEMENT_ITER = {
    "c2_gru_fused": (36.34 - 6.02) + 6.02 * 4,
    "c3_lstm": (74.89 - 10.00) + 10.00 * 4,
    "x_gru_long_fwd": (41.42 - 6.08) + 6.08 * 4,
    "x_hgru8_fwd": (327.70 - 6.07) + 6.07 * 4,
}
PEAK_VALU_TOPS = 78.6
# Issue basis: SQ_ACTIVE_INST_VALU counts the quad-cycles a SIMD spends
# issuing a wave's VALU instructions (one per plain instruction, two per
# transcendental, as the probes' own counters show).  A SIMD issues one such
# quad-cycle at a time unless two waves' plain instructions pair up, which
# the probes show happens for pure multiply-add streams (2 per quad-cycle: the
# 66.9 T rate) but hardly at all once transcendentals are mixed in (under 4%
# of quad-cycles in a probe of 8 transcendentals and 4-36 multiply-adds per
# step; 16% in the fused GRU, 7% in the LSTM).  The roof is then the
# single-issue rate, measured live with one wave per SIMD (alu_calibration,
# "fma_1wave"), against the issue quad-cycles per element and iteration:
ALU_ISSUE_PER_ELEMENT_ITER = {
    "c2_gru_fused": 42.35,
    "c3_lstm": 84.89,
    "x_gru_long_fwd": 47.50,
    "x_hgru8_fwd": 333.76,
}


def alu_roofline(name, elements, iterations, kernel_ms, calib=None):
    """Arithmetic roof: issue slots over the kernel time, against the
    published fp32 vector peak (the primary basis) and, when `calib` is given,
    against the measured multiply-add rate of this build (two waves per SIMD
    pairing their instructions) and the issue quad-cycles against the
    measured single-issue rate (one wave per SIMD)."""
    per = ALU_SLOTS_PER_ELEMENT_ITER[name]
    slots = per * elements * iterations
    achieved = slots / (kernel_ms * 1e-3) / 1e12
    out = {"bound": "alu", "achieved": achieved, "peak": PEAK_VALU_TOPS,
           "unit": "T VALU issue slots/s", "frac": achieved / PEAK_VALU_TOPS,
           "model": "%.1f slots per element and Newton iteration (transcendentals count 4), "
                    "%d iterations (the most any tile took)" % (per, iterations)}
    if calib is not None:
        fma = calib["fma"]["lane_ops_per_s"] / 1e12
        out["peak_measured_fma"] = fma
        out["frac_measured_fma"] = achieved / fma
        if "fma_1wave" in calib:
            one = calib["fma_1wave"]["lane_ops_per_s"] / 1e12
            issue = ALU_ISSUE_PER_ELEMENT_ITER[name] * elements * iterations / (kernel_ms * 1e-3) / 1e12
            out["issue"] = {"achieved": issue, "peak_single_issue": one, "frac": issue / one,
                            "model": "%.2f VALU issue quad-cycles x 64 lanes per element and Newton "
                                     "iteration (SQ_ACTIVE_INST_VALU)" % ALU_ISSUE_PER_ELEMENT_ITER[name]}
    return out


def _torch_gru_cell(h, pz, pr, pc, uz, ur, uc):
    import torch
    z = torch.sigmoid(pz + uz * h)
    r = torch.sigmoid(pr + ur * h)
    c = torch.tanh(pc + uc * (r * h))
    return (1 - z) * h + z * c


def _torch_lstm_cell(s, pi, pf, po, pg, ui, uf, uo, ug):
    import torch
    cp, hp = s[..., 0], s[..., 1]
    i = torch.sigmoid(pi + ui * hp)
    f = torch.sigmoid(pf + uf * hp)
    o = torch.sigmoid(po + uo * hp)
    g = torch.tanh(pg + ug * hp)
    c = f * cp + i * g
    return torch.stack([c, o * torch.tanh(c)], dim=-1)


class _env:
    """Set (or, with None, remove) an environment variable for a block and
    restore what was there before."""

    def __init__(self, name, value):
        self.name, self.value = name, value

    def __enter__(self):
        self.old = os.environ.get(self.name)
        if self.value is None:
            os.environ.pop(self.name, None)
        else:
            os.environ[self.name] = self.value

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop(self.name, None)
        else:
            os.environ[self.name] = self.old


def _event_median_ms(fn, reps, warmup=1):
    """Median over `reps` calls of fn, each between its own HIP event pair on
    the current stream (the stream the library launches on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    pairs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in pairs)
    return t[len(t) // 2]


# Sequence lengths and shape of the modality sweep (ParaRNN page, Fig. 5:
# time against L for ParaGRU and ParaLSTM, each way of evaluating them).
SWEEP_L = (512, 2048, 8192, 32768)
SWEEP_B, SWEEP_H = 16, 256


def modalities(dev, reps=3):
    """The ParaRNN page's Fig. 5 and Fig. 4 on synthetic inputs.

    Fig. 5: the GRU and the LSTM at B=16, H=256 and L = 2^9 ... 2^15 through
    every way this library evaluates them: sequential application (one
    thread per channel), tensor-op assembly with the library's scan as the
    reduction kernel (generic.newton_solve), one fused pass per Newton
    iteration, and the fully fused solver (one launch for the whole solve:
    the fused GRU kernel up to L = 512, the chained kernel beyond, and the
    chained kernel for every LSTM).  Inputs: torch's seeded generator on the
    device, p ~ N(0,1), u ~ U(-0.5, 0.5), zero initial state, tol 1e-4, cap
    32.  Times are medians of HIP-event pairs around each call.

    Fig. 4: max|delta| per Newton iteration from a zero start (tol = 0, no
    early stop) for both cells at B=8, H=256 and several L."""
    import torch

    from nonlinear_rnn_solve_pararnn_amd import api, generic
    tol, cap = 1e-4, 32
    out = {"shape": "B=%d H=%d, p ~ N(0,1), u ~ U(-0.5,0.5), zero initial state, tol %g, cap %d"
                    % (SWEEP_B, SWEEP_H, tol, cap),
           "timing": "median of %d HIP-event pairs per call (after one warm-up call)" % reps,
           "ms_per_call": {"gru": {}, "lstm": {}}, "speedup_fused_vs_sequential": {"gru": {}, "lstm": {}},
           "max_abs_vs_sequential": {"gru": {}, "lstm": {}}}
    for cell in ("gru", "lstm"):
        ng = 3 if cell == "gru" else 4
        var = "PARARNN_GRU_PATH" if cell == "gru" else "PARARNN_LSTM_PATH"
        for L in SWEEP_L:
            gen = torch.Generator(device=dev)
            gen.manual_seed(7000 + L + (0 if cell == "gru" else 1))
            p = [torch.randn(SWEEP_B, L, SWEEP_H, device=dev, generator=gen) for _ in range(ng)]
            u = [torch.rand(SWEEP_H, device=dev, generator=gen) - 0.5 for _ in range(ng)]
            if cell == "gru":
                h_out = torch.empty_like(p[0])
                seq = lambda: api.gru_sequential(*p, *u, out=h_out)  # noqa: E731
                torch_asm = lambda: generic.newton_solve(_torch_gru_cell, p, None, u, tol=tol,  # noqa: E731
                                                         max_iter=cap)
                newton = lambda: api.gru_forward(*p, *u, tol=tol, max_iter=cap, out=h_out)  # noqa: E731
                fused_path = "fused" if L <= 512 else None
                pick = lambda r: r  # noqa: E731
            else:
                h_out, c_out = torch.empty_like(p[0]), torch.empty_like(p[0])
                seq = lambda: api.lstm_sequential(*p, *u, out_h=h_out, out_c=c_out)  # noqa: E731
                torch_asm = lambda: generic.newton_solve(_torch_lstm_cell, p, None, u, tol=tol,  # noqa: E731
                                                         max_iter=cap, state_size=2)
                newton = lambda: api.lstm_forward(*p, *u, tol=tol, max_iter=cap,  # noqa: E731
                                                  out_h=h_out, out_c=c_out)
                fused_path = None
                pick = lambda r: r[0] if isinstance(r, tuple) else r[..., 1]  # noqa: E731
            ways = {"sequential": (seq, None),
                    "torch_assembly_hip_scan": (torch_asm, None),
                    "per_iteration_pass": (newton, "step"),
                    "fully_fused": (newton, fused_path)}
            ref = pick(seq()).clone()
            row, err = {}, {}
            for name, (fn, path) in ways.items():
                with _env(var, path):
                    row[name] = _event_median_ms(fn, reps)
                    err[name] = float((pick(fn()) - ref).abs().max())
            key = "L=%d" % L
            out["ms_per_call"][cell][key] = row
            out["max_abs_vs_sequential"][cell][key] = err
            out["speedup_fused_vs_sequential"][cell][key] = row["sequential"] / row["fully_fused"]
            log("modalities", cell, key, json.dumps(row))
            del p, u
            torch.cuda.empty_cache()
    # residual per iteration from a zero start, tol = 0 (no early stop)
    traces = {"gru": {}, "lstm": {}}
    for L in (64, 512, 4096, 32768):
        gen = torch.Generator(device=dev)
        gen.manual_seed(700 + L)
        for cell, ng in (("gru", 3), ("lstm", 4)):
            p = [torch.randn(8, L, 256, device=dev, generator=gen) for _ in range(ng)]
            u = [torch.rand(256, device=dev, generator=gen) - 0.5 for _ in range(ng)]
            tr = torch.zeros(12, device=dev)
            if cell == "gru":
                api.gru_forward(*p, *u, tol=0.0, max_iter=12, trace=tr)
            else:
                api.lstm_forward(*p, *u, tol=0.0, max_iter=12, trace=tr)
            traces[cell]["L=%d" % L] = [float(x) for x in tr.cpu()]
    out["residual_per_iteration"] = {"shape": "B=8 H=256, p ~ N(0,1), u ~ U(-0.5,0.5), zero start, "
                                              "max|delta| of iterations 1..12 (tol = 0)",
                                     "traces": traces}
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


def alu_calibration(dev):
    """Measured issue rates of plain fp32 multiply-adds and of exp2/reciprocal
    pairs (nonlinear_rnn_solve_pararnn_amd/probe/alu_probe.hip, compiled with
    the library's flags, packed fp32 off): lane operations per second over one
    launch of 8 independent register chains per thread, HIP events on the
    launch stream.  The basis next to the published fp32 vector peak for the
    arithmetic rooflines."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "nonlinear_rnn_solve_pararnn_amd", "libpararnn_probe.so"))
    for f in (lib.alu_probe_fma, lib.alu_probe_trans):
        f.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        f.restype = ctypes.c_int
    tpb, steps = lib.alu_probe_threads_per_block(), lib.alu_probe_steps_per_iter()
    blocks = 256 * 32  # 32 workgroups of 4 waves per CU: every SIMD busy
    out = torch.empty(blocks * tpb, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {}
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    # one workgroup of 4 waves per CU: one wave per SIMD, no pairing
    for name, fn, iters, nb in (("fma", lib.alu_probe_fma, 2048, blocks),
                                ("exp2_rcp", lib.alu_probe_trans, 256, blocks),
                                ("fma_1wave", lib.alu_probe_fma, 8192, ncu)):
        ops = nb * tpb * iters * steps * (2 if name == "exp2_rcp" else 1)
        for _ in range(2):
            assert fn(nb, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream)) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        assert fn(nb, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream)) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        res[name] = {"lane_ops_per_s": ops / (ms * 1e-3), "ms": ms, "lane_ops": ops}
    res["what"] = ("alu_probe.hip: v_fma (fmamk) chains, and exp2 + add + reciprocal chains "
                   "(2 transcendental lane-ops per step), %d workgroups of %d threads; fma_1wave: the "
                   "fma chains with one workgroup per CU (one wave per SIMD)" % (blocks, tpb))
    return res


def compose_probe(dev):
    """Dense 8x8 map compositions per second, vector lane groups (the block
    scans' row_then) against the matrix cores (v_mfma_f32_16x16x4_f32 on
    block-diagonal pairs of maps, an upper bound: no operand permutes, no b
    part), alu_probe.hip, HIP events on the launch stream."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "nonlinear_rnn_solve_pararnn_amd", "libpararnn_probe.so"))
    for f in (lib.alu_probe_lg8_compose, lib.alu_probe_mfma):
        f.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        f.restype = ctypes.c_int
    tpb = lib.alu_probe_threads_per_block()
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = ncu * 8  # eight workgroups of 4 waves per CU: 8 waves per SIMD
    out = torch.empty(blocks * tpb, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn, iters):
        for _ in range(2):
            assert fn(blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream)) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        assert fn(blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream)) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    it_v, it_m = 512, 2048
    tv = timed(lib.alu_probe_lg8_compose, it_v)
    vec = blocks * (tpb // 8) * it_v * lib.alu_probe_lg8_compose_per_group_iter() / tv
    tm = timed(lib.alu_probe_mfma, it_m)
    instr = blocks * (tpb // 64) * it_m * lib.alu_probe_mfma_per_wave_iter() / tm
    return {"vector_compositions_per_s": vec, "vector_ms": tv * 1e3,
            "mfma_instructions_per_s": instr, "mfma_tflops": instr * 2048 / 1e12, "mfma_ms": tm * 1e3,
            "mfma_compositions_per_s_bound": instr / 2, "vector_over_mfma_bound": vec / (instr / 2),
            "what": "8x8 affine maps; vector: lane groups of 8 with DPP multiply-adds, 4 chains per group; "
                    "mfma: 16x16x4 fp32, 4 instructions per 16x16x16 product = 2 compositions of A only; "
                    "%d workgroups of %d threads" % (blocks, tpb)}


def issue_probe(dev):
    """How a SIMD shares its issue between waves (alu_probe.hip): the
    multiply-add chains at 1, 2, 4 and 8 waves per SIMD (1, 2, 4, 8
    workgroups of 4 waves per CU), and the mix probe (4 exp2/add/reciprocal
    chains plus m multiply-adds per step) at 8 waves per SIMD.  Rates in lane
    operations per second; HIP events on the launch stream."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "nonlinear_rnn_solve_pararnn_amd", "libpararnn_probe.so"))
    lib.alu_probe_fma.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.alu_probe_mix.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    tpb, steps = lib.alu_probe_threads_per_block(), lib.alu_probe_steps_per_iter()
    msteps = lib.alu_probe_mix_steps_per_iter()
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(ncu * 8 * tpb, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(launch):
        for _ in range(2):
            assert launch() == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        assert launch() == 0
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    rows = []
    for wps in (1, 2, 4, 8):
        nb, iters = ncu * wps, 16384 // wps  # about 2 ms a launch
        sec = timed(lambda: lib.alu_probe_fma(nb, iters, ctypes.c_void_p(out.data_ptr()), sp))
        rows.append({"probe": "fma", "waves_per_simd": wps, "ms": sec * 1e3,
                     "fma_lane_ops_per_s": nb * tpb * iters * steps / sec})
    for m in (0, 4, 8, 16, 32):
        nb, iters = ncu * 8, 512
        sec = timed(lambda: lib.alu_probe_mix(nb, iters, m, ctypes.c_void_p(out.data_ptr()), sp))
        n = nb * tpb * iters * msteps  # lane-steps
        rows.append({"probe": "mix", "fma_per_step": m, "waves_per_simd": 8, "ms": sec * 1e3,
                     "trans_lane_ops_per_s": n * 8 / sec, "plain_lane_ops_per_s": n * (m + 4) / sec,
                     "ns_per_step_per_simd_lane": sec / n * 1e9 * ncu * 4 * 64})
    return rows


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
        elif name in ("x_linscan_blk4", "x_linscan_blk8"):
            k = self.w["k"]
            self.out = torch.empty(B, L, H, k, device=dev)
            op = api.OP_LINSCAN_BLK4 if k == 4 else api.OP_LINSCAN_BLK8
            self.ws = api.new_workspace(api.workspace_bytes(op, B, L, H), dev)
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
        elif name == "x_hgru8_bwd":
            k = self.w["k"]
            args = [t[x] for x in ("pz", "pr", "pc", "Uz", "Ur", "Uc")]
            h = api.hgru_forward(*args, None, tol=self.w["tol"], max_iter=self.w["cap"])
            self.out = (torch.empty(B, L, H, k, device=dev), torch.empty(B, L, H, k, device=dev),
                        torch.empty(B, L, H, k, device=dev), torch.empty(H, k, k, device=dev),
                        torch.empty(H, k, k, device=dev), torch.empty(H, k, k, device=dev), None)
            self.ws = api.new_workspace(api.workspace_bytes(api.OP_HGRU8_BACKWARD, B, L, H), dev)
            self._step = lambda: api.hgru_backward(*args, None, h, t["g"], want_h0=False, ws=self.ws,
                                                   out=self.out)
        elif name == "x_hgru8_fwd":
            cap = self.w["cap"]
            self.out = torch.empty(B, L, H, self.w["k"], device=dev)
            self.ws = api.new_workspace(api.workspace_bytes(api.OP_HGRU8_FORWARD, B, L, H, cap), dev)
            args = [t[k] for k in ("pz", "pr", "pc", "Uz", "Ur", "Uc")]
            self._step = lambda: api.hgru_forward(*args, None, tol=self.w["tol"], max_iter=cap,
                                                  out=self.out, info=self.info, ws=self.ws)
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


# Bytes read between timed reps to evict the MI355X's 256 MB last-level
# cache (MALL), so that no rep reads inputs the previous one left in it.  A
# read, not a write: a 512 MB write leaves the cache full of dirty lines
# whose write-back then competes with the timed step (the diagonal scan
# measured 153 us after a write against 130 us back to back).
EVICT_BYTES = 512 << 20


def time_workload(wl, steps, warmup, scratch):
    """Times K steps twice.

    back to back: K steps bracketed by a device synchronisation on both
      sides, timed by the wall clock and by one HIP event pair on the launch
      stream (the contract's ms per step and value come from the wall clock);
    cold: before each of K steps a 512 MB scratch read (the reduction of a
      buffer written once beforehand), then the step between its own HIP
      event pair on the launch stream; the median is the kernel duration the
      roofline uses."""
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
    warm = e0.elapsed_time(e1) / steps
    pairs = []
    for _ in range(steps):
        scratch.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        wl.step()
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    cold = sorted(a.elapsed_time(b) for a, b in pairs)
    return {"wall_ms": wall, "warm_event_ms": warm, "cold_median_ms": cold[len(cold) // 2],
            "cold_min_ms": cold[0], "cold_max_ms": cold[-1]}


def cpu_baseline(name, host, budget_s=10.0, single_s=4.0):
    """The fp64 oracle's sequential rollout (the definition of the result) on
    this host, timed over repetitions of the full workload for about
    `budget_s` seconds on every core the oracle uses and `single_s` on one."""
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
    reps, t = timed(budget_s, 400)
    out = {"value": n * reps / t, "unit": "elements/s", "cores": threads, "kind": "oracle",
           "sample": "%s, %d repetition(s), %.2f s" % (what, reps, t)}
    # the same on one core (channels are independent, so the threaded figure
    # is this one times the parallel efficiency)
    oracle.set_num_threads(1)
    try:
        reps1, t1 = timed(single_s, 400)
    finally:
        oracle.set_num_threads(threads)
    out["single_thread"] = {"value": n * reps1 / t1, "cores": 1,
                            "sample": "%d repetition(s), %.2f s" % (reps1, t1)}
    return out


# Newton workloads whose entry also carries the oracle timed on this host
# (a bounded sample: repetitions of the full workload for a few seconds).
CPU_BASELINE_OF = ("c2_gru_fused", "c3_lstm", "c4_gru_long_fwd_adj")


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
    ap.add_argument("--no-modalities", action="store_true",
                    help="leave out the modality sweep and residual traces")
    ap.add_argument("--modalities", action="store_true",
                    help="only the modality sweep and residual traces (one JSON line)")
    ap.add_argument("--compose-probe", action="store_true",
                    help="print 8x8 map compositions per second, vector lane groups against the matrix cores")
    ap.add_argument("--issue-probe", action="store_true",
                    help="print the issue-sharing probe table (alu_probe.hip) and exit")
    ap.add_argument("--alu-calibration", action="store_true",
                    help="print the measured fp32 multiply-add and exp2/reciprocal issue rates")
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
        print(json.dumps(modalities(dev)), flush=True)
        return

    if args.compose_probe:
        print(json.dumps(compose_probe(dev)))
        return
    if args.issue_probe:
        for row in issue_probe(dev):
            print(json.dumps(row), flush=True)
        return
    if args.alu_calibration:
        print(json.dumps(alu_calibration(dev)), flush=True)
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

    calib = alu_calibration(dev)
    log("alu calibration", json.dumps(calib))
    scratch = torch.zeros(EVICT_BYTES // 4, dtype=torch.float32, device=dev)
    names = [args.workload] if args.only else \
        [args.workload] + [n for n in ALG_BYTES if n != args.workload]
    results = {}
    for name in names:
        log("workload", name)
        wl = Workload(name, dev)
        iters = wl.iterations() if name in ("c2_gru_fused", "c3_lstm", "c4_gru_long_fwd_adj",
                                            "x_lstm_step", "x_gru_long_step",
                                            "x_gru_long_fwd", "x_hgru8_fwd") else None
        t = time_workload(wl, args.steps, args.warmup, scratch)
        kernel_ms = t["cold_median_ms"]
        results[name] = {
            "elements": wl.elements,
            "elements_per_s": wl.elements / (t["wall_ms"] * 1e-3),
            "ms_per_step": t["wall_ms"],
            "event_ms_per_step": kernel_ms,
            "timing": t,
            "newton_iterations": iters,
            "describe": DESCRIBE[name],
            "roofline": roofline(name, wl.elements, kernel_ms),
        }
        if name in ALU_SLOTS_PER_ELEMENT_ITER and iters:
            # the slot counts are per state element: k of them per head position for the head GRU
            n_state = wl.elements * (wl.w["k"] if wl.w.get("kind") == "hgru" else 1)
            results[name]["roofline_alu"] = alu_roofline(name, n_state, iters[0], kernel_ms, calib)
        if name != args.workload and name in CPU_BASELINE_OF and not args.no_cpu_baseline:
            log("cpu baseline (oracle) for", name)
            results[name]["cpu_baseline"] = cpu_baseline(name, wl.host, budget_s=5.0, single_s=2.0)
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
        "timing": head["timing"],
    }
    if args.workload == "c1_linscan":
        out["config"]["note"] = ("a linear recurrence is its own Newton linearisation: one Newton step "
                                 "(this bi-diagonal solve) is exact; the nonlinear Newton forwards are "
                                 "under workloads (c2_gru_fused, c3_lstm, c4_gru_long_fwd_adj)")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(args.workload, synth.workload_inputs(args.workload))
    else:
        out["cpu_baseline"] = None
    out["alu_calibration"] = calib
    if not args.only:
        out["device_copy"] = device_copy(dev)
    if len(results) > 1:
        out["workloads"] = {k: v for k, v in results.items() if k != args.workload}
    del scratch
    torch.cuda.empty_cache()
    if not args.only and not args.no_modalities:
        log("modalities and residual traces ...")
        out["modalities"] = modalities(dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
