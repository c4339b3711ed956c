"""The C ABI under HIP graph capture: every entry point only enqueues kernels
(no memset, no allocation, no host synchronisation), so a captured sequence
of calls replays correctly.  Each replay is checked against the oracle, with
the inputs changed in place between replays and eager calls in between."""
import pytest
import torch

from nonlinear_rnn_solve_pararnn_amd import api, synth
from tests.gpu_helpers import FWD_ATOL, GRAD_RTOL, dev, gru_args, host, max_abs, rel_inf, say

pytestmark = pytest.mark.gpu


def test_captured_scan_newton_and_adjoint_replay(orc):
    B, L, H = 2, 3000, 70  # chained GRU kernel (L > 512), several scan chunks
    ds = [synth.gru_inputs(B, L, H, seed=600 + r, h0=True, grad=True) for r in range(3)]
    dl = [synth.linscan_diag_inputs(B, L, H, seed=610 + r) for r in range(3)]
    keys = ("pz", "pr", "pc", "uz", "ur", "uc", "h0", "g")
    t = {k: dev(ds[0][k]) for k in keys}
    a, b = dev(dl[0]["a"]), dev(dl[0]["b"])
    # outputs and workspaces allocated before capture; one workspace per entry
    # point here (a shared one would also do: calls are ordered on the stream)
    hs = torch.empty(B, L, H, device="cuda")
    hg = torch.empty(B, L, H, device="cuda")
    info = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws_s = api.new_workspace(api.workspace_bytes(api.OP_LINSCAN_DIAG, B, L, H), a.device)
    ws_f = api.new_workspace(api.workspace_bytes(api.OP_GRU_FORWARD, B, L, H, 16), a.device)
    ws_a = api.new_workspace(api.workspace_bytes(api.OP_GRU_ADJOINT, B, L, H), a.device)
    p, u = [t["pz"], t["pr"], t["pc"]], [t["uz"], t["ur"], t["uc"]]
    grads = {}

    def calls():
        api.linscan_diag(a, b, out=hs, ws=ws_s)
        api.gru_forward(*p, *u, t["h0"], tol=1e-5, max_iter=16, out=hg, info=info, ws=ws_f)
        grads.update(api.adjoint_backward(api.CELL_GRU, p, u, hg, t["g"], t["h0"], ws=ws_a))

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()  # warm-up on the capture stream (workspaces, kernel loading)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for r in range(3):
        say("replay", r)
        for k in keys:
            t[k].copy_(dev(ds[r][k]))
        a.copy_(dev(dl[r]["a"]))
        b.copy_(dev(dl[r]["b"]))
        api.linscan_diag(b, a)  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert max_abs(host(hs), orc.linscan_diag(dl[r]["a"], dl[r]["b"])) <= FWD_ATOL
        href = orc.gru_rollout(*gru_args(ds[r]), h0=ds[r]["h0"])
        assert info.cpu().tolist()[1] == 1
        assert max_abs(host(hg), href) <= FWD_ATOL
        dp, du, dh0 = orc.gru_bptt(*gru_args(ds[r]), href, ds[r]["g"], h0=ds[r]["h0"])
        errs = [rel_inf(host(grads["p"][q]), dp[q]) for q in range(3)]
        errs += [rel_inf(host(grads["u"][q]), du[q]) for q in range(3)]
        errs.append(rel_inf(host(grads["h0"]), dh0))
        say(max(errs))
        assert max(errs) <= GRAD_RTOL


def test_captured_block_scans_and_warm_start_replay(orc):
    """The 8x8 and 4x4 lane-group scans and a warm-started chained LSTM forward
    under capture: three replays with the inputs changed in place, eager work
    in between, every replay against the oracle."""
    from tests.gpu_helpers import lstm_args
    import numpy as np
    B, L, H = 2, 700, 24
    d8 = [synth.linscan_blk_inputs(B, L, H, 8, seed=660 + r) for r in range(3)]
    d4 = [synth.linscan_blk_inputs(B, L, H, 4, seed=670 + r) for r in range(3)]
    dl = [synth.lstm_inputs(B, 1500, 40, seed=680 + r, h0=True) for r in range(3)]
    A8, b8 = dev(d8[0]["A"]), dev(d8[0]["b"])
    A4, b4 = dev(d4[0]["A"]), dev(d4[0]["b"])
    lk = ("pi", "pf", "po", "pg", "ui", "uf", "uo", "ug", "h0", "c0")
    tl = {k: dev(dl[0][k]) for k in lk}
    init_h = torch.zeros(B, 1500, 40, device="cuda")
    init_c = torch.zeros(B, 1500, 40, device="cuda")
    h8, h4 = torch.empty_like(b8), torch.empty_like(b4)
    hl, cl = torch.empty(B, 1500, 40, device="cuda"), torch.empty(B, 1500, 40, device="cuda")
    info = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws8 = api.new_workspace(api.workspace_bytes(api.OP_LINSCAN_BLK8, B, L, H), A8.device)
    ws4 = api.new_workspace(api.workspace_bytes(api.OP_LINSCAN_BLK4, B, L, H), A8.device)
    wsl = api.new_workspace(api.workspace_bytes(api.OP_LSTM_FORWARD, B, 1500, 40, 32), A8.device)

    def calls():
        api.linscan_blk(A8, b8, out=h8, ws=ws8)
        api.linscan_blk(A4, b4, out=h4, ws=ws4)
        api.lstm_forward(*[tl[k] for k in lk[:8]], tl["h0"], tl["c0"], tol=1e-5, max_iter=32,
                         out_h=hl, out_c=cl, info=info, ws=wsl, init_h=init_h, init_c=init_c)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for r in range(3):
        say("replay", r)
        A8.copy_(dev(d8[r]["A"]))
        b8.copy_(dev(d8[r]["b"]))
        A4.copy_(dev(d4[r]["A"]))
        b4.copy_(dev(d4[r]["b"]))
        for k in lk:
            tl[k].copy_(dev(dl[r][k]))
        # warm start from a perturbed rollout of this replay's inputs
        rh, rc = orc.lstm_rollout(*lstm_args(dl[r]), h0=dl[r]["h0"], c0=dl[r]["c0"])
        init_h.copy_(dev((rh + 0.01).astype(np.float32)))
        init_c.copy_(dev((rc - 0.01).astype(np.float32)))
        api.linscan_blk(A8 * 0.5, b8)  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert max_abs(host(h8), orc.linscan_blk(d8[r]["A"], d8[r]["b"])) <= FWD_ATOL
        assert max_abs(host(h4), orc.linscan_blk(d4[r]["A"], d4[r]["b"])) <= FWD_ATOL
        assert info.cpu().tolist()[1] == 1
        assert max(max_abs(host(hl), rh), max_abs(host(cl), rc)) <= FWD_ATOL


def test_captured_head_gru_forward_and_backward_replay(orc):
    """The head GRU's Newton forward (launches up to the cap, the later ones
    exiting at once) and its adjoint (scan plus the two dL/dU passes) under
    capture, each replay against the oracle's rollout and backpropagation
    through time, with the inputs changed in place and eager calls between
    replays."""
    B, L, NH, k = 2, 700, 9, 8
    ds = [synth.head_gru_inputs(B, L, NH, k, seed=870 + r, h0=True, grad=True) for r in range(3)]
    keys = ("pz", "pr", "pc", "Uz", "Ur", "Uc", "h0", "g")
    t = {x: dev(ds[0][x]) for x in keys}
    args = [t[x] for x in ("pz", "pr", "pc", "Uz", "Ur", "Uc")]
    h = torch.empty(B, L, NH, k, device="cuda")
    info = torch.zeros(2, dtype=torch.int32, device="cuda")
    out = tuple(torch.empty(B, L, NH, k, device="cuda") for _ in range(3)) + \
        tuple(torch.empty(NH, k, k, device="cuda") for _ in range(3)) + (torch.empty(B, NH, k, device="cuda"),)
    ws_f = api.new_workspace(api.workspace_bytes(api.OP_HGRU8_FORWARD, B, L, NH, 16), h.device)
    ws_b = api.new_workspace(api.workspace_bytes(api.OP_HGRU8_BACKWARD, B, L, NH), h.device)

    def calls():
        api.hgru_forward(*args, t["h0"], tol=1e-6, max_iter=16, out=h, info=info, ws=ws_f)
        api.hgru_backward(*args, t["h0"], h, t["g"], ws=ws_b, out=out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for r in range(3):
        say("head GRU replay", r)
        for x in keys:
            t[x].copy_(dev(ds[r][x]))
        api.hgru_forward(*[dev(ds[(r + 1) % 3][x]) for x in ("pz", "pr", "pc", "Uz", "Ur", "Uc")], None,
                         tol=1e-4, max_iter=8)  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        d = ds[r]
        p = [d[x] for x in ("pz", "pr", "pc", "Uz", "Ur", "Uc")]
        href = orc.hgru_rollout(*p, h0=d["h0"])
        assert info.cpu().tolist()[1] == 1
        assert max_abs(host(h), href) <= FWD_ATOL
        ref = orc.hgru_bptt(*p, host(h), d["g"], h0=d["h0"])
        errs = [rel_inf(host(gv), rv) for gv, rv in zip(out, ref)]
        say(errs)
        assert max(errs) <= GRAD_RTOL, errs
