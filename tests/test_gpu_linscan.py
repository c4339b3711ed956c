"""GPU parity of the exported linear-recurrence scans against the fp64 oracle."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_pararnn_amd import api, synth
from tests.gpu_helpers import FWD_ATOL, dev, host, max_abs, say

pytestmark = pytest.mark.gpu

# (B, L, H): time lanes (H < 32) and channel lanes (H >= 32), chunks of
# 4096 / 64 positions, ragged tails in L and in the channel blocks.
DIAG_SHAPES = [
    (1, 1, 1), (2, 100, 3), (3, 257, 70), (2, 5000, 1), (1, 70000, 2),
    (4, 1000, 64), (2, 3001, 33), (1, 64, 4), (3, 130, 200), (2, 300, 31), (2, 300, 32),
    (8, 3001, 300),  # more tiles than workgroup slots, ragged in L and in the channel block
]


@pytest.mark.parametrize("B,L,H", DIAG_SHAPES)
@pytest.mark.parametrize("with_h0", [False, True])
def test_linscan_diag_matches_oracle(orc, B, L, H, with_h0):
    say("linscan_diag", B, L, H, with_h0)
    d = synth.linscan_diag_inputs(B, L, H, seed=100 + B * 7 + H, h0=with_h0)
    h0 = dev(d["h0"]) if with_h0 else None
    h = host(api.linscan_diag(dev(d["a"]), dev(d["b"]), h0))
    ref = orc.linscan_diag(d["a"], d["b"], d["h0"] if with_h0 else None)
    assert max_abs(h, ref) <= FWD_ATOL


def _offset(x, k):
    """Copy of x whose data starts k floats past a 16-byte boundary."""
    buf = torch.zeros(x.numel() + 4, dtype=x.dtype, device=x.device)
    v = buf[k:k + x.numel()].view(x.shape)
    v.copy_(x)
    return v


# Tensors whose data start 4 bytes past a 16-byte boundary, against aligned
# ones, at tiles of 256 channels x 128 positions with ragged tails in L and in
# the channel block.
VIEW_SHAPES = [(1, 1, 32), (2, 129, 36), (2, 4100, 256), (1, 3000, 260), (3, 777, 1024), (1, 20000, 64)]


@pytest.mark.parametrize("B,L,H", VIEW_SHAPES)
@pytest.mark.parametrize("misalign", [0, 1])
def test_linscan_diag_aligned_and_offset_views(orc, B, L, H, misalign):
    say("linscan_diag paths", B, L, H, misalign)
    d = synth.linscan_diag_inputs(B, L, H, seed=300 + L + H, h0=True)
    a, b, h0 = dev(d["a"]), dev(d["b"]), dev(d["h0"])
    if misalign:
        a, b, h0 = _offset(a, misalign), _offset(b, misalign), _offset(h0, misalign)
        out = _offset(torch.empty_like(a), misalign)
    else:
        out = torch.empty_like(a)
    h = host(api.linscan_diag(a, b, h0, out=out))
    assert max_abs(h, orc.linscan_diag(d["a"], d["b"], d["h0"])) <= FWD_ATOL


def test_linscan_diag_signed_coefficients(orc):
    # a in (-1, 1): sign changes exercise the composition of negative factors
    d = synth.linscan_diag_inputs(2, 9000, 40, seed=7, alo=-1.0, ahi=1.0, h0=True)
    h = host(api.linscan_diag(dev(d["a"]), dev(d["b"]), dev(d["h0"])))
    assert max_abs(h, orc.linscan_diag(d["a"], d["b"], d["h0"])) <= FWD_ATOL


def test_linscan_diag_full_workload(orc):
    """B=16, L=4096, H=1024, a~U(0.5,1), b~N(0,1), h0=0: every output checked."""
    say("linscan_diag full workload")
    d = synth.workload_inputs("c1_linscan")
    h = host(api.linscan_diag(dev(d["a"]), dev(d["b"])))
    ref = orc.linscan_diag(d["a"], d["b"])
    err = max_abs(h, ref)
    say("max abs err", err)
    assert err <= FWD_ATOL


def test_linscan_diag_repeatable_within_tolerance(orc):
    d = synth.linscan_diag_inputs(2, 20000, 48, seed=11)
    a, b = dev(d["a"]), dev(d["b"])
    h1 = host(api.linscan_diag(a, b))
    for _ in range(5):
        assert max_abs(host(api.linscan_diag(a, b)), h1) <= 1e-5


# (8, 3001, 300): more tiles than workgroup slots, so the prefetching kernel
# runs several tiles per workgroup, alternating its two register sets, with a
# ragged last chunk and a ragged channel block
BLK2_SHAPES = [(1, 1, 1), (2, 100, 3), (2, 3000, 1), (3, 257, 70), (2, 700, 33), (1, 9000, 40), (8, 3001, 300)]


@pytest.mark.parametrize("B,L,H", BLK2_SHAPES)
@pytest.mark.parametrize("with_h0", [False, True])
def test_linscan_blk2_matches_oracle(orc, B, L, H, with_h0):
    say("linscan_blk2", B, L, H, with_h0)
    d = synth.linscan_blk2_inputs(B, L, H, seed=200 + B * 5 + H, h0=with_h0)
    h0 = dev(d["h0"]) if with_h0 else None
    h = host(api.linscan_blk2(dev(d["A"]), dev(d["b"]), h0))
    ref = orc.linscan_blk2(d["A"], d["b"], d["h0"] if with_h0 else None)
    assert max_abs(h, ref) <= FWD_ATOL


def test_linscan_blk2_full_workload(orc):
    """B=16, L=4096, H=512, A ~ U(-0.6,0.6), b ~ N(0,1), h0 = 0: every output checked."""
    say("linscan_blk2 full workload")
    d = synth.workload_inputs("x_linscan_blk2")
    h = host(api.linscan_blk2(dev(d["A"]), dev(d["b"])))
    err = max_abs(h, orc.linscan_blk2(d["A"], d["b"]))
    say("max abs err", err)
    assert err <= FWD_ATOL


def test_linscan_blk2_large(orc):
    d = synth.linscan_blk2_inputs(4, 4096, 1024, seed=5)
    h = host(api.linscan_blk2(dev(d["A"]), dev(d["b"])))
    assert max_abs(h, orc.linscan_blk2(d["A"], d["b"])) <= FWD_ATOL


def test_linscan_blk2_diagonal_blocks_equal_diag_scan():
    # cross-kernel special case: diagonal 2x2 blocks = two independent diag scans
    rng = np.random.default_rng(3)
    B, L, H = 2, 5000, 40
    a0 = rng.uniform(0.5, 1.0, (B, L, H)).astype(np.float32)
    a1 = rng.uniform(0.5, 1.0, (B, L, H)).astype(np.float32)
    A = np.zeros((B, L, H, 2, 2), np.float32)
    A[..., 0, 0] = a0
    A[..., 1, 1] = a1
    b = rng.standard_normal((B, L, H, 2)).astype(np.float32)
    h = host(api.linscan_blk2(dev(A), dev(b)))
    h0 = host(api.linscan_diag(dev(a0), dev(np.ascontiguousarray(b[..., 0]))))
    h1 = host(api.linscan_diag(dev(a1), dev(np.ascontiguousarray(b[..., 1]))))
    assert max_abs(h[..., 0], h0) <= 1e-5 and max_abs(h[..., 1], h1) <= 1e-5


def test_linscan_rejects_bad_arguments():
    a = torch.zeros(2, 10, 4, device="cuda:0")
    with pytest.raises(ValueError):
        api.linscan_diag(a, torch.zeros(2, 10, 5, device="cuda:0"))
    with pytest.raises(TypeError):
        api.linscan_diag(a.double(), a.double())
    ws = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(ValueError):
        api.linscan_diag(a, a, ws=ws)


def test_workspace_reused_across_entry_points_and_shapes(orc, monkeypatch):
    """One zero-filled workspace serves a sequence of calls of different entry
    points and shapes (every launch leaves its ticket header ready and its
    look-back records tagged with its own launch number)."""
    from tests.gpu_helpers import lstm_args
    monkeypatch.setenv("PARARNN_GRU_PATH", "step")
    big = max(api.workspace_bytes(op, 3, 5000, 70, 16) for op in range(6))
    ws = api.new_workspace(big, "cuda:0")
    d1 = synth.linscan_diag_inputs(3, 5000, 70, seed=21)
    d2 = synth.linscan_blk2_inputs(2, 700, 33, seed=22)
    d3 = synth.lstm_inputs(2, 300, 40, seed=23, h0=True)
    d4 = synth.linscan_diag_inputs(1, 4000, 3, seed=24)
    d5 = synth.gru_inputs(2, 2000, 5, seed=25)
    for rnd in range(3):
        say("round", rnd)
        h = host(api.linscan_diag(dev(d1["a"]), dev(d1["b"]), ws=ws))
        assert max_abs(h, orc.linscan_diag(d1["a"], d1["b"])) <= FWD_ATOL
        h = host(api.linscan_blk2(dev(d2["A"]), dev(d2["b"]), ws=ws))
        assert max_abs(h, orc.linscan_blk2(d2["A"], d2["b"])) <= FWD_ATOL
        info = torch.zeros(2, dtype=torch.int32, device="cuda:0")
        h, c = api.lstm_forward(*[dev(x) for x in lstm_args(d3)], dev(d3["h0"]), dev(d3["c0"]),
                                tol=1e-5, max_iter=16, info=info, ws=ws)
        hr, cr = orc.lstm_rollout(*lstm_args(d3), h0=d3["h0"], c0=d3["c0"])
        assert int(info[1]) == 1 and max_abs(host(h), hr) <= FWD_ATOL and max_abs(host(c), cr) <= FWD_ATOL
        h = host(api.linscan_diag(dev(d4["a"]), dev(d4["b"]), ws=ws))
        assert max_abs(h, orc.linscan_diag(d4["a"], d4["b"])) <= FWD_ATOL
        g = [dev(d5[k]) for k in ("pz", "pr", "pc", "uz", "ur", "uc")]
        h = host(api.gru_forward(*g, tol=1e-5, max_iter=16, info=info, ws=ws))
        ref = orc.gru_rollout(*(d5[k] for k in ("pz", "pr", "pc", "uz", "ur", "uc")))
        assert int(info[1]) == 1 and max_abs(h, ref) <= FWD_ATOL


def test_two_streams_with_their_own_workspaces(orc):
    """Calls enqueued on two streams at once, each stream with the workspace
    the binding keeps for it, overlap on the device and stay independent."""
    d1 = synth.linscan_diag_inputs(4, 6000, 96, seed=31)
    d2 = synth.linscan_diag_inputs(3, 5000, 2, seed=32)
    a1, b1, a2, b2 = dev(d1["a"]), dev(d1["b"]), dev(d2["a"]), dev(d2["b"])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    out1, out2 = [], []
    for _ in range(4):
        with torch.cuda.stream(s1):
            out1.append(api.linscan_diag(a1, b1))
        with torch.cuda.stream(s2):
            out2.append(api.linscan_diag(a2, b2))
    torch.cuda.synchronize()
    ref1, ref2 = orc.linscan_diag(d1["a"], d1["b"]), orc.linscan_diag(d2["a"], d2["b"])
    for h in out1:
        assert max_abs(host(h), ref1) <= FWD_ATOL
    for h in out2:
        assert max_abs(host(h), ref2) <= FWD_ATOL


# 4x4 blocks: 16 blocks per wave (each block's rows on 4 lanes), chunks of 8
# waves x 8 positions; ragged tails in L and in the blocks of a wave.  The
# thread-per-block kernel (time and channel lanes) is covered by
# test_linscan_blk4_thread_path.
BLK4_SHAPES = [(1, 1, 1), (2, 100, 3), (2, 1500, 2), (3, 257, 70), (2, 300, 31), (2, 300, 32),
               (4, 1000, 64), (1, 64, 4), (2, 97, 130)]


@pytest.mark.parametrize("B,L,H", BLK4_SHAPES)
@pytest.mark.parametrize("with_h0", [False, True])
def test_linscan_blk4_matches_oracle(orc, B, L, H, with_h0):
    say("linscan_blk4", B, L, H, with_h0)
    d = synth.linscan_blk_inputs(B, L, H, 4, seed=300 + B * 7 + H, h0=with_h0)
    h0 = dev(d["h0"]) if with_h0 else None
    h = host(api.linscan_blk(dev(d["A"]), dev(d["b"]), h0))
    ref = orc.linscan_blk(d["A"], d["b"], d["h0"] if with_h0 else None)
    err = max_abs(h, ref)
    say(err)
    assert err <= FWD_ATOL


def test_linscan_blk4_full_workload(orc):
    """The 4x4 scan at the measured size, B=16, L=2048, H=256, every element."""
    say("linscan_blk4 full workload")
    d = synth.workload_inputs("x_linscan_blk4")
    h = host(api.linscan_blk(dev(d["A"]), dev(d["b"])))
    err = max_abs(h, orc.linscan_blk(d["A"], d["b"]))
    say(err)
    assert err <= FWD_ATOL


def test_linscan_blk_k2_is_the_2x2_scan(orc):
    d = synth.linscan_blk2_inputs(2, 700, 40, seed=310, h0=True)
    h = host(api.linscan_blk(dev(d["A"]), dev(d["b"]), dev(d["h0"])))
    assert max_abs(h, orc.linscan_blk2(d["A"], d["b"], d["h0"])) <= FWD_ATOL


def test_linscan_blk4_repeated_calls_share_a_workspace(orc):
    """Back-to-back calls on one workspace (launch tags keep the records of the
    calls apart) give the same result as fresh ones."""
    d = synth.linscan_blk_inputs(2, 2000, 96, 4, seed=311)
    A, b = dev(d["A"]), dev(d["b"])
    ws = api.new_workspace(api.workspace_bytes(api.OP_LINSCAN_BLK4, 2, 2000, 96), A.device)
    outs = [host(api.linscan_blk(A, b, ws=ws)) for _ in range(3)]
    ref = orc.linscan_blk(d["A"], d["b"])
    for h in outs:
        assert max_abs(h, ref) <= FWD_ATOL


def test_linscan_blk4_thread_path(orc, monkeypatch):
    """The one-thread-per-block 4x4 kernel, still selectable, on both lane
    layouts with ragged tails."""
    monkeypatch.setenv("PARARNN_BLK4_PATH", "thread")
    for B, L, H in [(2, 1500, 2), (3, 257, 70)]:
        say("linscan_blk4 thread path", B, L, H)
        d = synth.linscan_blk_inputs(B, L, H, 4, seed=340 + H, h0=True)
        h = host(api.linscan_blk(dev(d["A"]), dev(d["b"]), dev(d["h0"])))
        assert max_abs(h, orc.linscan_blk(d["A"], d["b"], d["h0"])) <= FWD_ATOL


# 8x8 blocks: 8 heads per wave, chunks of 4 waves x 7 positions; ragged head
# blocks (H not a multiple of 8), ragged chunks, a single head over a long L.
BLK8_SHAPES = [(1, 1, 1), (2, 100, 3), (3, 257, 9), (2, 1500, 2), (2, 300, 16), (1, 64, 8),
               (2, 97, 13), (1, 3000, 1)]


@pytest.mark.parametrize("B,L,H", BLK8_SHAPES)
@pytest.mark.parametrize("with_h0", [False, True])
def test_linscan_blk8_matches_oracle(orc, B, L, H, with_h0):
    say("linscan_blk8", B, L, H, with_h0)
    d = synth.linscan_blk_inputs(B, L, H, 8, seed=400 + B * 7 + H, h0=with_h0)
    h0 = dev(d["h0"]) if with_h0 else None
    h = host(api.linscan_blk(dev(d["A"]), dev(d["b"]), h0))
    err = max_abs(h, orc.linscan_blk(d["A"], d["b"], d["h0"] if with_h0 else None))
    say(err)
    assert err <= FWD_ATOL


def test_linscan_blk8_full_workload(orc):
    """The 8x8 scan at the measured size, B=16, L=2048, H=64 heads, every element."""
    say("linscan_blk8 full workload")
    d = synth.workload_inputs("x_linscan_blk8")
    h = host(api.linscan_blk(dev(d["A"]), dev(d["b"])))
    err = max_abs(h, orc.linscan_blk(d["A"], d["b"]))
    say(err)
    assert err <= FWD_ATOL


def test_linscan_blk8_repeated_calls_share_a_workspace(orc):
    d = synth.linscan_blk_inputs(2, 2000, 24, 8, seed=411)
    A, b = dev(d["A"]), dev(d["b"])
    ws = api.new_workspace(api.workspace_bytes(api.OP_LINSCAN_BLK8, 2, 2000, 24), A.device)
    outs = [host(api.linscan_blk(A, b, ws=ws)) for _ in range(3)]
    ref = orc.linscan_blk(d["A"], d["b"])
    for h in outs:
        assert max_abs(h, ref) <= FWD_ATOL


def test_linscan_blk_rejects_unsupported_k():
    A = torch.zeros(1, 4, 2, 3, 3, device="cuda")
    b = torch.zeros(1, 4, 2, 3, device="cuda")
    with pytest.raises(api.PararnnError):
        api.linscan_blk(A, b)


# Block scans on tensors whose data start 4, 8 or 12 bytes past a 16-byte
# boundary (the per-float load path) against aligned ones (16-byte blocks),
# channel lanes and time lanes, ragged tails in L and in the channel block.
BLK_VIEW_SHAPES = [(1, 1, 1), (2, 129, 36), (2, 1030, 3), (1, 3000, 70)]


@pytest.mark.parametrize("B,L,H", BLK_VIEW_SHAPES)
@pytest.mark.parametrize("misalign", [0, 1, 2])
def test_linscan_blk2_aligned_and_offset_views(orc, B, L, H, misalign):
    say("linscan_blk2 paths", B, L, H, misalign)
    d = synth.linscan_blk2_inputs(B, L, H, seed=320 + L + H, h0=True)
    A, b, h0 = dev(d["A"]), dev(d["b"]), dev(d["h0"])
    out = torch.empty_like(b)
    if misalign:
        A, b, h0, out = (_offset(x, misalign) for x in (A, b, h0, out))
    h = host(api.linscan_blk2(A, b, h0, out=out))
    assert max_abs(h, orc.linscan_blk2(d["A"], d["b"], d["h0"])) <= FWD_ATOL


@pytest.mark.parametrize("B,L,H", BLK_VIEW_SHAPES)
@pytest.mark.parametrize("misalign", [0, 1, 3])
def test_linscan_blk4_aligned_and_offset_views(orc, B, L, H, misalign):
    say("linscan_blk4 paths", B, L, H, misalign)
    d = synth.linscan_blk_inputs(B, L, H, 4, seed=330 + L + H, h0=True)
    A, b, h0 = dev(d["A"]), dev(d["b"]), dev(d["h0"])
    out = torch.empty_like(b)
    if misalign:
        A, b, h0, out = (_offset(x, misalign) for x in (A, b, h0, out))
    h = host(api.linscan_blk(A, b, h0, out=out))
    assert max_abs(h, orc.linscan_blk(d["A"], d["b"], d["h0"])) <= FWD_ATOL


@pytest.mark.parametrize("B,L,H", BLK_VIEW_SHAPES)
@pytest.mark.parametrize("misalign", [0, 1, 3])
def test_linscan_blk8_aligned_and_offset_views(orc, B, L, H, misalign):
    say("linscan_blk8 paths", B, L, H, misalign)
    d = synth.linscan_blk_inputs(B, L, H, 8, seed=430 + L + H, h0=True)
    A, b, h0 = dev(d["A"]), dev(d["b"]), dev(d["h0"])
    out = torch.empty_like(b)
    if misalign:
        A, b, h0, out = (_offset(x, misalign) for x in (A, b, h0, out))
    h = host(api.linscan_blk(A, b, h0, out=out))
    assert max_abs(h, orc.linscan_blk(d["A"], d["b"], d["h0"])) <= FWD_ATOL
