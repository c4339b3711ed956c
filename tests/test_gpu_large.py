"""GPU parity beyond 2^31 elements per tensor (64-bit indexing everywhere):
the diagonal scan, the fused GRU forward and the chained GRU forward on
tensors of more than 2^31 floats (8.6 GB each), checked on sampled channels
against the oracle.  Inputs are drawn on the device with torch's seeded
generator (the sizes are too large to draw on the host); the sampled
channels' inputs are copied back and given to the oracle."""
import pytest
import torch

from nonlinear_rnn_solve_pararnn_amd import api
from tests.gpu_helpers import FWD_ATOL, max_abs, say

pytestmark = pytest.mark.gpu


def _gen(seed):
    return torch.Generator(device="cuda").manual_seed(seed)


def _col(x, b, j):
    """Channel (b, j) of a [B, L, H] device tensor as a [1, L, 1] host array."""
    return x[b, :, j].contiguous().cpu().numpy()[None, :, None]


def _free():
    torch.cuda.synchronize()
    api.release_workspaces()
    torch.cuda.empty_cache()


def test_linscan_diag_beyond_2_31_elements(orc):
    B, L, H = 2, (1 << 20) + 3, 1030  # 2,160,072,300 elements
    assert B * L * H > 2 ** 31
    say("linscan_diag", B, L, H)
    g = _gen(400)
    a = torch.rand((B, L, H), generator=g, device="cuda") * 0.5 + 0.5
    b = torch.randn((B, L, H), generator=g, device="cuda")
    h = api.linscan_diag(a, b)
    for bb, j in [(0, 0), (1, H - 1), (1, 517), (0, 1029), (1, 64)]:
        err = max_abs(_col(h, bb, j), orc.linscan_diag(_col(a, bb, j), _col(b, bb, j)))
        say(bb, j, err)
        assert err <= FWD_ATOL
    del a, b, h
    _free()


@pytest.mark.parametrize("H", [(1 << 18) + 16, (1 << 18) + 10])
def test_gru_fused_beyond_2_31_elements(orc, H):
    """L = 512: the fused kernel, with whole and ragged 16-channel tiles."""
    B, L = 16, 512
    assert B * L * H > 2 ** 31
    say("gru fused", B, L, H)
    g = _gen(401)
    p = [torch.randn((B, L, H), generator=g, device="cuda") * 0.5 for _ in range(3)]
    u = [torch.rand(H, generator=g, device="cuda") - 0.5 for _ in range(3)]
    info = torch.zeros(2, dtype=torch.int32, device="cuda")
    h = api.gru_forward(*p, *u, tol=1e-5, max_iter=12, info=info)
    assert info.cpu().tolist()[1] == 1
    for bb, j in [(0, 0), (15, H - 1), (7, 131075), (3, H - 17)]:
        ref = orc.gru_rollout(*[_col(x, bb, j) for x in p], *[x[j:j + 1].cpu().numpy() for x in u])
        err = max_abs(_col(h, bb, j), ref)
        say(bb, j, err)
        assert err <= FWD_ATOL
    del p, u, h
    _free()


def test_gru_chained_beyond_2_31_elements(orc):
    """L = 2^20 + 5 with channel lanes: the chained kernel across workgroups."""
    B, L, H = 2, (1 << 20) + 5, 1030
    assert B * L * H > 2 ** 31
    say("gru chain", B, L, H)
    g = _gen(402)
    p = [torch.randn((B, L, H), generator=g, device="cuda") for _ in range(3)]
    u = [torch.rand(H, generator=g, device="cuda") - 0.5 for _ in range(3)]
    info = torch.zeros(2, dtype=torch.int32, device="cuda")
    h = api.gru_forward(*p, *u, tol=1e-5, max_iter=8, info=info)
    assert info.cpu().tolist()[1] == 1
    for bb, j in [(0, 0), (1, H - 1), (1, 1000), (0, 513)]:
        ref = orc.gru_rollout(*[_col(x, bb, j) for x in p], *[x[j:j + 1].cpu().numpy() for x in u])
        err = max_abs(_col(h, bb, j), ref)
        say(bb, j, err)
        assert err <= FWD_ATOL
    del p, u, h
    _free()


def test_linscan_blk8_beyond_2_31_floats(orc):
    """8x8 blocks: A holds more than 2^31 floats (and the records more than
    2^31 words' worth of index range); sampled heads against the oracle."""
    B, L, H = 2, (1 << 17) + 5, 130  # A: 2 x 131077 x 130 x 64 = 2,181,121,280 floats
    assert B * L * H * 64 > 2 ** 31
    say("linscan_blk8", B, L, H)
    g = _gen(430)
    A = (torch.rand((B, L, H, 8, 8), generator=g, device="cuda") - 0.5) * 0.6
    b = torch.randn((B, L, H, 8), generator=g, device="cuda")
    h = api.linscan_blk(A, b)
    for bb, j in [(0, 0), (1, H - 1), (1, 64), (0, 127)]:
        Aj = A[bb, :, j].contiguous().cpu().numpy()[None, :, None]
        bj = b[bb, :, j].contiguous().cpu().numpy()[None, :, None]
        err = max_abs(h[bb, :, j].contiguous().cpu().numpy()[None, :, None], orc.linscan_blk(Aj, bj))
        say(bb, j, err)
        assert err <= FWD_ATOL
    del A, b, h
    _free()
