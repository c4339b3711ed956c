"""Host-only checks of the C-ABI library: it loads, exports every function the
header declares, and its workspace query (pure host arithmetic) behaves.
No kernel is launched here."""
import ctypes
import os
import re

import pytest

from nonlinear_rnn_solve_pararnn_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "pararnn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"if", "sizeof"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.LIB_PATH):
        from nonlinear_rnn_solve_pararnn_amd import build
        build.build()
    return api.load_library()


def test_header_declares_the_five_entry_points():
    names = _declared()
    for n in ("rnn_linscan_diag", "rnn_linscan_blk2", "pararnn_gru_forward",
              "pararnn_lstm_forward", "pararnn_adjoint_backward"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(api.EXPORTS) <= set(_declared())


def test_workspace_query(lib, monkeypatch):
    for op in range(7):
        assert api.workspace_bytes(op, 2, 100, 70, 8) > 0
        assert api.workspace_bytes(op, 0, 100, 70, 8) == 0
        assert api.workspace_bytes(op, 2, -1, 70, 8) == 0
    assert api.workspace_bytes(api.OP_GRU_FORWARD, 2, 100, 70, 0) == 0
    assert api.workspace_bytes(99, 2, 100, 70, 8) == 0
    # the fused GRU kernel (L <= 512) needs none beyond the minimum; a forced
    # override is sized for the kernel it forces
    assert api.workspace_bytes(api.OP_GRU_FORWARD, 16, 512, 4096, 32) == 256
    # past 512 positions: the chained kernel, here with workgroups owning
    # whole chains (1024 chains), which keeps no records
    assert api.workspace_bytes(api.OP_GRU_FORWARD, 16, 513, 4096, 32) == 256
    # grows with the iteration cap: records of every iteration on the chained
    # path (caps up to 64), one max|delta| slot per iteration beyond
    for op in (api.OP_GRU_FORWARD, api.OP_LSTM_FORWARD):
        assert api.workspace_bytes(op, 16, 4096, 64, 60) > api.workspace_bytes(op, 16, 4096, 64, 2)
        assert api.workspace_bytes(op, 16, 4096, 64, 500) > api.workspace_bytes(op, 16, 4096, 64, 100)
    # the chained kernel's whole-chain form (as many chains as workgroup
    # slots: the LSTM at B=8, L=2048, H=2048) keeps no records either
    assert api.workspace_bytes(api.OP_LSTM_FORWARD, 8, 2048, 2048, 32) == 256
    monkeypatch.setenv("PARARNN_LSTM_PATH", "chain")
    assert api.workspace_bytes(api.OP_LSTM_FORWARD, 8, 2048, 2048, 32) > 10 ** 8
    monkeypatch.setenv("PARARNN_LSTM_PATH", "local")
    assert api.workspace_bytes(api.OP_LSTM_FORWARD, 2, 700, 64, 32) == 256
    monkeypatch.setenv("PARARNN_GRU_PATH", "local")
    assert api.workspace_bytes(api.OP_GRU_FORWARD, 2, 700, 64, 32) == 256
    assert api.workspace_bytes(api.OP_GRU_FORWARD, 2, 70000, 1, 32) > 256  # time lanes: always chained
    monkeypatch.setenv("PARARNN_GRU_PATH", "step")
    assert api.workspace_bytes(api.OP_GRU_FORWARD, 16, 512, 4096, 32) > 256
    monkeypatch.setenv("PARARNN_GRU_PATH", "chain")
    assert api.workspace_bytes(api.OP_GRU_FORWARD, 16, 512, 4096, 32) > 256
    assert api.workspace_bytes(api.OP_GRU_FORWARD, 16, 513, 4096, 32) > 256


def test_invalid_arguments_rejected_on_host(lib):
    # validation happens before any HIP call: NULL pointers / bad sizes
    n = None
    assert lib.rnn_linscan_diag(0, 10, 10, n, n, n, n, n, 0, n) == -1
    assert lib.pararnn_gru_forward(1, 10, 10, *([n] * 9), ctypes.c_float(1e-4), 5, n, n, n, 0, n) == -1
    assert lib.pararnn_lstm_forward(1, 10, 10, *([n] * 14), ctypes.c_float(1e-4), 5, n, n, n, 0, n) == -1
    assert lib.pararnn_adjoint_backward(7, 1, 10, 10, *([n] * 13), 0, n) == -1
    assert lib.pararnn_gru_sequential(1, 0, 10, *([n] * 8), n) == -1
    assert lib.rnn_linscan_blk(4, 1, 10, 10, n, n, n, n, n, 0, n) == -1
    assert lib.rnn_linscan_blk(0, 1, 10, 10, n, n, n, n, n, 0, n) == -1
    assert lib.rnn_linscan_blk(3, 1, 10, 10, n, n, n, n, n, 0, n) == -3  # unsupported k
    assert lib.pararnn_lstm_sequential(1, 10, 10, *([n] * 12), n) == -1
    assert lib.pararnn_status_string(-1) == b"invalid argument"


def test_initial_iterate_must_not_overlap_outputs(lib):
    """A warm start's initial iterate is read while the outputs are written:
    any overlap is rejected before anything is enqueued (the pointers below
    are never dereferenced)."""
    B, L, H = 1, 10, 10
    nbytes = B * L * H * 4
    fake = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(8)]
    h = ctypes.c_void_p(0x100000)
    for off in (0, 4, nbytes - 4, -(nbytes - 4)):
        init = ctypes.c_void_p(0x100000 + off)
        assert lib.pararnn_gru_forward(B, L, H, *fake[:6], None, init, h, ctypes.c_float(1e-4), 5,
                                       None, None, None, 0, None) == -1
    c = ctypes.c_void_p(0x200000)
    for hi, ci in ((ctypes.c_void_p(0x200000), None), (None, ctypes.c_void_p(0x100000 + 8)),
                   (ctypes.c_void_p(0x200000 + nbytes - 4), None)):
        assert lib.pararnn_lstm_forward(B, L, H, *fake[:8], None, None, hi, ci, h, c,
                                        ctypes.c_float(1e-4), 5, None, None, None, 0, None) == -1


def test_blk8_workspace_query():
    # header 256 B, then per chunk of 28 positions (4 waves x 7) 9 aggregate
    # words and 1 inclusive word per (batch row, head, row)
    nq, nrow = -(-2048 // 28), 16 * 64 * 8
    assert api.workspace_bytes(api.OP_LINSCAN_BLK8, 16, 2048, 64) == 256 + nq * 9 * nrow * 8 + nq * nrow * 8
    assert api.workspace_bytes(api.OP_LINSCAN_BLK8, 0, 2048, 64) == 0


def test_product_path_does_not_use_the_oracle():
    """The binding and the kernels never import or link the oracle."""
    pkg = os.path.join(ROOT, "nonlinear_rnn_solve_pararnn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text and "oracle.c" not in text, f


def test_binding_calls_match_the_declared_signatures(lib):
    """Every library call in the binding passes as many arguments as its
    ctypes signature declares, and every status check names what failed."""
    import ast
    tree = ast.parse(open(api.__file__).read())
    calls = checks = 0
    for node in ast.walk(tree):
        if not isinstance(node, ast.Call):
            continue
        f = node.func
        if isinstance(f, ast.Name) and f.id == "_check":
            checks += 1
            assert len(node.args) == 2 and not node.keywords, ast.unparse(node)[:120]
        if (isinstance(f, ast.Attribute) and isinstance(f.value, ast.Name) and f.value.id == "lib"
                and f.attr.startswith(("pararnn_", "rnn_"))):
            calls += 1
            assert not any(isinstance(a, ast.Starred) for a in node.args), f.attr
            assert len(node.args) == len(getattr(lib, f.attr).argtypes), f.attr
    assert calls >= 10 and checks >= 10
