"""MI355X-native parallel Newton evaluation of nonlinear RNNs.

The computation lives in libpararnn.so (HIP kernels for gfx950, C ABI in
include/pararnn.h); ``api`` is its thin torch binding.  Importing the package
does not load the library; the first call does, and raises if it is missing.
"""
from .api import (CELL_GRU, CELL_LSTM, PararnnError, adjoint_backward, gru_forward,  # noqa: F401
                  gru_sequential, linscan_blk, linscan_blk2, linscan_diag, load_library, lstm_forward,
                  lstm_sequential, workspace_bytes)
