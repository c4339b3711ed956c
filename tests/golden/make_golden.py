"""Writes c0_gru_rollout.txt: the fp64 oracle's sequential GRU rollout of the
tiny workload (B=1, L=64, H=4, seeded synthetic inputs, h0 = 0).

    python tests/golden/make_golden.py

Calls only the oracle and the seeded input generator.  The file also records
the sum of the fp32 inputs so that a change in the generator shows up as a
fixture mismatch rather than as a silent change of the compared values.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from nonlinear_rnn_solve_pararnn_amd import synth  # noqa: E402

KEYS = ("pz", "pr", "pc", "uz", "ur", "uc", "h0")
OUT = os.path.join(HERE, "c0_gru_rollout.txt")


def input_checksum(d):
    return float(sum(np.asarray(d[k], np.float64).sum() for k in KEYS))


def main():
    d = synth.workload_inputs("c0_gru_tiny")
    h = oracle.gru_rollout(*(d[k] for k in KEYS[:6]), h0=d["h0"])
    B, L, H = h.shape
    with open(OUT, "w") as f:
        f.write("# fp64 sequential GRU rollout, workload c0_gru_tiny (B=%d L=%d H=%d)\n" % (B, L, H))
        f.write("# written by tests/golden/make_golden.py from the oracle only\n")
        f.write("input_checksum %.17g\n" % input_checksum(d))
        for t in range(L):
            f.write(" ".join("%.17g" % v for v in h[0, t]) + "\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
