"""Writes oracle_small_step.npz: oracle outputs on a fixed seeded 6x10 input.

It calls only the CPU oracle, so the stored values are the oracle's and pin it
against unintended change. Run from the repository root:
    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import muon_oracle as O  # noqa: E402


def main():
    rng = np.random.default_rng(20260)
    w, g, m = (rng.standard_normal((6, 10)) for _ in range(3))
    r = O.muon_step_ref(w, g, m, lr=0.02, weight_decay=0.01, heads=2, mu=0.95, nesterov=True, scale=1.0)
    np.savez(os.path.join(HERE, "oracle_small_step.npz"), w=w, g=g, m=m,
             w_new=r["w"], o=r["o"], m_new=r["m"])


if __name__ == "__main__":
    main()
