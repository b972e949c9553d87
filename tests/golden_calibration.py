"""Reader of tests/golden/calibration_N64_H12_T1024.txt, the float64 oracle's scores of every
head of the calibration workload (written by tests/golden/make_calibration_golden.py, which
calls only the oracle and the seeded input generator)."""
from __future__ import annotations

import os

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "calibration_N64_H12_T1024.txt")


def load() -> dict:
    tau, s_var, s_kl, sq = {}, {}, {}, {}
    ranks = {}
    with open(PATH) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            tok = line.split()
            if tok[0] == "head":
                h = int(tok[1])
                tau[h], s_var[h], s_kl[h], sq[h] = (float(x) for x in tok[2:6])
            else:
                ranks[tok[0]] = [int(x) for x in tok[1:]]
    H = len(tau)
    arr = lambda d: np.array([d[h] for h in range(H)])
    return dict(tau=arr(tau), s_var=arr(s_var), s_kl=arr(s_kl), a_hat_sq=arr(sq),
                rank_var=ranks["rank_var"], rank_kl=ranks["rank_kl"])
