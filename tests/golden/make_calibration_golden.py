"""Writes calibration_N64_H12_T1024.txt: the float64 oracle's scores of every head of the
calibration workload (N = 64 sequences, H = 12 heads, T = 1024, d_h = 64, bf16 Q and K, per-head
temperatures log-spaced over [0.1, 4]; seed 4 of the input generator).

    python tests/golden/make_calibration_golden.py

It calls only the CPU oracle (oracle/saf_oracle.py) and the seeded input generator
(hybrid_static_pattern_amd/inputs.py, random numbers only). Stored per head: s_var of Eq. (1)
(part 二.1 of "When Can Attention Heads Be Statically Defined?: 中文精读笔记"), the forward-KL
score s^KL of the same part, and the sum over all entries of A-hat squared (a fingerprint of
the whole mean pattern); then both rankings (ascending, ties to the lower index). Takes
about two minutes on eight cores.
"""
from __future__ import annotations

import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from hybrid_static_pattern_amd import inputs  # noqa: E402
from oracle import saf_oracle  # noqa: E402

OUT = os.path.join(HERE, "calibration_N64_H12_T1024.txt")


def main() -> None:
    spec = inputs.CALIBRATION
    C = inputs.make_calibration(**spec)
    scale = 1.0 / math.sqrt(C["D"])
    H = C["H"]
    s_var, s_kl, sq = np.empty(H), np.empty(H), np.empty(H)
    for h in range(H):
        q, k = C["q"][:, h:h + 1], C["k"][:, h:h + 1]
        A_hat, sv, _ = saf_oracle.var_score(q, k, scale)
        _, sk, _ = saf_oracle.kl_score(q, k, scale)
        s_var[h], s_kl[h], sq[h] = sv[0], sk[0], float((A_hat[0] ** 2).sum())
        print(f"head {h}: tau {C['tau'][h]:.4f} s_var {s_var[h]:.6e} s_kl {s_kl[h]:.6e}", flush=True)
    with open(OUT, "w") as f:
        f.write("# Calibration workload scores from the float64 CPU oracle; written by\n")
        f.write("# tests/golden/make_calibration_golden.py (see its docstring for the inputs).\n")
        f.write(f"# N={C['N']} H={H} T={C['T']} D={C['D']} seed={C['seed']} scale=1/sqrt(D)\n")
        f.write("# head tau s_var s_kl sum_ij(A_hat^2)\n")
        for h in range(H):
            f.write(f"head {h} {float(C['tau'][h])!r} {float(s_var[h])!r} {float(s_kl[h])!r} {float(sq[h])!r}\n")
        f.write("rank_var " + " ".join(str(int(x)) for x in saf_oracle.rank_heads(s_var)) + "\n")
        f.write("rank_kl " + " ".join(str(int(x)) for x in saf_oracle.rank_heads(s_kl)) + "\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
