"""Writes signsel_errors.txt: the oracle's attention-output error of every candidate sign pattern on the
seeded sign-selection workload (8 calibration samples, 32 query / 8 kv heads, d=128, 512 keys each,
4-bit codes, 200 candidates), for the GPU test that checks the full-size selection.

Only the oracle computes these numbers (AXELRAM, Key Points / Abstract: a one-time choice among candidate
sign patterns on calibration samples, ranked here by attention-output error).  Run from the repository
root:  python tests/golden/make_signsel_errors.py   (about 30 s on 8 cores).
"""
import math
import os
import sys
from multiprocessing import Pool

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

OUT = os.path.join(HERE, "signsel_errors.txt")


def _inputs():
    sh = W.SIGNSEL
    return sh, W.queries(sh), W.keys(sh), W.values(sh), W.sign_candidates(sh)


def _part(rows):
    sh, q, k, v, cands = _inputs()
    lv, th = oracle.codebook(sh.d, sh.b)
    e, _ = oracle.sign_errors(lv, th, cands[rows[0]:rows[1]], q, k, v, 1.0 / math.sqrt(sh.d))
    return e


def main():
    oracle.build(force=False)
    C = W.SIGN_CANDIDATES
    parts = [(i, min(i + 25, C)) for i in range(0, C, 25)]
    with Pool(min(8, len(parts))) as pool:
        errs = np.concatenate(pool.map(_part, parts))
    best = int(np.argmin(errs))
    with open(OUT, "w") as f:
        f.write("# oracle attention-output error sum|o_c - o|^2 / sum|o|^2 of each candidate sign pattern\n")
        f.write("# workload: signsel (B=8 Hq=32 Hkv=8 d=128 T=512 b=4, fp16, seed %d), %d candidates\n"
                % (W.SIGNSEL.seed, C))
        f.write("# written by tests/golden/make_signsel_errors.py (oracle only)\n")
        f.write("best %d\n" % best)
        for c, e in enumerate(errs):
            f.write("%d %.12e\n" % (c, e))
    print("best", best, "error", errs[best], "worst", errs.max())


if __name__ == "__main__":
    main()
