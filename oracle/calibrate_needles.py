"""Calibrate the needle amplitude of the 128K workload with the oracle (test infrastructure).

The 128K workload asks for about 75% of causal (row, kv head, chunk) pairs to receive zero
routing weight.  This script bisects the needle amplitude A of the seeded generator so
that the oracle's Stage 0 + Stage 1, on sampled query rows weighted by how many chunks
they route over, gives a zero-weight fraction of 0.75 +- 0.02.  It calls only the oracle
and the input generator; its result is stored as CALIBRATED_AMP in the workload table.

    python -m oracle.calibrate_needles [--target 0.75] [--blocks 64]
"""
import argparse
import dataclasses
import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from long_context_sparse_stage0_amd import synth  # noqa: E402
from long_context_sparse_stage0_amd.workloads import PREFILL_128K_GQA  # noqa: E402
from oracle import dash_oracle as O  # noqa: E402


def zero_fraction_at(amp, w, blocks, rows_per_block, seed=7):
    w = dataclasses.replace(w, needle_amp=amp)
    x = synth.prefill_inputs(w)
    scale = 1.0 / math.sqrt(w.D)
    summ = O.chunk_summaries(x["k"], x["head_cls"], scale)
    rng = np.random.default_rng(seed)
    nblk = w.T // 64
    # causal weighting: block i routes over i chunks
    pb = np.arange(nblk, dtype=np.float64)
    pb /= pb.sum()
    picks = rng.choice(nblk, size=blocks, replace=True, p=pb)
    zero = tot = 0
    for blk in picks:
        for t in blk * 64 + rng.choice(64, size=rows_per_block, replace=False):
            for kvh in range(w.Hkv):
                qg = x["q"][0, kvh * w.G:(kvh + 1) * w.G, t]
                wb, _, _ = O.route_row(qg, summ[0, kvh], int(t), alpha=w.alpha, gamma=w.gamma,
                                       scale=scale)
                zero += int((wb == 0.0).sum())
                tot += wb.size
    return zero / tot


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--target", type=float, default=0.75)
    ap.add_argument("--blocks", type=int, default=64)
    ap.add_argument("--rows-per-block", type=int, default=2)
    ap.add_argument("--lo", type=float, default=0.0)
    ap.add_argument("--hi", type=float, default=1.0)
    ap.add_argument("--iters", type=int, default=10)
    a = ap.parse_args()
    w = PREFILL_128K_GQA
    lo, hi = a.lo, a.hi
    f_lo = zero_fraction_at(lo, w, a.blocks, a.rows_per_block)
    f_hi = zero_fraction_at(hi, w, a.blocks, a.rows_per_block)
    print(f"A={lo:.4f}: {f_lo:.4f}   A={hi:.4f}: {f_hi:.4f}", flush=True)
    best = (abs(f_lo - a.target), lo, f_lo)
    for _ in range(a.iters):
        mid = 0.5 * (lo + hi)
        f = zero_fraction_at(mid, w, a.blocks, a.rows_per_block)
        print(f"A={mid:.4f}: {f:.4f}", flush=True)
        best = min(best, (abs(f - a.target), mid, f))
        if (f < a.target) == (f_lo < a.target):
            lo, f_lo = mid, f
        else:
            hi = mid
        if abs(f - a.target) < 0.005:
            break
    print(f"calibrated amplitude {best[1]:.4f} gives zero fraction {best[2]:.4f}")


if __name__ == "__main__":
    main()
