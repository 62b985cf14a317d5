"""Find the draft-noise scale sigma of the B=256, K=8, V=151936 workload.

The workload builds q = softmax(l / T_b + N(0, sigma^2)) and asks for a mean
acceptance of about 0.75, where a draft row's acceptance is
A = sum_x min(p(x), q(x)) with p = softmax(l / T_b) (the acceptance of the
verify rule; Ch.12 "投机解码：以小博大" §12.2.2, the quantity A in the proof).
p comes from the oracle (fp64); q and the logits from rs_workloads.  The
bisection reuses the same seeded logits and noise for every sigma.

Usage: python oracle/calibrate_sigma.py [--B 128] [--target 0.75]
"""
import argparse
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
import rs_workloads as W  # noqa: E402


def mean_acceptance(B: int, sigma: float, V: int = 151936) -> float:
    w = W.make([8] * B, V, logit_std=4.0, temperature=("uniform", 0.3, 1.2), q_mode="noise",
               q_sigma=sigma, q_over_T=True, gen_seed=1004)
    p = oracle.probs(w.logits, w.cu_num_draft_tokens, w.temperature)
    rows = W.draft_rows(w.num_draft).numpy()
    q = w.draft_probs.double().numpy()
    return float(np.minimum(p[rows], q).sum(axis=1).mean())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--B", type=int, default=128)
    ap.add_argument("--target", type=float, default=0.75)
    ap.add_argument("--iters", type=int, default=12)
    a = ap.parse_args()
    lo, hi = 0.3, 2.0
    for _ in range(a.iters):
        mid = 0.5 * (lo + hi)
        A = mean_acceptance(a.B, mid)
        print(f"sigma={mid:.4f} mean A={A:.4f}", flush=True)
        if A > a.target:
            lo = mid
        else:
            hi = mid
    s = round(0.5 * (lo + hi), 2)
    print(f"sigma={s:.2f} mean A={mean_acceptance(a.B, s):.4f} over {8 * a.B} draft rows")


if __name__ == "__main__":
    main()
