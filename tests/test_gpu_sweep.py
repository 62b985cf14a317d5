"""Randomized GPU parity sweep against the CPU oracle, fixed seeds.

Each case draws a batch size, ragged draft counts (including K_b = 0), a
vocabulary from 7 to 151936 tokens (ragged tails, sizes around the 64K and
chunk boundaries), bf16 or fp32 logits, draft distributions present or absent,
uniform, spread or mixed greedy / random temperatures, logit scales, rounded
logits (ties, signed zeros) and, for part of the cases, per-request top-k /
top-p settings including the off values.  The path is the library's
automatic choice.  The bar is the parity tests' one: tokens and counts
bit-exact on every request the oracle does not flag as a near tie, p(x*)
within the same relative tolerance.
"""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_rs_amd as rs
import rs_workloads as W
from parity import compare, compare_p, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

VOCABS = [7, 100, 1000, 4097, 32000, 65537, 151936]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device (run the CPU suite with -m 'not gpu')")
    rs.load_library()


def _draw(rng):
    V = int(rng.choice(VOCABS))
    bmax = 300 if V <= 32000 else (96 if V <= 65537 else 40)
    B = int(rng.integers(1, bmax + 1))
    kmax = int(rng.integers(0, 11))
    ks = rng.integers(0, kmax + 1, size=B).tolist()
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    q_mode = "noise" if rng.random() < 0.6 else "none"
    kind = int(rng.integers(0, 3))
    temp = 1.0 if kind == 0 else (("uniform", 0.2, 1.5) if kind == 1 else
                                  rng.choice([0.0, 0.5, 1.0, -1.0, 1.3], size=B).tolist())
    std = float(rng.choice([0.5, 2.0, 4.0]))
    draft_mode = "sample_q" if q_mode == "noise" else str(rng.choice(["argmax_mix", "uniform"]))
    w = W.make(ks, V, dtype=dtype, logit_std=std, temperature=temp, q_mode=q_mode,
               q_sigma=float(rng.choice([0.3, 0.8, 1.5])), draft_mode=draft_mode, seed=int(rng.integers(0, 2**40)),
               gen_seed=int(rng.integers(0, 2**31)), device="cuda")
    if rng.random() < 0.3:  # few distinct values: ties everywhere, -0 and +0 among them
        w.logits = (torch.round(w.logits.float() * 2) / 2).to(dtype).contiguous()
    filtered = rng.random() < 0.4
    if filtered:
        tk = rng.choice([0, 1, 5, 50, 1000, V - 1, V + 2], size=B).astype(np.int32).tolist()
        tp = rng.choice([1.0, 0.5, 0.9, 0.99, 0.0], size=B).astype(np.float32).tolist()
        w = w.with_filters(tk, tp)
    desc = f"B={B} K<={kmax} V={V} {str(dtype).split('.')[-1]} q={q_mode} T-kind={kind} std={std}" + \
           (" filtered" if filtered else "")
    return w, desc


@pytest.mark.parametrize("seed", [101, 202, 303])
def test_random_parity_sweep(seed):
    rng = np.random.default_rng(seed)
    for case in range(25):
        w, desc = _draw(rng)
        print(f"[gpu-case] sweep {seed} case {case}: {desc}", flush=True)
        g = run_gpu(w, want_p=True)
        o = run_oracle(w)
        compare(g, o, w)
        compare_p(g, o)
