"""Pins of the oracle's greedy path (temperature 0): accept iff the draft equals
the target argmax, emit the target argmax at the first mismatch or as the bonus
[第12章 投机解码：以小博大 §12.2.4; 投机解码（Speculative Decoding）端到端深挖 §7.1].

Checked against the worked examples the pages print (tests/golden) and against
brute force built on numpy's argmax (first occurrence = lowest index on ties).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _rows_with_argmax(targets, V, rng):
    rows = rng.standard_normal((len(targets), V)).astype(np.float32)
    for i, t in enumerate(targets):
        rows[i, t] = rows[i].max() + 1.0
    return rows


def brute_force(rows, drafts, cu, max_k):
    B = len(cu) - 1
    out = np.full((B, max_k + 1), -1, np.int32)
    nacc = np.zeros(B, np.int32)
    for b in range(B):
        s, e = cu[b], cu[b + 1]
        g = [int(np.argmax(rows[s + b + j])) for j in range(e - s + 1)]
        n = e - s
        for j in range(e - s):
            if drafts[s + j] != g[j]:
                n = j
                break
        out[b, :n] = drafts[s:s + n]
        out[b, n] = g[n]
        nacc[b] = n
    return out, nacc


def test_worked_examples():
    cases = json.load(open(os.path.join(HERE, "golden", "greedy_worked_examples.json")))["cases"]
    rng = np.random.default_rng(0)
    for c in cases:
        K = len(c["drafts"])
        rows = _rows_with_argmax(c["argmax"], 6, rng)
        cu = np.array([0, K], np.int32)
        for r in (oracle.verify_greedy(rows, np.array(c["drafts"], np.int32), cu, K),
                  oracle.verify(rows, None, np.array(c["drafts"], np.int32), cu,
                                np.array([-1.0], np.float32), 0, K)):  # T = -1 sentinel
            assert r.num_accepted[0] == c["num_accepted"], c["cite"]
            toks = [t for t in r.tokens[0].tolist() if t >= 0]
            assert toks == c["tokens"], c["cite"]
            assert len(toks) == c["num_accepted"] + 1


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_brute_force_with_bf16_ties(seed):
    rng = np.random.default_rng(seed)
    B, V, max_k = 300, 257, 8
    ks = rng.integers(0, max_k + 1, size=B)
    cu = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    D, R = int(cu[-1]), int(cu[-1]) + B
    lg = torch.from_numpy(rng.standard_normal((R, V)).astype(np.float32) * 3).to(torch.bfloat16)
    rows = lg.float().numpy()
    # force exact ties at the maximum in a third of the rows (the higher index never wins)
    for r in range(0, R, 3):
        a, b = sorted(rng.choice(V, 2, replace=False))
        m = rows[r].max()
        rows[r, a] = rows[r, b] = m
    lg = torch.from_numpy(rows).to(torch.bfloat16)
    rows = lg.float().numpy()
    # drafts: the first-occurrence argmax, the last-occurrence argmax, or random
    drafts = np.empty(D, np.int32)
    for b in range(B):
        for j in range(ks[b]):
            row = rows[cu[b] + b + j]
            pick = rng.random()
            if pick < 0.6:
                drafts[cu[b] + j] = np.argmax(row)
            elif pick < 0.8:
                drafts[cu[b] + j] = V - 1 - np.argmax(row[::-1])
            else:
                drafts[cu[b] + j] = rng.integers(0, V)
    exp_out, exp_n = brute_force(rows, drafts, cu, max_k)
    r = oracle.verify_greedy(lg, drafts, cu, max_k)
    np.testing.assert_array_equal(r.num_accepted, exp_n)
    np.testing.assert_array_equal(r.tokens, exp_out)
    assert (r.flags == 0).all()
    # the same requests marked greedy inside a mixed call give the same answer
    T = np.where(np.arange(B) % 2 == 0, -1.0, 0.0).astype(np.float32)
    r2 = oracle.verify(lg, None, drafts, cu, T, 5, max_k)
    np.testing.assert_array_equal(r2.tokens, exp_out)
