"""Pins of the n-gram proposer oracle (oracle/ngram.py) [第12章 投机解码：以小博大
§12.4.4]:
 - the worked example the pages print (tests/golden/ngram_worked_example.json);
 - the leftmost occurrence against a library search (bytes.find on a
   fixed-width encoding of the tokens, aligned hits only);
 - longer n first, k capped by max_model_len, short contexts, no match.
"""
import json
import os

import numpy as np
import pytest

from oracle import ngram

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ngram_worked_example.json")


def test_worked_example():
    g = json.load(open(GOLDEN))
    assert ngram.propose(g["context"], g["min_n"], g["max_n"], g["k"], 1 << 30) == g["expected"]


def _enc(seq):
    return np.asarray(seq, dtype=">u4").tobytes()


def _library_propose(ctx, min_n, max_n, k, max_model_len):
    N = len(ctx)
    k_eff = min(k, max_model_len - N)
    if k_eff <= 0:
        return []
    hay_all = _enc(ctx)
    for n in range(max_n, min_n - 1, -1):
        if 2 * n > N:
            continue
        hay = hay_all[: 4 * (N - n)]  # occurrences must end before the pattern starts
        needle = _enc(ctx[N - n:])
        pos = hay.find(needle)
        while pos != -1 and pos % 4:
            pos = hay.find(needle, pos + 1)
        if pos != -1:
            s = pos // 4
            return list(ctx[s + n: s + n + k_eff])
    return []


@pytest.mark.parametrize("seed", range(20))
def test_against_library_search(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 400))
    vocab = int(rng.choice([3, 5, 20, 1000]))
    ctx = rng.integers(0, vocab, size=N).tolist()
    if N > 30 and seed % 2:  # plant a repeat of the tail
        L = int(rng.integers(2, 9))
        s = int(rng.integers(0, N - 2 * L))
        ctx[s:s + L] = ctx[N - L:]
    for (mn, mx, k, mml) in ((1, 3, 5, 1 << 30), (2, 8, 4, 1 << 30), (3, 5, 10, N + 3), (4, 4, 2, N)):
        assert ngram.propose(ctx, mn, mx, k, mml) == _library_propose(ctx, mn, mx, k, mml), (seed, mn, mx, k)


def test_longer_pattern_wins_and_edges():
    ctx = [7, 8, 9, 1, 8, 9, 2, 7, 8, 9]
    # the 3-gram [7,8,9] occurs at 0 -> [1, 8, 9]; the 2-gram would have given [1, 8]
    assert ngram.propose(ctx, 2, 3, 3, 1 << 30) == [1, 8, 9]
    assert ngram.propose(ctx, 2, 2, 3, 1 << 30) == [1, 8, 9]  # [8,9] leftmost at 1
    assert ngram.propose(ctx, 2, 3, 3, len(ctx) + 1) == [1]  # k capped by max_model_len
    assert ngram.propose(ctx, 2, 3, 3, len(ctx)) == []
    assert ngram.propose([1, 2, 3], 2, 3, 3, 100) == []      # context shorter than 2n
    assert ngram.propose([5, 5], 1, 1, 3, 100) == [5]         # [5] at 0, the rest of the context
    assert ngram.propose([1, 2, 3, 4], 1, 2, 3, 100) == []    # no match
