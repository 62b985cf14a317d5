"""Pins of the acceptance statistics oracle (oracle/stats.py).

 - the worked example the pages print [投机解码（Speculative Decoding）端到端深挖
   §13]: K=4, 10 verifies, 25 accepted, 35 completion tokens -> alpha = 0.625,
   tau = 3.5, realised by a concrete sequence of 10 accept counts summing to 25;
 - per-position counts are the survival function of the accept counts
   [第12章 投机解码：以小博大 §12.7.5]: their sum is the accepted total, they
   never increase with the position, and position 0 counts the verifies with
   at least one acceptance;
 - the emitted tokens per step follow the oracle's verify output (n + 1
   tokens per request [§12.3.4]) on a real batch;
 - chain law: with i.i.d. acceptance probability A the mean accept length
   matches (1 - A^(K+1)) / (1 - A) [第12章 §12.5.1] (statistical, through the
   verify oracle).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import stats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_stats_worked_example.json")


def test_worked_example():
    g = json.load(open(GOLDEN))
    K, V = g["K"], g["verifies"]
    accepted = [4, 3, 2, 1, 0, 4, 4, 3, 2, 2]  # any 10 counts in [0, K] that sum to 25
    assert sum(accepted) == g["accepted_total"]
    c = None
    for n in accepted:  # one request per verify step
        c = stats.accumulate(c, [n], [0, K])
    assert c["num_verifies"] == V
    assert c["num_draft_tokens"] == V * K
    assert c["num_emitted_tokens"] == g["completion_tokens"]
    assert stats.accept_rate(c) == pytest.approx(g["accept_rate"], abs=0)
    assert stats.accept_length(c) == pytest.approx(g["accept_length"], abs=0)
    assert c["num_drafts"] == V


def test_per_position_is_survival_function():
    rng = np.random.default_rng(1)
    B, K = 300, 7
    n = rng.integers(0, K + 1, size=B)
    cu = np.arange(B + 1) * K
    c = stats.accumulate(None, n, cu)
    pp = np.array(c["accepted_per_pos"])
    assert pp.sum() == n.sum() == c["num_accepted_tokens"]
    assert np.all(np.diff(pp) <= 0)
    assert pp[0] == (n >= 1).sum()
    for j in range(K):
        assert pp[j] == (n > j).sum()
    assert np.all(pp[K:] == 0)


def test_ragged_invalid_and_zero_draft_requests():
    n = [2, -1, 0, 1, 0]
    cu = [0, 3, 5, 5, 6, 6]  # K = 3, 2, 0, 1, 0
    c = stats.accumulate(None, n, cu)
    assert c["num_verifies"] == 4            # the invalid request is skipped
    assert c["num_drafts"] == 2              # requests 0 and 3 proposed drafts (2 and 4 have none)
    assert c["num_draft_tokens"] == 3 + 0 + 1 + 0
    assert c["num_accepted_tokens"] == 3
    assert c["num_emitted_tokens"] == 3 + 4
    assert c["accepted_per_pos"][:3] == [2, 1, 0]


def test_accumulates_across_steps():
    c = stats.accumulate(None, [1, 2], [0, 2, 4])
    c = stats.accumulate(c, [0], [0, 3])
    assert c["num_verifies"] == 3 and c["num_draft_tokens"] == 7 and c["num_accepted_tokens"] == 3
    assert stats.to_array(c).shape == (5 + stats.MAX_POS,)


@pytest.mark.slow
def test_accept_length_chain_law():
    from scipy import special
    V, B, K, T = 8, 200_000, 4, 1.0
    rng = np.random.default_rng(77)
    l = (rng.standard_normal(V) * 1.5).astype(np.float32)
    p = special.softmax(l.astype(np.float64) / T)
    qv = special.softmax(l.astype(np.float64) + rng.standard_normal(V) * 0.8).astype(np.float32)
    qd = qv.astype(np.float64) / qv.sum(dtype=np.float64)
    A = np.minimum(p, qv.astype(np.float64)).sum()
    rows = np.ascontiguousarray(np.broadcast_to(l, (B, K + 1, V)).reshape(B * (K + 1), V))
    drafts = rng.choice(V, size=B * K, p=qd).astype(np.int32)
    q = np.ascontiguousarray(np.broadcast_to(qv, (B * K, V)))
    cu = np.arange(B + 1, dtype=np.int32) * K
    r = oracle.verify(rows, q, drafts, cu, np.full(B, T, np.float32), 5, K)
    c = stats.accumulate(None, r.num_accepted, cu)
    emitted = (r.tokens >= 0).sum(axis=1)
    assert c["num_emitted_tokens"] == emitted.sum()
    tau = stats.accept_length(c)
    assert abs(tau - (1 - A ** (K + 1)) / (1 - A)) < 5 * emitted.std() / np.sqrt(B)
