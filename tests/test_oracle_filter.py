"""Pins of the oracle's top-k / top-p filtering of the target distribution
[Ch.12 "投机解码：以小博大" §12.2.3 (temperature, top-k and top-p constrain the
target distribution of rejection sampling); §12.9 (compute_probs applies them
per token)].  The pages fix that the target distribution is filtered before
the accept test, the residual and the bonus; they do not print the filter's
tie rules, so the oracle's reading (strictly-larger counts and masses, ties
kept together) is pinned against independent constructions:

 - top-k against torch.topk (a library selection) on rows without ties;
 - top-p against the sort-ascending / cumulative-sum construction (drop the
   tokens whose ascending cumulative probability is at most 1 - top_p), which
   coincides with the reading on rows without ties;
 - hand-derived tie cases, the degenerate settings (k = 1, top_p -> 0,
   filters off) and the renormalisation;
 - the output law: with a filtered target p' the emitted token follows p'
   exactly and the acceptance rate is sum min(p', q) (chi-square, 10^6 trials),
   which is the proof of §12.2.2 with p' as the target.
"""
import numpy as np
import pytest
import torch
from scipy import special, stats

import oracle

PVAL = 1e-3


def _support(p):
    return set(np.flatnonzero(p > 0).tolist())


@pytest.mark.parametrize("seed", range(8))
def test_top_k_matches_torch_topk(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(5, 300))
    l = rng.permutation(V).astype(np.float64) * 0.37 - 20.0  # distinct values
    T = float(rng.uniform(0.3, 2.0))
    for k in sorted({1, 2, 3, V // 2, V - 1}):
        p, tie = oracle.filtered_probs_row(l, T, top_k=k)
        want = set(torch.topk(torch.tensor(l), k).indices.tolist())
        assert _support(p) == want, (V, k)
        assert not tie


@pytest.mark.parametrize("seed", range(8))
def test_top_p_matches_ascending_cumsum(seed):
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(5, 400))
    l = rng.standard_normal(V) * float(rng.uniform(0.5, 4.0))
    T = float(rng.uniform(0.3, 1.5))
    probs = special.softmax(l / T)
    for top_p in (0.05, 0.3, 0.5, 0.8, 0.9, 0.95, 0.999):
        order = np.argsort(probs)  # ascending
        csum = np.cumsum(probs[order])
        if np.min(np.abs(csum - (1.0 - top_p))) < 1e-9:
            continue  # a boundary within rounding: not a pin
        keep = set(order[csum > 1.0 - top_p].tolist())
        p, _ = oracle.filtered_probs_row(l, T, top_p=top_p)
        assert _support(p) == keep, (V, top_p)


def test_top_k_then_top_p_order():
    # top-p is taken on the top-k-renormalised distribution
    rng = np.random.default_rng(5)
    V = 200
    l = rng.permutation(V).astype(np.float64) * 0.05
    T, k, top_p = 0.7, 20, 0.6
    topk = torch.topk(torch.tensor(l), k).indices.numpy()
    pk = np.zeros(V)
    pk[topk] = special.softmax(l[topk] / T)
    order = np.argsort(pk)
    csum = np.cumsum(pk[order])
    keep = set(order[(csum > 1.0 - top_p) & (pk[order] > 0)].tolist())
    p, _ = oracle.filtered_probs_row(l, T, top_k=k, top_p=top_p)
    assert _support(p) == keep


def test_ties_are_kept_together():
    l = np.array([5.0, 4.0, 4.0, 4.0, 1.0, 4.0, 0.0])
    # top-k = 2: the k-th largest value is 4, every 4 stays
    p, _ = oracle.filtered_probs_row(l, 1.0, top_k=2)
    assert _support(p) == {0, 1, 2, 3, 5}
    # top-p just above the mass of the maximum: the whole group of 4s stays
    w = np.exp(l - 5.0)
    pmax = w[0] / w.sum()
    p, _ = oracle.filtered_probs_row(l, 1.0, top_p=pmax * 1.01)
    assert _support(p) == {0, 1, 2, 3, 5}
    # top-p at or below the mass of the maximum keeps the maximum only
    p, _ = oracle.filtered_probs_row(l, 1.0, top_p=pmax * 0.99)
    assert _support(p) == {0}


def test_signed_zeros_are_one_value():
    # -0 and +0 are the same logit: a threshold among zeros keeps both signs,
    # and the result equals that of the row with every zero positive
    l = np.array([2.0, 0.0, -0.0, 0.0, -0.0, -0.0, -3.0, 1.0])
    pos = l + 0.0  # the same values, no negative zero (-0 + +0 = +0)
    assert np.signbit(l).sum() == 4 and np.signbit(pos).sum() == 1
    for k, tp in ((3, 1.0), (4, 1.0), (0, 0.7), (0, 0.9), (5, 0.8)):
        p, _ = oracle.filtered_probs_row(l, 1.0, top_k=k, top_p=tp)
        q, _ = oracle.filtered_probs_row(pos, 1.0, top_k=k, top_p=tp)
        np.testing.assert_array_equal(p, q)
        assert _support(p) >= {1, 2, 3, 4, 5}  # every zero kept


def test_degenerate_settings():
    rng = np.random.default_rng(9)
    l = rng.standard_normal(50) * 3
    T = 0.8
    full = special.softmax(l / T)
    for k, tp in ((0, 1.0), (50, 1.0), (-3, 1.0), (0, 0.0), (0, 1.5), (60, -1.0)):
        p, _ = oracle.filtered_probs_row(l, T, top_k=k, top_p=tp)
        np.testing.assert_allclose(p, full, rtol=1e-12)
    for k, tp in ((1, 1.0), (0, 1e-6), (1, 0.5)):
        p, _ = oracle.filtered_probs_row(l, T, top_k=k, top_p=tp)
        want = np.zeros(50)
        want[np.argmax(l)] = 1.0
        np.testing.assert_array_equal(p, want)


@pytest.mark.parametrize("seed", range(4))
def test_renormalised_on_support(seed):
    rng = np.random.default_rng(40 + seed)
    l = rng.standard_normal(1000) * 2
    T = 1.1
    p, _ = oracle.filtered_probs_row(l, T, top_k=300, top_p=0.7)
    full = special.softmax(l / T)
    s = p > 0
    assert abs(p.sum() - 1) < 1e-12
    np.testing.assert_allclose(p[s], full[s] / full[s].sum(), rtol=1e-12)


def test_top_p_near_tie_flag():
    l = np.array([2.0, 1.0, 0.0, -1.0])
    w = np.exp(l)
    m0 = w[0] / w.sum()
    _, tie = oracle.filtered_probs_row(l, 1.0, top_p=m0 * (1 + 1e-9))
    assert tie
    _, tie = oracle.filtered_probs_row(l, 1.0, top_p=m0 * (1 + 1e-3))
    assert not tie


def _chi2(counts, probs):
    counts = np.asarray(counts, np.float64)
    exp = np.asarray(probs, np.float64) * counts.sum()
    assert counts[exp == 0].sum() == 0, "mass observed where the law has none"
    keep = exp >= 5
    obs, ex = counts[keep], exp[keep]
    if (~keep).any():
        obs = np.append(obs, counts[~keep].sum())
        ex = np.append(ex, exp[~keep].sum())
    m = ex > 0
    if m.sum() < 2:
        return 1.0
    return stats.chisquare(obs[m], ex[m] * obs[m].sum() / ex[m].sum()).pvalue


@pytest.mark.slow
@pytest.mark.parametrize("V,T,k,tp,q_mode,seed", [(16, 1.0, 6, 1.0, "q", 1), (16, 0.8, 0, 0.8, "q", 2),
                                                  (12, 1.3, 8, 0.9, "q", 3), (16, 1.0, 5, 0.85, "onehot", 4)])
def test_filtered_output_law(V, T, k, tp, q_mode, seed):
    """The emitted token follows p' exactly; acceptance = sum min(p', q)."""
    rng = np.random.default_rng(seed)
    B = 1_000_000
    l0 = (rng.standard_normal(V) * 1.5).astype(np.float32)
    l1 = (rng.standard_normal(V) * 1.5).astype(np.float32)
    p0, _ = oracle.filtered_probs_row(l0.astype(np.float64), np.float32(T), top_k=k, top_p=tp)
    p1, _ = oracle.filtered_probs_row(l1.astype(np.float64), np.float32(T), top_k=k, top_p=tp)
    rows = np.ascontiguousarray(np.broadcast_to(np.stack([l0, l1]), (B, 2, V)).reshape(2 * B, V))
    cu = np.arange(B + 1, dtype=np.int32)
    if q_mode == "q":
        qv = special.softmax(l0.astype(np.float64) + rng.standard_normal(V)).astype(np.float32)
        qd = qv.astype(np.float64) / qv.sum(dtype=np.float64)
        drafts = rng.choice(V, size=B, p=qd).astype(np.int32)
        q = np.ascontiguousarray(np.broadcast_to(qv, (B, V)))
        qd = qv.astype(np.float64)
    else:
        xs = int(np.argsort(p0)[-2])  # a kept token that is not the only one
        drafts = np.full(B, xs, np.int32)
        q = None
        qd = np.zeros(V)
        qd[xs] = 1.0
    r = oracle.verify(rows, q, drafts, cu, np.full(B, T, np.float32), seed=seed, max_k=1,
                      top_k=np.full(B, k, np.int32), top_p=np.full(B, tp, np.float32))
    assert r.near_tie.mean() < 1e-4  # accept-test ties at ~1e-6 per decision
    first = r.tokens[:, 0]
    assert _chi2(np.bincount(first, minlength=V), p0) > PVAL
    A = np.minimum(p0, qd).sum()
    acc = r.num_accepted == 1
    assert abs(acc.mean() - A) < 5 * np.sqrt(A * (1 - A) / B) + 1e-12
    if acc.any():
        assert _chi2(np.bincount(r.tokens[acc, 1], minlength=V), p1) > PVAL


def test_greedy_ignores_filters():
    rng = np.random.default_rng(3)
    V, B, K = 40, 6, 3
    lg = (rng.standard_normal((B * (K + 1), V)) * 2).astype(np.float32)
    cu = np.arange(B + 1, dtype=np.int32) * K
    drafts = rng.integers(0, V, size=B * K).astype(np.int32)
    T = np.full(B, -1.0, np.float32)
    a = oracle.verify(lg, None, drafts, cu, T, 1, K)
    b = oracle.verify(lg, None, drafts, cu, T, 1, K, top_k=np.full(B, 1, np.int32),
                      top_p=np.full(B, 0.1, np.float32))
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.num_accepted, b.num_accepted)


def test_filters_off_match_unfiltered_verify():
    rng = np.random.default_rng(4)
    V, B, K = 300, 20, 4
    lg = (rng.standard_normal((B * (K + 1), V)) * 3).astype(np.float32)
    cu = np.arange(B + 1, dtype=np.int32) * K
    q = special.softmax(rng.standard_normal((B * K, V)), axis=1).astype(np.float32)
    drafts = np.array([rng.choice(V, p=q[i].astype(np.float64) / q[i].sum(dtype=np.float64))
                       for i in range(B * K)], np.int32)
    T = rng.uniform(0.5, 1.5, B).astype(np.float32)
    a = oracle.verify(lg, q, drafts, cu, T, 8, K)
    b = oracle.verify(lg, q, drafts, cu, T, 8, K, top_k=np.zeros(B, np.int32), top_p=np.ones(B, np.float32))
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.num_accepted, b.num_accepted)
