"""Pins of the oracle's verify arithmetic against what the pages and the
mathematics fix (no reference implementation exists).

 - softmax p: scipy.special.softmax in fp64 (a library routine).
 - (1) output marginal = p exactly: chi-square on 10^6 trials at tiny V, with q
   present, q absent (one-hot) and T != 1  [Ch.12 "投机解码：以小博大" §12.2.2].
 - (2) acceptance probability = sum_y min(p, q)  [§12.2.2, the quantity A];
   accepted drafts follow min(p, q), rejected trials follow the residual
   max(0, p - q) / sum  [§12.2.1 step 3].
 - (3) tokens per step follow the truncated geometric law behind
   E[tokens] = (1 - A^(K+1)) / (1 - A)  [§12.5.1].
 - the exact joint law of (accepted prefix, emitted token) over two positions
   with distinct p_j, q_j (catches row / slot / position index mistakes).
 - special cases: q = p accepts everything; disjoint supports reject
   everything and still emit p; one-hot q accepts with probability p(x*);
   K = 0 is plain categorical sampling (the exponential race / Gumbel-max
   textbook case).
"""
import numpy as np
import pytest
from scipy import special, stats

import oracle

PVAL = 1e-3  # pre-registered threshold; every seed below is fixed


def _softmax(l, T=1.0):
    return special.softmax(np.asarray(l, np.float64) / T)


def _chi2_ok(counts, probs, min_expected=5.0):
    counts = np.asarray(counts, np.float64)
    exp = np.asarray(probs, np.float64) * counts.sum()
    keep = exp >= min_expected
    obs_k, exp_k = counts[keep], exp[keep]
    # fold the sparse cells into one so totals still match
    if (~keep).any():
        obs_k = np.append(obs_k, counts[~keep].sum())
        exp_k = np.append(exp_k, exp[~keep].sum())
    mask = exp_k > 0
    assert counts[exp == 0].sum() == 0, "mass observed where the law has none"
    if mask.sum() < 2:  # a one-cell law: nothing left to test once the rest is empty
        return 1.0
    return stats.chisquare(obs_k[mask], exp_k[mask] * obs_k[mask].sum() / exp_k[mask].sum()).pvalue


def _batch(row_logits, q_rows, drafts, T):
    """row_logits [B, K+1, V], q_rows [B, K, V] or None, drafts [B, K], T [B] -> oracle args."""
    B, K1, V = row_logits.shape
    K = K1 - 1
    cu = np.arange(B + 1, dtype=np.int32) * K
    lg = np.ascontiguousarray(row_logits.reshape(B * K1, V), np.float32)
    q = None if q_rows is None else np.ascontiguousarray(q_rows.reshape(B * K, V), np.float32)
    return lg, q, np.ascontiguousarray(drafts.reshape(-1), np.int32), cu, np.asarray(T, np.float32)


# ---------------------------------------------------------------- softmax
@pytest.mark.parametrize("V", [1, 7, 1000, 151936])
@pytest.mark.parametrize("T", [0.01, 0.3, 1.0, 7.5])
def test_softmax_matches_scipy(V, T):
    rng = np.random.default_rng(V)
    l = (rng.standard_normal(V) * 4).astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(oracle.softmax_row(l, T), _softmax(l, T), rtol=1e-12, atol=1e-300)


def test_probs_widen_bf16_exactly():
    import torch
    g = torch.Generator().manual_seed(3)
    lg = (torch.randn(6, 300, generator=g) * 3).to(torch.bfloat16)
    cu = torch.tensor([0, 2, 4], dtype=torch.int32)
    T = torch.tensor([0.7, -1.0])
    P = oracle.probs(lg, cu, T)
    for r in range(3):
        np.testing.assert_allclose(P[r], _softmax(lg[r].float().numpy(), np.float32(0.7)), rtol=1e-12)
    assert np.isnan(P[3:]).all()  # greedy request: no p


# ---------------------------------------------------- (1) + (2): one position
N_TRIALS = 1_000_000


def _one_position(V, T, q_mode, seed):
    rng = np.random.default_rng(seed)
    l0 = rng.standard_normal(V) * 1.5
    l1 = rng.standard_normal(V) * 1.5  # bonus row differs from the draft row
    p0, p1 = _softmax(l0.astype(np.float32), T), _softmax(l1.astype(np.float32), T)
    B = N_TRIALS
    rows = np.broadcast_to(np.stack([l0, l1]).astype(np.float32), (B, 2, V))
    if q_mode == "q":
        qv = _softmax(l0 + rng.standard_normal(V) * 1.2).astype(np.float32)
        qv /= qv.sum(dtype=np.float64)
        drafts = rng.choice(V, size=(B, 1), p=qv.astype(np.float64) / qv.sum(dtype=np.float64))
        qrows = np.broadcast_to(qv, (B, 1, V))
        qd = qv.astype(np.float64)
    else:  # one-hot q at a fixed draft token
        xs = int(np.argsort(p0)[V // 2])
        drafts = np.full((B, 1), xs)
        qrows = None
        qd = np.zeros(V)
        qd[xs] = 1.0
    lg, q, d, cu, Tb = _batch(rows, qrows, drafts, np.full(B, T))
    r = oracle.verify(lg, q, d, cu, Tb, seed=seed, max_k=1)
    return r, p0, p1, qd, drafts.reshape(-1)


@pytest.mark.slow
@pytest.mark.parametrize("V,T,q_mode,seed", [(8, 1.0, "q", 11), (16, 1.0, "q", 12), (8, 0.6, "q", 13),
                                              (16, 1.7, "onehot", 14), (8, 1.0, "onehot", 15)])
def test_marginal_is_p_and_acceptance_is_sum_min(V, T, q_mode, seed):
    r, p0, p1, qd, drafts = _one_position(V, T, q_mode, seed)
    assert (r.flags & oracle.FLAG_INVALID).sum() == 0
    first = r.tokens[:, 0]
    # (1) the first emitted token is distributed exactly as p  [§12.2.2]
    assert _chi2_ok(np.bincount(first, minlength=V), p0) > PVAL
    # (2) acceptance rate = A = sum min(p, q)  [§12.2.2]
    A = np.minimum(p0, qd).sum()
    acc = r.num_accepted == 1
    sd = np.sqrt(A * (1 - A) / acc.size)
    assert abs(acc.mean() - A) < 5 * sd + 1e-12
    # accepted drafts follow min(p, q) / A; rejected trials follow max(0, p - q) / (1 - A)
    if acc.any() and A < 1:
        assert _chi2_ok(np.bincount(drafts[acc], minlength=V), np.minimum(p0, qd) / A) > PVAL
        res = np.maximum(p0 - qd, 0)
        assert _chi2_ok(np.bincount(first[~acc], minlength=V), res / res.sum()) > PVAL
        # the bonus after an accepted draft follows p of the next row  [§12.3.2]
        assert _chi2_ok(np.bincount(r.tokens[acc, 1], minlength=V), p1) > PVAL
    # counts: n accepted -> n + 1 emitted tokens, -1 after  [§12.3.4]
    emitted = (r.tokens >= 0).sum(axis=1)
    np.testing.assert_array_equal(emitted, r.num_accepted + 1)


# ------------------------------------------------------ (3) truncated geometric
@pytest.mark.slow
@pytest.mark.parametrize("K", [1, 4, 8])
def test_tokens_per_step_truncated_geometric(K):
    V, B, T = 8, 200_000, 1.0
    rng = np.random.default_rng(100 + K)
    l = (rng.standard_normal(V) * 1.5).astype(np.float32)
    p = _softmax(l, T)
    qv = _softmax(l.astype(np.float64) + rng.standard_normal(V) * 0.9).astype(np.float32)
    qd = qv.astype(np.float64) / qv.sum(dtype=np.float64)
    A = np.minimum(p, qv.astype(np.float64)).sum()
    rows = np.broadcast_to(l, (B, K + 1, V))
    drafts = rng.choice(V, size=(B, K), p=qd)
    lg, q, d, cu, Tb = _batch(rows, np.broadcast_to(qv, (B, K, V)), drafts, np.full(B, T))
    r = oracle.verify(lg, q, d, cu, Tb, seed=K, max_k=K)
    n = r.num_accepted
    law = np.array([A**i * (1 - A) for i in range(K)] + [A**K])
    assert _chi2_ok(np.bincount(n, minlength=K + 1), law) > PVAL
    # E[tokens per step] = (1 - A^(K+1)) / (1 - A)  [§12.5.1]
    tokens = n + 1
    mean = (1 - A ** (K + 1)) / (1 - A)
    sd = tokens.std() / np.sqrt(B)
    assert abs(tokens.mean() - mean) < 5 * sd


# ------------------------------------------------------- exact joint law, K = 2
@pytest.mark.slow
def test_joint_law_two_positions():
    V, B, T, K = 4, 1_000_000, 0.9, 2
    rng = np.random.default_rng(7)
    L = (rng.standard_normal((K + 1, V)) * 1.2).astype(np.float32)
    P = np.stack([_softmax(L[j], T) for j in range(K + 1)])
    Q = np.stack([_softmax(L[j].astype(np.float64) / T + rng.standard_normal(V) * 1.0)
                  for j in range(K)]).astype(np.float32)
    Qd = Q.astype(np.float64)
    drafts = np.stack([rng.choice(V, size=B, p=Qd[j] / Qd[j].sum()) for j in range(K)], axis=1)
    lg, q, d, cu, Tb = _batch(np.broadcast_to(L, (B, K + 1, V)), np.broadcast_to(Q, (B, K, V)),
                              drafts, np.full(B, T))
    r = oracle.verify(lg, q, d, cu, Tb, seed=99, max_k=K)
    mn = [np.minimum(P[j], Qd[j]) for j in range(K)]
    res = [np.maximum(P[j] - Qd[j], 0) for j in range(K)]
    law, cell = [], {}
    for t in range(V):  # rejected at position 0
        cell[(t, -1, -1)] = len(law); law.append(res[0][t])
    for a in range(V):  # accepted a, rejected at position 1
        for t in range(V):
            cell[(a, t, -1)] = len(law); law.append(mn[0][a] * res[1][t])
    for a in range(V):  # both accepted, bonus from row 2
        for b in range(V):
            for t in range(V):
                cell[(a, b, t)] = len(law); law.append(mn[0][a] * mn[1][b] * P[2][t])
    law = np.array(law)
    assert abs(law.sum() - 1) < 1e-9
    idx = np.array([cell[tuple(row)] for row in r.tokens.tolist()])
    assert _chi2_ok(np.bincount(idx, minlength=law.size), law) > PVAL


# ---------------------------------------------------------------- special cases
def test_q_equal_p_accepts_everything():
    V, B, K, T = 16, 20000, 3, 1.3
    rng = np.random.default_rng(5)
    l = (rng.standard_normal(V) * 2).astype(np.float32)
    p = _softmax(l, T)
    qv = p.astype(np.float32)
    drafts = rng.choice(V, size=(B, K), p=qv.astype(np.float64) / qv.sum(dtype=np.float64))
    lg, q, d, cu, Tb = _batch(np.broadcast_to(l, (B, K + 1, V)), np.broadcast_to(qv, (B, K, V)), drafts, np.full(B, T))
    r = oracle.verify(lg, q, d, cu, Tb, seed=1, max_k=K)
    assert (r.num_accepted == K).all()
    assert _chi2_ok(np.bincount(r.tokens[:, K], minlength=V), p) > PVAL


def test_disjoint_supports_reject_and_still_emit_p():
    V, B, T = 8, 100000, 1.0
    l = np.array([0.5, -0.3, 1.1, 0.0, -1e4, -1e4, -1e4, -1e4], np.float32)
    p = _softmax(l, T)
    assert (p[4:] == 0).all()
    qv = np.array([0, 0, 0, 0, 0.1, 0.2, 0.3, 0.4], np.float32)
    rng = np.random.default_rng(8)
    drafts = rng.choice(V, size=(B, 1), p=qv.astype(np.float64) / qv.sum(dtype=np.float64))
    lg, q, d, cu, Tb = _batch(np.broadcast_to(l, (B, 2, V)), np.broadcast_to(qv, (B, 1, V)), drafts, np.full(B, T))
    r = oracle.verify(lg, q, d, cu, Tb, seed=2, max_k=1)
    assert (r.num_accepted == 0).all()
    assert _chi2_ok(np.bincount(r.tokens[:, 0], minlength=V), p) > PVAL


def test_zero_drafts_is_categorical_sampling():
    V, B, T = 12, 300000, 0.8
    rng = np.random.default_rng(9)
    l = (rng.standard_normal(V) * 1.5).astype(np.float32)
    lg = np.ascontiguousarray(np.broadcast_to(l, (B, V)), np.float32)
    cu = np.zeros(B + 1, np.int32)
    r = oracle.verify(lg, None, np.zeros(0, np.int32), cu, np.full(B, T, np.float32), seed=3, max_k=0)
    assert (r.num_accepted == 0).all()
    assert _chi2_ok(np.bincount(r.tokens[:, 0], minlength=V), _softmax(l, T)) > PVAL


def test_invalid_metadata_emits_minus_one():
    V = 10
    lg = np.zeros((5, V), np.float32)
    cu = np.array([0, 2, 4], np.int32)          # B = 2, D = 4? rows = D + B = 6 != 5
    with pytest.raises(ValueError):
        oracle.verify(lg, None, np.zeros(4, np.int32), cu, np.ones(2, np.float32), 0, 2)
    lg = np.zeros((6, V), np.float32)
    d = np.array([1, 2, 3, 99], np.int32)      # request 1 has an out-of-range draft
    r = oracle.verify(lg, None, d, cu, np.ones(2, np.float32), 0, 2)
    assert r.flags[1] & oracle.FLAG_INVALID and r.num_accepted[1] == -1 and (r.tokens[1] == -1).all()
    assert r.num_accepted[0] >= 0
    r = oracle.verify(lg, None, np.array([1, 2, 3, 4], np.int32), cu, np.ones(2, np.float32), 0, 1)
    assert (r.flags & oracle.FLAG_INVALID).all()  # K_b = 2 > max_k = 1


# ------------------------------------------------------------- near-tie flags
def test_accept_test_near_tie_flag():
    """|p(x*) - u q(x*)| <= eps p(x*) flags the request; a wider margin does not."""
    V, seed = 4, 31
    l = np.array([0.3, -0.2, 0.9, 0.1], np.float32)
    p = _softmax(l, 1.0)
    u = oracle.accept_uniforms(seed, [0], [0])[0]
    assert u > 0
    for rel, flagged in ((3e-7, True), (-3e-7, True), (5e-6, False), (-5e-6, False)):
        qs = np.float32(p[2] / u * (1 + rel))
        qrow = np.full(V, 0.01, np.float32)
        qrow[2] = qs
        realised = u * float(qs) / p[2] - 1  # margin after fp32 rounding of q
        lg = np.ascontiguousarray(np.stack([l, l]), np.float32)
        r = oracle.verify(lg, qrow[None, :], np.array([2], np.int32), np.array([0, 1], np.int32),
                          np.array([1.0], np.float32), seed, 1)
        assert bool(r.flags[0] & oracle.FLAG_ACCEPT_TIE) == (abs(realised) <= 1e-6)
        assert bool(r.flags[0] & oracle.FLAG_ACCEPT_TIE) == flagged
        assert r.num_accepted[0] == (1 if realised < 0 else 0)


def test_race_near_tie_flag():
    """Bonus race (K = 0): two keys p_x / E_x within ~1e-7 are flagged, 1e-3 apart are not."""
    seed, V = 41, 4
    E = oracle.race_exponentials(seed, 0, 0, 0, V)
    for delta, flagged in ((1e-7, True), (1e-3, False)):
        l = np.array([0.0, np.log(E[1] / E[0]) + delta, -30.0, -30.0], np.float64)
        lg = l.astype(np.float32)[None, :]
        r = oracle.verify(lg, None, np.zeros(0, np.int32), np.array([0, 0], np.int32),
                          np.array([1.0], np.float32), seed, 0)
        assert bool(r.flags[0] & oracle.FLAG_RACE_TIE) == flagged
        assert r.tokens[0, 0] in (0, 1)


# ------------------------------------------------------- all-zero residual
def _zero_residual_batch(V, B, seed, q_of_p, T=1.0):
    """K = 1 per request, all requests sharing one draft row and one bonus row;
    q = q_of_p(p0) (fp32, not normalised), drafts drawn from p0."""
    rng = np.random.default_rng(seed)
    l0 = (rng.standard_normal(V) * 1.5).astype(np.float32)
    l1 = (rng.standard_normal(V) * 1.5).astype(np.float32)
    p0, p1 = _softmax(l0, T), _softmax(l1, T)
    qv = np.asarray(q_of_p(p0), np.float32)
    drafts = rng.choice(V, size=(B, 1), p=p0)
    lg, q, d, cu, Tb = _batch(np.broadcast_to(np.stack([l0, l1]), (B, 2, V)), np.broadcast_to(qv, (B, 1, V)),
                              drafts, np.full(B, T))
    return oracle.verify(lg, q, d, cu, Tb, seed=seed, max_k=1), p0, p1, qv, drafts.reshape(-1)


@pytest.mark.slow
def test_zero_residual_q_twice_p_falls_back_to_p():
    """q = 2p is not normalised; the library takes q as given (q >= 0 only).
    The accept test u * 2p(x*) < p(x*) holds iff u < 1/2, so exactly half of
    the drafts are accepted, whatever x*.  At a rejection max(0, p - q) is zero
    everywhere and the residual of [Ch.12 §12.2.1 step 3] is undefined; the
    reading races over p at the same position.  So: every rejected request,
    and no other, carries FLAG_ZERO_RESIDUAL; the fallback is exact (no near
    tie); the rejected trials' token follows p; the bonus follows the next
    row's p; the first emitted token follows p overall."""
    V, B = 8, N_TRIALS
    r, p0, p1, qv, drafts = _zero_residual_batch(V, B, 23, lambda p: 2.0 * p)
    rej = r.num_accepted == 0
    assert abs(rej.mean() - 0.5) < 5 * 0.5 / np.sqrt(B)
    zr = (r.flags & oracle.FLAG_ZERO_RESIDUAL) != 0
    np.testing.assert_array_equal(zr, rej)
    # near ties only from accept coins next to u = 1/2
    # (|1 - 2u| <= 1e-6: a few grid points of 2^-24), or from genuine near ties
    # of the fallback race's top two keys p / E
    assert r.near_tie.sum() <= 10
    for b in np.nonzero(r.near_tie)[0]:
        if r.flags[b] & oracle.FLAG_RACE_TIE:
            keys = np.sort(p0 / oracle.race_exponentials(23, int(b), 0, 0, V))
            assert keys[-1] - keys[-2] <= 3e-6 * keys[-1]
    assert _chi2_ok(np.bincount(r.tokens[rej, 0], minlength=V), p0) > PVAL
    assert _chi2_ok(np.bincount(r.tokens[~rej, 1], minlength=V), p1) > PVAL
    assert _chi2_ok(np.bincount(r.tokens[:, 0], minlength=V), p0) > PVAL
    # the fallback's token is the race over p with the position's exponentials:
    # recompute one rejected request's winner from the race definition
    b = int(np.nonzero(rej)[0][0])
    E = oracle.race_exponentials(23, b, 0, 0, V)
    assert r.tokens[b, 0] == int(np.argmax(p0 / E))
    assert r.cand[b, 0] == r.tokens[b, 0] and (r.cand[b, 1:] == -1).all()


def test_zero_residual_fragile_is_a_race_near_tie():
    """q(x*) = 2p(x*) (rejections), every other q(x) = p(x)(1 + 3e-7): the
    residual is zero everywhere, but p(1 + 1e-6) - q > 0 for the other tokens,
    so a perturbed p would race over them instead of falling back: the
    request is a race near tie, and its candidates hold the fallback winner
    and every token whose residual could be positive."""
    V, B = 8, 4000

    def q_of_p(p):
        q = (p * (1 + 3e-7)).astype(np.float32)
        assert (q.astype(np.float64) > p).all() and (q.astype(np.float64) < p * (1 + 1e-6)).all()
        return q

    rng = np.random.default_rng(5)
    l0 = (rng.standard_normal(V) * 1.5).astype(np.float32)
    l1 = (rng.standard_normal(V) * 1.5).astype(np.float32)
    p0 = _softmax(l0)
    xs = int(np.argmax(p0))
    qv = q_of_p(p0)
    qv[xs] = np.float32(2 * p0[xs])
    drafts = np.full((B, 1), xs)
    lg, q, d, cu, Tb = _batch(np.broadcast_to(np.stack([l0, l1]), (B, 2, V)), np.broadcast_to(qv, (B, 1, V)),
                              drafts, np.full(B, 1.0))
    r = oracle.verify(lg, q, d, cu, Tb, seed=7, max_k=1)
    rej = r.num_accepted == 0
    assert 0.4 < rej.mean() < 0.6
    fl = r.flags[rej]
    assert ((fl & oracle.FLAG_ZERO_RESIDUAL) != 0).all() and ((fl & oracle.FLAG_RACE_TIE) != 0).all()
    others = [x for x in range(V) if x != xs]
    for b in np.nonzero(rej)[0][:50]:
        c = set(int(x) for x in r.cand[b] if x >= 0)
        assert int(r.tokens[b, 0]) in c and set(others) <= c
    assert (r.flags[~rej] & oracle.FLAG_ZERO_RESIDUAL == 0).all()


def test_zero_residual_fragile_winner_is_a_race_near_tie():
    """One token keeps a residual of 3e-7 p (q just below p) and wins the race
    alone; under the perturbation that residual vanishes and the fallback
    would race over p, so the request is a race near tie whose candidates hold
    both winners; a residual of 1e-3 p is not."""
    V, B = 8, 2000
    rng = np.random.default_rng(9)
    l0 = (rng.standard_normal(V) * 1.5).astype(np.float32)
    l1 = (rng.standard_normal(V) * 1.5).astype(np.float32)
    p0 = _softmax(l0)
    order = np.argsort(p0)
    xs, keep = int(order[-1]), int(order[0])
    for rel, fragile in ((3e-7, True), (1e-3, False)):
        qv = (2 * p0).astype(np.float32)
        qv[keep] = np.float32(p0[keep] * (1 - rel))
        assert qv[keep] < p0[keep]
        drafts = np.full((B, 1), xs)
        lg, q, d, cu, Tb = _batch(np.broadcast_to(np.stack([l0, l1]), (B, 2, V)), np.broadcast_to(qv, (B, 1, V)),
                                  drafts, np.full(B, 1.0))
        r = oracle.verify(lg, q, d, cu, Tb, seed=11, max_k=1)
        rej = r.num_accepted == 0
        assert rej.any()
        assert (r.tokens[rej, 0] == keep).all()  # the only positive residual
        assert not (r.flags[rej] & oracle.FLAG_ZERO_RESIDUAL).any()
        tie = (r.flags[rej] & oracle.FLAG_RACE_TIE) != 0
        assert tie.all() if fragile else not tie.any()
        if fragile:
            for b in np.nonzero(rej)[0][:50]:
                E = oracle.race_exponentials(11, int(b), 0, 0, V)
                fb = int(np.argmax(p0 / E))
                assert keep in r.cand[b] and fb in r.cand[b]
