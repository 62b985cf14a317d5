"""Pins of the oracle's tree verify (rso_verify_tree) [投机解码深度实战 §四;
投机解码（Speculative Decoding）端到端深挖 §6.2, §7.1, §7.2]:

 - the greedy walks the pages draw (tests/golden/tree_worked_examples.json);
 - a one-child-per-node tree is the chain: tokens and counts equal the chain
   oracle with one-hot q (same random numbers), greedy and random;
 - exact law of one layer: with siblings s_1..s_m the walk accepts s_i with
   probability p(s_i) and otherwise emits the residual p without the
   siblings, so the first emitted token follows p (chi-square, 10^6 trials);
   after accepting s_i the bonus follows that node's row; a repeated sibling
   token is skipped and the law still holds;
 - greedy against brute force (numpy argmax walk) on random trees;
 - invalid trees (parent after its child, token out of range, too deep).
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle
import rs_workloads as W

PVAL = 1e-3
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_worked_examples.json")


def _rows_from_argmax(argmax, V=8):
    rows = np.zeros((len(argmax), V), np.float32)
    for r, a in enumerate(argmax):
        rows[r, a] = 5.0
    return rows


def test_greedy_worked_examples():
    for c in json.load(open(GOLDEN))["cases"]:
        lg = _rows_from_argmax(c["argmax"])
        n = len(c["tokens"])
        r = oracle.verify_tree(lg, np.array(c["tokens"], np.int32), np.array(c["parents"], np.int32),
                               np.array([0, n], np.int32), np.array([0.0], np.float32), 0, n, 3)
        assert r.num_accepted[0] == c["num_accepted"], c["cite"]
        k = c["num_accepted"]
        assert r.path[0, :k].tolist() == c["path"]
        assert r.tokens[0, :k + 1].tolist() == c["out"]
        assert (r.tokens[0, k + 1:] == -1).all() and (r.path[0, k:] == -1).all()


@pytest.mark.parametrize("temp", [0.0, 1.0, 0.7])
def test_chain_tree_is_the_chain(temp):
    w = W.make([4, 0, 6, 3, 8, 1, 5, 2] * 3, 500, dtype="float32" and __import__("torch").float32,
               temperature=temp, q_mode="none", draft_mode="argmax_mix", seed=11, gen_seed=77)
    ks = w.num_draft
    parents = np.concatenate([np.arange(k) - 1 for k in ks]).astype(np.int32)
    chain = oracle.verify(w.logits, None, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature, w.seed, w.max_k)
    tree = oracle.verify_tree(w.logits, w.draft_token_ids, parents, w.cu_num_draft_tokens, w.temperature, w.seed,
                              w.max_k, w.max_k)
    np.testing.assert_array_equal(tree.num_accepted, chain.num_accepted)
    np.testing.assert_array_equal(tree.tokens, chain.tokens)
    for b, k in enumerate(ks):
        n = tree.num_accepted[b]
        assert tree.path[b, :n].tolist() == list(range(n))


def _chi2(counts, probs):
    counts = np.asarray(counts, np.float64)
    exp = np.asarray(probs, np.float64) * counts.sum()
    assert counts[exp == 0].sum() == 0
    keep = exp >= 5
    small = (exp > 0) & ~keep  # lumped into one bin; impossible outcomes (checked empty above) are left out
    obs, ex = counts[keep], exp[keep]
    if small.any():
        obs, ex = np.append(obs, counts[small].sum()), np.append(ex, exp[small].sum())
    return stats.chisquare(obs, ex * obs.sum() / ex.sum()).pvalue


@pytest.mark.slow
@pytest.mark.parametrize("sib_tokens,T", [([5, 2, 7], 1.0), ([1, 6], 0.6), ([3, 3, 0], 1.3)])
def test_one_layer_exact_law(sib_tokens, T):
    V, B = 8, 1_000_000
    rng = np.random.default_rng(sum(sib_tokens))
    m = len(sib_tokens)
    L = (rng.standard_normal((1 + m, V)) * 1.3).astype(np.float32)  # root row, then one row per sibling
    p = special.softmax(L[0].astype(np.float64) / np.float32(T))
    lg = np.ascontiguousarray(np.broadcast_to(L, (B, 1 + m, V)).reshape(B * (1 + m), V))
    tokens = np.tile(np.array(sib_tokens, np.int32), B)
    parents = np.full(B * m, -1, np.int32)
    cu = (np.arange(B + 1) * m).astype(np.int32)
    r = oracle.verify_tree(lg, tokens, parents, cu, np.full(B, T, np.float32), 123, m, 2)
    assert r.near_tie.mean() < 1e-4
    first = r.tokens[:, 0]
    assert _chi2(np.bincount(first, minlength=V), p) > PVAL
    distinct = []
    for t in sib_tokens:
        if t not in distinct:
            distinct.append(t)
    acc = r.num_accepted == 1
    # sibling i is accepted with probability p(its token); a repeat is never taken
    node_of = {t: sib_tokens.index(t) for t in distinct}
    counts = [int((acc & (r.path[:, 0] == node_of[t])).sum()) for t in distinct] + [int((~acc).sum())]
    law = [p[t] for t in distinct] + [1 - sum(p[t] for t in distinct)]
    assert _chi2(counts, law) > PVAL
    # the bonus after accepting sibling i follows that node's row
    for t in distinct:
        i = node_of[t]
        sel = acc & (r.path[:, 0] == i)
        if sel.sum() > 2000:
            pi = special.softmax(L[1 + i].astype(np.float64) / np.float32(T))
            assert _chi2(np.bincount(r.tokens[sel, 1], minlength=V), pi) > PVAL


def test_greedy_against_brute_force():
    import torch
    w = W.make_tree(12, 300, depth=4, branching=(3, 2, 2, 1), max_nodes=40, dtype=torch.float32, temperature=0.0,
                    draft_noise=0.7, gen_seed=5)
    r = oracle.verify_tree(w.logits, w.node_tokens, w.node_parents, w.cu_num_nodes, w.temperature, 0, w.max_nodes,
                           w.max_depth)
    lg = w.logits.numpy()
    tok, par = w.node_tokens.numpy(), w.node_parents.numpy()
    n = w.max_nodes
    for b in range(w.B):
        base = b * (n + 1)
        cur, path = -1, []
        while True:
            g = int(np.argmax(lg[base + 1 + cur]))
            kids = [i for i in range(n) if par[b * n + i] == cur and tok[b * n + i] == g]
            if not kids:
                break
            cur = kids[0]
            path.append(cur)
        assert r.num_accepted[b] == len(path)
        assert r.path[b, :len(path)].tolist() == path
        assert r.tokens[b, len(path)] == g


def test_invalid_trees():
    lg = np.zeros((4 * 4, 8), np.float32)
    cu = np.array([0, 3, 6, 9, 12], np.int32)
    tokens = np.array([1, 2, 3, 1, 2, 3, 1, 9, 3, 1, 2, 3], np.int32)
    parents = np.array([-1, 0, 1, -1, 2, 0, -1, 0, 0, -1, 0, 1], np.int32)
    r = oracle.verify_tree(lg, tokens, parents, cu, np.ones(4, np.float32), 0, 3, 2)
    # request 0: depth 3 > max_depth 2; 1: parent after its child; 2: token 9 >= V; 3: depth 3 again
    assert (r.flags & oracle.FLAG_INVALID).tolist() == [8, 8, 8, 8]
    assert (r.num_accepted == -1).all() and (r.tokens == -1).all()
    r = oracle.verify_tree(lg, tokens, parents, cu, np.ones(4, np.float32), 0, 3, 3)
    assert (r.flags & oracle.FLAG_INVALID).tolist() == [0, 8, 8, 0]


def test_every_token_drafted_never_reaches_the_zero_residual():
    """In a tree the post-rejection residual is p without the stop node's
    children.  It is all zero only if the children cover every token of
    positive p, but then their accumulated p is 1 (up to fp64 rounding) and the
    coin u < 1 always accepts one of them [端到端深挖 §7.2]: a rejection means
    the uncovered tokens carry at least 1 - u >= 2^-24 of the mass.  So the
    tree's zero-residual fallback is unreachable; with every one of V tokens
    drafted at every node no request stops there or takes the fallback."""
    V, B = 8, 3000
    rng = np.random.default_rng(4)
    parents = [-1] * V + list(range(V))          # every token at the root, then one child each
    tokens = list(range(V)) + list(rng.integers(0, V, size=V))
    n = len(parents)
    lg = (rng.standard_normal((B * (n + 1), V)) * 2).astype(np.float32)
    cu = np.arange(B + 1, dtype=np.int32) * n
    r = oracle.verify_tree(lg, np.tile(np.array(tokens, np.int32), B), np.tile(np.array(parents, np.int32), B), cu,
                           np.full(B, 0.9, np.float32), 3, n, 3)
    assert (r.num_accepted >= 1).all()
    assert not (r.flags & oracle.FLAG_ZERO_RESIDUAL).any()


# ---- draft distributions: the extra token after a stop from max(0, p - q) ----
# [投机解码（Speculative Decoding）端到端深挖 §7.2: after a rejection the extra
# token is sampled from relu(target_probs - draft_probs)]

def _probs_rows(w):
    return oracle.probs(w.logits, w.cu_num_nodes, w.temperature)


def test_q_on_the_siblings_is_the_default_rule():
    """q_c = p_c on the tokens of c's children and 0 elsewhere makes
    max(0, p - q) the residual p without the siblings: the same tokens as
    without draft distributions, request for request."""
    import torch
    w = W.make_tree(24, 300, depth=4, branching=(3, 2, 2, 1), max_nodes=40, dtype=torch.float32,
                    temperature=("uniform", 0.5, 1.2), draft_noise=0.7, seed=5, gen_seed=15)
    p = _probs_rows(w)
    tok, par = w.node_tokens.numpy(), w.node_parents.numpy()
    cu = w.cu_num_nodes.numpy()
    q = np.zeros_like(p, dtype=np.float32)
    for b in range(w.B):
        s, e = int(cu[b]), int(cu[b + 1])
        for c in range(-1, e - s):
            row = s + b + 1 + c
            kids = tok[s:e][par[s:e] == c]
            q[row, kids] = p[row, kids]
    a = oracle.verify_tree(w.logits, w.node_tokens, w.node_parents, w.cu_num_nodes, w.temperature, w.seed,
                           w.max_nodes, w.max_depth)
    g = oracle.verify_tree(w.logits, w.node_tokens, w.node_parents, w.cu_num_nodes, w.temperature, w.seed,
                           w.max_nodes, w.max_depth, draft_probs=q)
    ok = ~(a.near_tie | g.near_tie)
    assert ok.sum() >= w.B - 2
    np.testing.assert_array_equal(g.num_accepted[ok], a.num_accepted[ok])
    np.testing.assert_array_equal(g.tokens[ok], a.tokens[ok])
    np.testing.assert_array_equal(g.path[ok], a.path[ok])


@pytest.mark.slow
@pytest.mark.parametrize("qkind", ["dirichlet", "peaked"])
def test_q_one_layer_law(qkind):
    """One layer of siblings S under the root: sibling s is accepted with
    probability p(s) (the roulette ignores q), and a stop emits max(0, p - q) /
    Z, so the first token's law is p(x) [x in S] + (1 - p(S)) max(0, p - q)(x) / Z."""
    V, B, T = 8, 400_000, 0.9
    rng = np.random.default_rng(21 if qkind == "dirichlet" else 22)
    sib = [2, 5]
    L = (rng.standard_normal((1 + len(sib), V)) * 1.2).astype(np.float32)
    p = special.softmax(L[0].astype(np.float64) / np.float32(T))
    q0 = rng.dirichlet(np.ones(V)) if qkind == "dirichlet" else np.eye(V)[np.argmax(p)] * 0.9 + 0.1 / V
    Q = np.tile(rng.dirichlet(np.ones(V), size=1 + len(sib)).astype(np.float32), (1, 1))
    Q[0] = q0.astype(np.float32)
    m = len(sib)
    lg = np.ascontiguousarray(np.broadcast_to(L, (B, 1 + m, V)).reshape(B * (1 + m), V))
    qq = np.ascontiguousarray(np.broadcast_to(Q, (B, 1 + m, V)).reshape(B * (1 + m), V))
    tokens = np.tile(np.array(sib, np.int32), B)
    parents = np.full(B * m, -1, np.int32)
    cu = (np.arange(B + 1) * m).astype(np.int32)
    r = oracle.verify_tree(lg, tokens, parents, cu, np.full(B, T, np.float32), 99, m, 2, draft_probs=qq)
    assert r.near_tie.mean() < 1e-4
    res = np.maximum(0.0, p - Q[0].astype(np.float64))
    pS = sum(p[s] for s in sib)
    law = (1 - pS) * res / res.sum()
    for s in sib:
        law[s] += p[s]
    assert _chi2(np.bincount(r.tokens[:, 0], minlength=V), law) > PVAL


def test_q_all_zero_residual_falls_back_to_p():
    """q = 2p at the root: max(0, p - q) is zero everywhere, so every stop at
    the root takes the race over p, flagged (as in the chain)."""
    V, B, T = 8, 4000, 1.0
    rng = np.random.default_rng(8)
    L = (rng.standard_normal((2, V)) * 1.0).astype(np.float32)
    p = special.softmax(L[0].astype(np.float64) / np.float32(T))
    Q = np.stack([2 * p, np.full(V, 1.0 / V)]).astype(np.float32)
    lg = np.ascontiguousarray(np.broadcast_to(L, (B, 2, V)).reshape(B * 2, V))
    qq = np.ascontiguousarray(np.broadcast_to(Q, (B, 2, V)).reshape(B * 2, V))
    tokens = np.full(B, int(np.argmin(p)), np.int32)  # an unlikely child: most requests stop at the root
    cu = np.arange(B + 1, dtype=np.int32)
    r = oracle.verify_tree(lg, tokens, np.full(B, -1, np.int32), cu, np.full(B, T, np.float32), 5, 1, 2,
                           draft_probs=qq)
    stop = r.num_accepted == 0
    assert stop.mean() > 0.8
    assert ((r.flags[stop] & oracle.FLAG_ZERO_RESIDUAL) != 0).all()
    assert not (r.flags[~stop] & oracle.FLAG_ZERO_RESIDUAL).any()
    assert _chi2(np.bincount(r.tokens[stop, 0], minlength=V), p) > PVAL


def test_q_ignored_at_a_childless_node():
    """A walk that ends at a leaf rejected nothing: the extra token follows the
    leaf's p whatever its draft row holds (here q peaked on p's mode, which
    max(0, p - q) would never emit)."""
    V, B, T = 6, 20000, 1.0
    rng = np.random.default_rng(12)
    L = (rng.standard_normal((2, V)) * 1.0).astype(np.float32)
    L[0, 3] += 6.0  # the root almost always accepts its one child, token 3
    p_leaf = special.softmax(L[1].astype(np.float64) / np.float32(T))
    Q = np.stack([np.full(V, 1.0 / V), np.eye(V)[np.argmax(p_leaf)]]).astype(np.float32)
    lg = np.ascontiguousarray(np.broadcast_to(L, (B, 2, V)).reshape(B * 2, V))
    qq = np.ascontiguousarray(np.broadcast_to(Q, (B, 2, V)).reshape(B * 2, V))
    cu = np.arange(B + 1, dtype=np.int32)
    r = oracle.verify_tree(lg, np.full(B, 3, np.int32), np.full(B, -1, np.int32), cu, np.full(B, T, np.float32), 6,
                           1, 2, draft_probs=qq)
    leaf = r.num_accepted == 1
    assert leaf.mean() > 0.9
    assert _chi2(np.bincount(r.tokens[leaf, 1], minlength=V), p_leaf) > PVAL
    assert (r.tokens[leaf, 1] == np.argmax(p_leaf)).mean() > 0.5 * p_leaf.max()


def test_tree_workload_recipe():
    """The EAGLE-style tree inputs: every request has the breadth-first shape,
    children are distinct top tokens of their parent's noisy row, and the
    draft rows are that row's softmax (one per tree position, summing to 1)."""
    import torch
    w = W.make_tree(5, 400, depth=3, branching=(3, 2, 1), max_nodes=20, dtype=torch.float32, temperature=0.8,
                    draft_noise=0.5, seed=1, gen_seed=9, with_q=True)
    n = w.max_nodes
    par = w.node_parents.numpy().reshape(w.B, n)
    tok = w.node_tokens.numpy().reshape(w.B, n)
    assert (par == par[0]).all() and w.max_depth == 3
    q = w.draft_probs.numpy().astype(np.float64)
    assert q.shape == (w.N + w.B, 400) and (q >= 0).all()
    np.testing.assert_allclose(q.sum(1), 1.0, rtol=1e-5)
    for b in range(w.B):
        for node_row in range(-1, n):
            kids = [i for i in range(n) if par[b, i] == node_row]
            if not kids:
                continue
            row = b * (n + 1) + 1 + node_row
            ks = tok[b, kids]
            assert len(set(ks.tolist())) == len(kids)
            # the children are the draft row's most likely tokens, in order
            order = np.argsort(-q[row], kind="stable")[:len(kids)]
            assert ks.tolist() == order.tolist()
