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
from parity import compare, compare_p, compare_tree, run_gpu, run_oracle

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
        compare_p(g, o, w)


def _random_trees(rng, with_q=False):
    """Ragged random trees (node i's parent uniform over the earlier nodes and
    the prefix), children's tokens mostly near the top of their parent's row,
    sometimes random or repeated; mixed greedy / random temperatures.  with_q:
    also draft distributions, one per tree position, each the softmax of its
    row plus N(0, 1) noise."""
    V = int(rng.choice([7, 1000, 32000, 151936]))
    B = int(rng.integers(1, 40 if V > 32000 else 100))
    max_nodes = int(rng.choice([8, 20, 64]))
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    counts = rng.integers(0, max_nodes + 1, size=B)
    parents, tokens, depth_max = [], [], 0
    rows = []
    for b in range(B):
        n = int(counts[b])
        par = [int(rng.integers(-1, i)) for i in range(n)]
        dep = []
        for i, p_ in enumerate(par):
            dep.append(0 if p_ < 0 else dep[p_] + 1)
        depth_max = max([depth_max] + [d + 1 for d in dep])
        lg = torch.from_numpy((rng.standard_normal((n + 1, V)) * float(rng.choice([1.0, 3.0]))).astype(np.float32))
        tk = []
        for i, p_ in enumerate(par):
            r = lg[p_ + 1]
            u = rng.random()
            if u < 0.6:
                tk.append(int(torch.topk(r, min(3, V)).indices[int(rng.integers(0, min(3, V)))]))
            elif u < 0.8 and tk:
                tk.append(tk[int(rng.integers(0, len(tk)))])  # a repeated token
            else:
                tk.append(int(rng.integers(0, V)))
        parents += par
        tokens += tk
        rows.append(lg)
    logits = torch.cat(rows).to(dtype).contiguous().cuda()
    q = None
    if with_q:
        lq = torch.cat(rows)
        noise = torch.from_numpy(rng.standard_normal(lq.shape).astype(np.float32))
        q = torch.softmax(lq + noise, dim=1).contiguous().cuda()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    T = torch.tensor(rng.choice([0.0, 0.6, 1.0, 1.4], size=B).astype(np.float32)).cuda()
    w = W.TreeWorkload("random trees", logits, torch.tensor(tokens, dtype=torch.int32).cuda(),
                       torch.tensor(parents, dtype=torch.int32).cuda(), cu, T, int(rng.integers(0, 2**40)),
                       [int(c) for c in counts], depth_max, draft_probs=q)
    return w, max_nodes, (f"B={B} V={V} max_nodes={max_nodes} {str(dtype).split('.')[-1]} depth {depth_max}"
                          + (" with q" if with_q else ""))


@pytest.mark.parametrize("seed,with_q", [(11, False), (12, False), (13, True), (14, True)])
def test_random_tree_sweep(seed, with_q):
    import oracle
    rng = np.random.default_rng(seed)
    for case in range(12):
        w, max_nodes, desc = _random_trees(rng, with_q)
        print(f"[gpu-case] tree sweep {seed} case {case}: {desc}", flush=True)
        max_depth = max(w.max_depth, 1)
        out, path, n = rs.verify_tree(w.logits, w.node_tokens, w.node_parents, w.cu_num_nodes, w.temperature,
                                      seed=w.seed, max_nodes=max_nodes, max_depth=max_depth,
                                      draft_probs=w.draft_probs)
        torch.cuda.synchronize()
        c = w.to("cpu")
        o = oracle.verify_tree(c.logits, c.node_tokens, c.node_parents, c.cu_num_nodes, c.temperature, c.seed,
                               max_nodes, max_depth, draft_probs=c.draft_probs)
        compare_tree(out.cpu().numpy(), path.cpu().numpy(), n.cpu().numpy(), o, w, max_depth)


@pytest.mark.parametrize("seed", [21, 22])
def test_random_ngram_sweep(seed):
    from oracle import ngram
    rng = np.random.default_rng(seed)
    for case in range(15):
        B = int(rng.integers(1, 200))
        vocab = int(rng.choice([3, 20, 1000, 151936]))
        lo = int(rng.integers(0, 50))
        length = (lo, lo + int(rng.integers(0, 3000)))
        min_n = int(rng.integers(1, 5))
        max_n = min_n + int(rng.integers(0, 8))
        k = int(rng.integers(1, 12))
        flat, cu = W.make_contexts(B, length, vocab, copy_prob=float(rng.choice([0.0, 0.5, 0.9])),
                                   seed=int(rng.integers(0, 2**31)), device="cuda")
        cuh = cu.cpu().numpy()
        lens = np.diff(cuh)
        mml = int(rng.choice([1 << 40, int(lens.max()) + int(rng.integers(0, k + 2)) if lens.size else 1]))
        print(f"[gpu-case] ngram sweep {seed} case {case}: B={B} len={length} vocab={vocab} n={min_n}-{max_n} "
              f"k={k} max_model_len={mml}", flush=True)
        d, n, c = rs.ngram_propose(flat, cu, min_n=min_n, max_n=max_n, k=k, max_model_len=mml)
        torch.cuda.synchronize()
        f = flat.cpu().numpy()
        ctxs = [f[cuh[b]:cuh[b + 1]] for b in range(B)]
        want, wcnt = ngram.propose_batch(ctxs, min_n, max_n, k, mml)
        n, c, d = n.cpu().numpy(), c.cpu().numpy(), d.cpu().numpy()
        np.testing.assert_array_equal(n, wcnt)
        np.testing.assert_array_equal(c, np.concatenate([[0], np.cumsum(wcnt)]))
        for b in range(B):
            np.testing.assert_array_equal(d[c[b]:c[b + 1]], want[b, :wcnt[b]])
