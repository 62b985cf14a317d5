"""GPU parity of tree verify (rs_verify_tree through the C ABI) against the
CPU oracle [投机解码深度实战 §四; 投机解码（Speculative Decoding）端到端深挖 §6.2,
§7.1, §7.2]: accepted paths, counts and emitted tokens bit-exact on every
request the oracle does not flag as a near tie; a one-child-per-node tree
must give exactly the chain verify's output (rs_verify, no draft
probabilities) on the GPU; invalid trees get -1 rows.
"""
import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_rs_amd as rs
import rs_workloads as W
from parity import compare_tree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device (run the CPU suite with -m 'not gpu')")
    rs.load_library()


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _run(w):
    out, path, n = rs.verify_tree(w.logits, w.node_tokens, w.node_parents, w.cu_num_nodes, w.temperature,
                                  seed=w.seed, max_nodes=w.max_nodes, max_depth=w.max_depth,
                                  draft_probs=w.draft_probs)
    torch.cuda.synchronize()
    return out.cpu().numpy(), path.cpu().numpy(), n.cpu().numpy()


def _oracle(w):
    c = w.to("cpu")
    return oracle.verify_tree(c.logits, c.node_tokens, c.node_parents, c.cu_num_nodes, c.temperature, c.seed,
                              c.max_nodes, c.max_depth, draft_probs=c.draft_probs)


def _compare(w, g, o, max_flagged=1):
    out, path, n = g
    f = compare_tree(out, path, n, o, w, w.max_depth)
    assert f <= max_flagged
    return f


CASES = [
    # name, B, V, dtype, depth, branching, max_nodes, temperature
    ("eagle bf16 V=151936 B=64", 64, 151936, torch.bfloat16, 5, (4, 2, 2, 1, 1), 64, ("uniform", 0.5, 1.2)),
    ("eagle bf16 greedy V=151936", 32, 151936, torch.bfloat16, 5, (4, 2, 2, 1, 1), 64, 0.0),
    # at most 12 workgroups per request: the walk streams rows in 12-vector chunks
    ("eagle bf16 V=151936 B=128", 128, 151936, torch.bfloat16, 5, (4, 2, 2, 1, 1), 64, ("uniform", 0.5, 1.2)),
    ("wide fp32 V=32000 mixed", 40, 32000, torch.float32, 3, (8, 3, 1), 64, [0.0, 0.8, 1.0, -1.0] * 10),
    ("deep bf16 V=50000", 24, 50000, torch.bfloat16, 8, (2, 2, 2, 1, 1, 1, 1, 1), 48, 1.0),
    ("tiny V=7 fp32", 50, 7, torch.float32, 3, (3, 2, 1), 20, 0.9),
    # a vocabulary of more than 2^19 tokens, odd size: ragged last race chunk
    ("big vocab bf16 V=600001", 3, 600001, torch.bfloat16, 3, (3, 2, 1), 16, ("uniform", 0.6, 1.2)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_tree_parity(case):
    name, B, V, dt, depth, br, mn, T = case
    w = W.make_tree(B, V, depth=depth, branching=br, max_nodes=mn, dtype=dt, temperature=T, seed=31,
                    gen_seed=3000 + B, device="cuda", name=name)
    _say(f"{name}: B={w.B} nodes/request={w.max_nodes} depth={w.max_depth}")
    g = _run(w)
    o = _oracle(w)
    f = _compare(w, g, o)
    _say(f"{name}: flagged {f}, mean accepted {o.num_accepted.mean():.3f}")


def test_chain_tree_equals_chain_verify():
    w = W.make([4, 0, 6, 3, 8, 1, 5, 2] * 8, 151936, dtype=torch.bfloat16, logit_std=3.0,
               temperature=[0.7, 1.0, 0.0, 1.2] * 16, q_mode="none", draft_mode="argmax_mix", seed=9, gen_seed=91,
               device="cuda")
    parents = torch.tensor(np.concatenate([np.arange(k) - 1 for k in w.num_draft]).astype(np.int32), device="cuda")
    out_c, n_c = rs.verify(w.logits, None, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature, seed=w.seed,
                           max_k=w.max_k)
    out_t, path_t, n_t = rs.verify_tree(w.logits, w.draft_token_ids, parents, w.cu_num_draft_tokens, w.temperature,
                                        seed=w.seed, max_nodes=w.max_k, max_depth=w.max_k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(n_t.cpu().numpy(), n_c.cpu().numpy())
    np.testing.assert_array_equal(out_t.cpu().numpy(), out_c.cpu().numpy())


def test_duplicate_siblings_root_only_and_invalid():
    V = 1000
    g = torch.Generator().manual_seed(4)
    # request 0: duplicate sibling tokens; 1: no nodes (bonus only); 2: parent after child (invalid);
    # 3: token out of range (invalid); 4: a full 64-node star
    trees = [([5, 5, 9, 5], [-1, -1, -1, 0]), ([], []), ([1, 2], [1, -1]), ([3, V + 2], [-1, 0]),
             (list(range(100, 164)), [-1] * 64)]
    tok = torch.tensor([t for tr in trees for t in tr[0]], dtype=torch.int32)
    par = torch.tensor([p for tr in trees for p in tr[1]], dtype=torch.int32)
    cu = torch.tensor(np.concatenate([[0], np.cumsum([len(t[0]) for t in trees])]), dtype=torch.int32)
    B, N = len(trees), int(cu[-1])
    logits = torch.randn(N + B, V, generator=g) * 2
    logits[:, 5] += 4  # make the duplicated token likely
    T = torch.tensor([1.0, 0.8, 1.0, 1.0, 1.1])
    w = W.TreeWorkload("edge", logits.cuda(), tok.cuda(), par.cuda(), cu.cuda(), T.cuda(), 17,
                       [len(t[0]) for t in trees], 2)
    w.num_nodes = [len(t[0]) for t in trees]
    out, path, n = rs.verify_tree(w.logits, w.node_tokens, w.node_parents, w.cu_num_nodes, w.temperature, seed=17,
                                  max_nodes=64, max_depth=2)
    torch.cuda.synchronize()
    o = oracle.verify_tree(logits, tok, par, cu, T, 17, 64, 2)
    np.testing.assert_array_equal(n.cpu().numpy(), o.num_accepted)
    np.testing.assert_array_equal(out.cpu().numpy(), o.tokens)
    np.testing.assert_array_equal(path.cpu().numpy(), o.path)
    assert o.num_accepted[2] == -1 and o.num_accepted[3] == -1


def test_tree_rerun_bit_identical():
    w = W.make_tree(32, 151936, temperature=1.0, seed=3, gen_seed=44, device="cuda")
    a, b = _run(w), _run(w)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


Q_CASES = [
    # name, B, V, dtype, depth, branching, max_nodes, temperature
    ("q eagle bf16 V=151936 B=48", 48, 151936, torch.bfloat16, 5, (4, 2, 2, 1, 1), 64, ("uniform", 0.5, 1.2)),
    ("q eagle bf16 V=151936 B=96", 96, 151936, torch.bfloat16, 5, (4, 2, 2, 1, 1), 64, ("uniform", 0.5, 1.2)),
    ("q wide fp32 V=32001 mixed", 32, 32001, torch.float32, 3, (8, 3, 1), 64, [0.0, 0.8, 1.0, -1.0] * 8),
    ("q tiny V=7 fp32", 50, 7, torch.float32, 3, (3, 2, 1), 20, 0.9),
    ("q big vocab bf16 V=600001", 3, 600001, torch.bfloat16, 3, (3, 2, 1), 16, 1.0),
]


@pytest.mark.parametrize("case", Q_CASES, ids=[c[0] for c in Q_CASES])
def test_tree_parity_with_draft_probs(case):
    """With draft distributions the extra token after a stop at a node with
    children is the race over max(0, p - q) of that node's row; a childless
    node's extra token still follows p."""
    name, B, V, dt, depth, br, mn, T = case
    w = W.make_tree(B, V, depth=depth, branching=br, max_nodes=mn, dtype=dt, temperature=T, seed=37,
                    gen_seed=5000 + B, device="cuda", name=name, with_q=True)
    _say(f"{name}: B={w.B} nodes/request={w.max_nodes} depth={w.max_depth}")
    g = _run(w)
    o = _oracle(w)
    f = _compare(w, g, o)
    _say(f"{name}: flagged {f}, mean accepted {o.num_accepted.mean():.3f}")


def test_tree_q_on_siblings_equals_no_q():
    """q_c = p_c on c's children's tokens and 0 elsewhere: max(0, p - q) is p
    without the children, so the tokens equal those of the call without q."""
    w = W.make_tree(24, 50000, depth=4, branching=(3, 2, 2, 1), max_nodes=40, dtype=torch.float32,
                    temperature=("uniform", 0.6, 1.2), seed=23, gen_seed=77, device="cuda")
    c = w.to("cpu")
    cu, tok, par = c.cu_num_nodes.numpy(), c.node_tokens.numpy(), c.node_parents.numpy()
    Tb = torch.where(c.temperature > 0, c.temperature, torch.ones_like(c.temperature))
    rows_T = torch.repeat_interleave(Tb, torch.tensor([n + 1 for n in c.num_nodes]))
    p = torch.softmax(c.logits.double() / rows_T.double()[:, None], 1)
    q = torch.zeros_like(c.logits)
    for b in range(w.B):
        s, e = int(cu[b]), int(cu[b + 1])
        for node in range(-1, e - s):
            kids = torch.as_tensor(tok[s:e][par[s:e] == node], dtype=torch.long)
            row = s + b + 1 + node
            q[row, kids] = p[row, kids].float()
    a = _run(w)
    w.draft_probs = q.cuda()
    g = _run(w)
    o = _oracle(w)
    _compare(w, g, o, max_flagged=2)
    ok = ~o.near_tie
    for x, y in zip(a, g):
        np.testing.assert_array_equal(x[ok], y[ok])


def test_tree_q_zero_residual_falls_back_to_p():
    """q = 2p at every row: max(0, p - q) is zero wherever p > 0, so each stop
    at a node with children races p (flagged by the oracle) and must still
    match its candidates."""
    w = W.make_tree(40, 4096, depth=3, branching=(2, 2, 1), max_nodes=16, dtype=torch.float32, temperature=1.0,
                    seed=41, gen_seed=78, device="cuda")
    c = w.to("cpu")
    p = torch.softmax(c.logits.double(), 1)
    w.draft_probs = (2 * p).float().cuda()
    g = _run(w)
    o = _oracle(w)
    _compare(w, g, o, max_flagged=w.B)


def test_tree_draft_probs_argument_checks():
    """draft_probs must be fp32 with N + B rows of V on the logits' device, and
    16-byte aligned (a view one element in fails in the library)."""
    w = W.make_tree(4, 1000, depth=2, branching=(2, 1), max_nodes=8, dtype=torch.float32, seed=3, gen_seed=71,
                    device="cuda", with_q=True)
    args = (w.logits, w.node_tokens, w.node_parents, w.cu_num_nodes, w.temperature)
    kw = dict(seed=w.seed, max_nodes=w.max_nodes, max_depth=w.max_depth)
    with pytest.raises(ValueError):
        rs.verify_tree(*args, draft_probs=w.draft_probs[:-1], **kw)
    with pytest.raises(TypeError):
        rs.verify_tree(*args, draft_probs=w.draft_probs.double(), **kw)
    flat = torch.empty(w.draft_probs.numel() + 1, dtype=torch.float32, device="cuda")
    flat[1:] = w.draft_probs.reshape(-1)
    with pytest.raises(RuntimeError):
        rs.verify_tree(*args, draft_probs=flat[1:].view_as(w.draft_probs), **kw)
    out, path, n = rs.verify_tree(*args, draft_probs=w.draft_probs, **kw)
    torch.cuda.synchronize()
    assert (n.cpu() >= 0).all()
