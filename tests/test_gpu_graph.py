"""HIP graph capture of the entry points.  Each call only enqueues kernels on
the caller's stream (no host synchronisation, allocation or memset), so it can
be captured once and replayed.  Every replay runs on inputs rewritten in place
since the last one, with eager calls and host synchronisations in between, and
must reproduce an eager call on the same inputs bit for bit: tokens, counts,
accepted tree paths, n-gram drafts and acceptance counters.
"""
import pytest
import torch

import rejection_sampling_verify_rs_amd as rs
import rs_workloads as W

pytestmark = pytest.mark.gpu

REPLAYS = (1, 2, 0, 1)  # input copy used by each replay


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device (run the CPU suite with -m 'not gpu')")
    rs.load_library()


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _capture(fn):
    """Warm fn up on a side stream, then capture it; returns (graph, outputs)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    return g, outs


def _check_replays(static, copies, fn, eager):
    """static: input tensors the graph reads; copies[i]: the same inputs of copy
    i; fn: the captured call; eager(inputs) -> outputs on fresh buffers."""
    g, outs = _capture(fn)
    for i in REPLAYS:
        for dst, src in zip(static, copies[i]):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        want = eager(copies[i])
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay on copy {i}: output {k} differs from the eager call"
    return outs


CHAIN = [
    # name, num_draft, V, dtype, q_mode, temperature, Debug knobs, filters
    ("stream bf16 B=64 K=8 V=32000", [8] * 64, 32000, torch.bfloat16, "noise", ("uniform", 0.3, 1.2),
     dict(sampling_path=3), (None, None)),
    ("phased fp32 ragged V=50000", [0, 3, 8, 5, 1, 8, 2, 7] * 4, 50000, torch.float32, "noise",
     [0.0, 0.9, 1.1, 0.7] * 8, dict(sampling_path=2), (None, None)),
    ("per-request bf16 B=4 K=5 V=32000 no q", [5] * 4, 32000, torch.bfloat16, "none", 0.8,
     dict(sampling_path=1), (None, None)),
    ("filtered bf16 B=32 K=4 V=151936", [4] * 32, 151936, torch.bfloat16, "noise", ("uniform", 0.5, 1.5),
     dict(), (50, 0.9)),
]


@pytest.mark.parametrize("case", CHAIN, ids=[c[0] for c in CHAIN])
def test_verify_graph_replays(case):
    name, nd, V, dt, qm, T, knobs, (tk, tp) = case
    _say(f"graph {name}")
    dm = "sample_q" if qm == "noise" else "argmax_mix"
    ws_ = [W.make(nd, V, dtype=dt, q_mode=qm, draft_mode=dm, temperature=T, seed=77, gen_seed=4100 + i,
                  device="cuda").with_filters(tk, tp) for i in range(3)]
    w = ws_[0]
    fields = lambda x: [t for t in (x.logits, x.draft_probs, x.draft_token_ids, x.temperature) if t is not None]
    static = [t.clone() for t in fields(w)]
    logits, q = static[0], (static[1] if w.draft_probs is not None else None)
    draft, temp = static[-2], static[-1]
    filtered = tk is not None or tp is not None
    nbytes = rs.workspace_size(w.B, w.D, w.max_k, V, dt, filtered)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.max_k + 1), dtype=torch.int32, device="cuda")
    nacc = torch.empty((w.B,), dtype=torch.int32, device="cuda")
    counters = torch.zeros(rs.STATS_COUNTERS, dtype=torch.int64, device="cuda")
    eager_counters = torch.zeros_like(counters)

    def call(lg, qq, dr, tt, o, n, wsp, ctr):
        rs.verify(lg, qq, dr, w.cu_num_draft_tokens, tt, seed=w.seed, max_k=w.max_k, out=o, num_accepted=n,
                  workspace=wsp, debug=rs.Debug(**knobs), top_k=w.top_k, top_p=w.top_p)
        rs.accept_stats_accumulate(n, w.cu_num_draft_tokens, ctr)
        return o, n, ctr

    def eager(inp):
        lg, qq = inp[0], (inp[1] if w.draft_probs is not None else None)
        o, n = torch.empty_like(out), torch.empty_like(nacc)
        call(lg, qq, inp[-2], inp[-1], o, n, torch.empty_like(ws), eager_counters)
        return o, n, eager_counters

    # the warm-up and the capture add nothing to the counters the replays check
    def fn():
        return call(logits, q, draft, temp, out, nacc, ws, counters)

    g, outs = _capture(fn)
    counters.zero_()
    for i in REPLAYS:
        for dst, src in zip(static, fields(ws_[i])):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        want = eager(fields(ws_[i]))
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"{name}: replay on copy {i}: output {k} differs from the eager call"
    assert int(counters.sum()) > 0


def test_verify_greedy_graph_replays():
    _say("graph verify_greedy bf16 B=48 K=6 V=65536")
    ws_ = [W.make([6] * 48, 65536, temperature=0.0, q_mode="none", draft_mode="argmax_mix", seed=5,
                  gen_seed=4200 + i, device="cuda") for i in range(3)]
    w = ws_[0]
    logits, draft = w.logits.clone(), w.draft_token_ids.clone()
    ws = torch.empty(max(rs.workspace_size(w.B, w.D, w.max_k, w.V, w.logits.dtype), 1), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((w.B, w.max_k + 1), dtype=torch.int32, device="cuda")
    nacc = torch.empty((w.B,), dtype=torch.int32, device="cuda")

    def fn():
        return rs.verify_greedy(logits, draft, w.cu_num_draft_tokens, max_k=w.max_k, out=out, num_accepted=nacc,
                                workspace=ws)

    def eager(inp):
        return rs.verify_greedy(inp[0], inp[1], w.cu_num_draft_tokens, max_k=w.max_k)

    _check_replays([logits, draft], [(x.logits, x.draft_token_ids) for x in ws_], fn, eager)


def test_verify_tree_graph_replays():
    _say("graph verify_tree bf16 B=16 V=151936")
    ts = [W.make_tree(16, 151936, temperature=("uniform", 0.5, 1.2), seed=9, gen_seed=4300 + i, device="cuda")
          for i in range(3)]
    t = ts[0]
    logits, tokens, temp = t.logits.clone(), t.node_tokens.clone(), t.temperature.clone()
    out = torch.empty((t.B, t.max_depth + 1), dtype=torch.int32, device="cuda")
    path = torch.empty((t.B, t.max_depth), dtype=torch.int32, device="cuda")
    nacc = torch.empty((t.B,), dtype=torch.int32, device="cuda")
    lib = rs.load_library()
    ws = torch.empty(max(int(lib.rs_verify_tree_workspace_size(t.B, t.V)), 1), dtype=torch.uint8, device="cuda")

    def run(lg, tk, tt, **bufs):
        return rs.verify_tree(lg, tk, t.node_parents, t.cu_num_nodes, tt, seed=t.seed, max_nodes=t.max_nodes,
                              max_depth=t.max_depth, **bufs)

    def fn():
        return run(logits, tokens, temp, out=out, accepted_nodes=path, num_accepted=nacc, workspace=ws)

    _check_replays([logits, tokens, temp], [(x.logits, x.node_tokens, x.temperature) for x in ts], fn,
                   lambda inp: run(*inp))


def test_ngram_graph_replays():
    _say("graph ngram_propose B=32 x 2048-token contexts")
    ctx = [W.make_contexts(32, 2048, 151936, seed=60 + i, device="cuda") for i in range(3)]
    flat, cu = ctx[0][0].clone(), ctx[0][1].clone()

    # only the first cu_num_draft_tokens[-1] drafts are defined
    def valid(drafts, num, cu_d):
        return drafts[: int(cu_d[-1])], num, cu_d

    g, outs = _capture(lambda: rs.ngram_propose(flat, cu, min_n=2, max_n=4, k=5))
    for i in REPLAYS:
        flat.copy_(ctx[i][0])
        cu.copy_(ctx[i][1])
        g.replay()
        torch.cuda.synchronize()
        got = valid(*[o.clone() for o in outs])
        want = valid(*rs.ngram_propose(ctx[i][0], ctx[i][1], min_n=2, max_n=4, k=5))
        assert got[0].numel() > 0
        for k, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay on copy {i}: output {k} differs from the eager call"
