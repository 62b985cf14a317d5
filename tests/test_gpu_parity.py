"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on
the same seeded inputs.  Token ids and accepted counts must match bit for bit
on every request the oracle does not flag as a near tie; p(x*) must match to
1e-5 relative.  Cases cover the five measured workloads at full size (in the
launch configuration the benchmark uses), ragged batches that span several
chunks with unaligned rows and ragged tails, the method's degenerate cases and
the launch-shape / run-to-run determinism of the output.
"""
import numpy as np
import pytest
import torch
from scipy import special, stats

import oracle
import rejection_sampling_verify_rs_amd as rs
import rs_workloads as W
from parity import GpuResult, compare, compare_p, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device (run the CPU suite with -m 'not gpu')")
    rs.load_library()


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


# ---------------------------------------------------------- measured workloads
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_workload_full_size(n):
    w = W.config(n, device="cuda")
    _say(f"workload {n}: {w.name} B={w.B} D={w.D} V={w.V}")
    g = run_gpu(w, want_p=True)
    o = run_oracle(w)
    rep = compare(g, o, w)
    worst = compare_p(g, o, w)
    _say(f"workload {n}: flagged {rep['flagged']}/{rep['requests']}, max p rel err {worst:.3e}, "
         f"mean accepted {o.num_accepted.mean():.3f}")
    assert rep["flagged"] <= 1


def test_workload2_greedy_entry():
    w = W.config(2, device="cuda")
    _say("workload 2 through rs_verify_greedy")
    g = run_gpu(w, greedy_entry=True)
    o = run_oracle(w, greedy_entry=True)
    np.testing.assert_array_equal(g.num_accepted, o.num_accepted)
    np.testing.assert_array_equal(g.tokens, o.tokens)


# ------------------------------------------------- ragged, unaligned, several chunks
SMALL = [
    # (name, B, K range, V, dtype, q_mode, temperature)
    ("bf16 q ragged V=40013", 37, (0, 8), 40013, torch.bfloat16, "noise", ("uniform", 0.3, 1.5)),
    ("fp32 q ragged V=9001", 19, (0, 6), 9001, torch.float32, "noise", 1.0),
    ("bf16 onehot mixed-greedy V=65537", 41, (1, 5), 65537, torch.bfloat16, "none", "mixed"),
    ("fp32 onehot V=7", 25, (0, 4), 7, torch.float32, "none", 0.9),
    ("bf16 q V=1", 6, (0, 3), 1, torch.bfloat16, "noise", 1.0),
    ("bf16 q max_k=32 V=3000", 9, (30, 32), 3000, torch.bfloat16, "noise", 0.7),
    ("bf16 q all K=0 V=20000", 33, (0, 0), 20000, torch.bfloat16, "noise", 1.1),
    ("bf16 q K=1 B=3000 V=517", 3000, (1, 1), 517, torch.bfloat16, "noise", 1.0),
]


def _small(name, B, krange, V, dtype, q_mode, temp, seed):
    rng = np.random.default_rng(seed)
    ks = rng.integers(krange[0], krange[1] + 1, size=B).tolist()
    if temp == "mixed":
        temp = [0.0 if i % 3 == 0 else (-1.0 if i % 3 == 1 else 0.8) for i in range(B)]
    dm = "sample_q" if q_mode == "noise" else "argmax_mix"
    return W.make(ks, V, dtype=dtype, logit_std=3.0, temperature=temp, q_mode=q_mode, q_sigma=0.8,
                  draft_mode=dm, seed=seed, gen_seed=5000 + seed, device="cuda", name=name)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_ragged(case):
    w = _small(*case, seed=len(case[0]))
    _say(f"{w.name}: B={w.B} D={w.D} max_k={w.max_k}")
    g = run_gpu(w, want_p=True)
    o = run_oracle(w)
    compare(g, o, w)
    compare_p(g, o, w)


def test_full_probs_small():
    w = _small("probs", 5, (0, 4), 5003, torch.bfloat16, "noise", ("uniform", 0.2, 2.0), seed=3)
    _say("full p rows, V=5003")
    g = run_gpu(w, want_probs=True)
    P = oracle.probs(w.to("cpu").logits, w.to("cpu").cu_num_draft_tokens, w.to("cpu").temperature)
    big = P >= 2.0 ** -100
    rel = np.abs(g.probs[big] - P[big]) / P[big]
    assert rel.max() <= 1e-5, rel.max()
    assert np.all(np.abs(g.probs[~big]) <= 2.0 ** -99)


# ------------------------------------------------------------- determinism
def test_launch_shapes_give_identical_output():
    w = W.config(4, device="cuda", B=24)
    _say("launch-shape sweep on B=24 K=8 V=151936")
    ref = run_gpu(w)
    o = run_oracle(w)
    compare(ref, o, w)
    for nv, tpt, path, phases in [(1, 8, 2, (-1,)), (4, 32, 2, (1,)), (16, 8, 2, (3,)), (16, 32, 2, (5,)),
                                  (4, 8, 2, (8,)), (16, 32, 2, (2, 5)), (4, 32, 2, (1, 3, 6)), (16, 32, 1, ()),
                                  (1, 32, 1, ()), (16, 32, 3, ()), (16, 8, 3, (1,)), (4, 32, 3, (9,)),
                                  (1, 8, 3, (2,)), (4, 8, 3, (5,))]:
        g = run_gpu(w, row_nv=nv, race_tpt=tpt, path=path, phases=phases)
        compare(g, o, w)
        ok = ~o.near_tie  # a near tie may resolve either way, and differently per launch shape
        np.testing.assert_array_equal(g.tokens[ok], ref.tokens[ok])
        np.testing.assert_array_equal(g.num_accepted[ok], ref.num_accepted[ok])


@pytest.mark.parametrize("n", [3, 4, 5])
@pytest.mark.parametrize("path,phases", [(1, ()), (2, (-1,)), (2, (2,)), (2, (1, 2, 4)), (3, ()), (3, (1,))])
def test_paths_and_phases_full_size(n, path, phases):
    """The per-request path, the one-phase split path (every row), other
    phase splits and the stream path all match the oracle at full size."""
    w = W.config(n, device="cuda")
    _say(f"workload {n}: path {path}, phase ends {phases}")
    g = run_gpu(w, path=path, phases=phases, want_p=True)
    o = run_oracle(w)
    compare(g, o, w)
    compare_p(g, o, w)


@pytest.mark.parametrize("ks,V,want", [([4], 1024, 1), ([5] * 8, 1024, 1), ([4] * 16, 32000, 3), ([8] * 32, 151936, 3),
                                       ([8] * 64, 151936, 2), ([8] * 96, 151936, 2), ([8] * 128, 151936, 3),
                                       ([3] * 512, 32000, 3)])
def test_automatic_path_choice(ks, V, want):
    """The automatic rule picks the per-request path for tiny batches with
    short walks; the stream path when the logits total at most 128 MB or
    from B x chunks per row >= 512 (16-vector chunks); the phased split
    otherwise.  The chosen path matches the oracle."""
    w = W.make(ks, V, dtype=torch.bfloat16, logit_std=4.0, temperature=("uniform", 0.3, 1.2), q_mode="noise",
               q_sigma=0.8, seed=41, gen_seed=4100 + len(ks), device="cuda")
    d = rs.Debug()
    out, n = rs.verify(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                       seed=w.seed, max_k=w.max_k, debug=d)
    torch.cuda.synchronize()
    _say(f"B={w.B} K={ks[0]} V={V}: path {d.path_taken}")
    assert d.path_taken == want
    o = run_oracle(w)
    compare(GpuResult(out.cpu().numpy(), n.cpu().numpy()), o, w)


def test_rerun_is_bit_identical():
    w = W.config(5, device="cuda")
    _say("workload 5 twice")
    a, b = run_gpu(w), run_gpu(w)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.num_accepted, b.num_accepted)


def test_back_to_back_calls_share_one_workspace():
    """Calls queued back to back on one stream with one workspace (no host
    synchronisation between them), alternating inputs and shapes, each give
    the output of a lone call: the per-call hand-off state (arrival counters,
    partials, chunk winners, records) never leaks from one call into the next,
    even from a workspace that starts out as garbage."""
    dev = torch.device("cuda")
    ws_ = [W.config(4, device=dev, copy=0), W.config(5, device=dev), W.config(4, device=dev, copy=1)]
    _say("back-to-back calls: workload 4 copy 0, workload 5, workload 4 copy 1")
    refs = [run_gpu(w) for w in ws_]
    for w, r in zip(ws_, refs):
        compare(r, run_oracle(w), w)
    size = max(rs.workspace_size(w.B, w.D, w.max_k, w.V, w.logits.dtype) for w in ws_)
    ws = torch.full((size,), 0xFF, dtype=torch.uint8, device=dev)
    outs = []
    for k in range(12):
        w = ws_[k % 3]
        out, n = rs.verify(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                           seed=w.seed, max_k=w.max_k, workspace=ws)
        outs.append((k % 3, out, n))
    torch.cuda.synchronize()
    for i, out, n in outs:
        np.testing.assert_array_equal(out.cpu().numpy(), refs[i].tokens)
        np.testing.assert_array_equal(n.cpu().numpy(), refs[i].num_accepted)


# ------------------------------------------------------------- degenerate cases
def _custom(rows, q, drafts, ks, T, seed=0):
    dev = torch.device("cuda")
    cu = torch.zeros(len(ks) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(ks, dtype=torch.int32), 0)
    return W.Workload("custom", rows.to(dev).contiguous(), None if q is None else q.to(dev).contiguous(),
                      torch.as_tensor(drafts, dtype=torch.int32).to(dev), cu.to(dev),
                      torch.as_tensor(T, dtype=torch.float32).to(dev), seed, list(ks))


def test_tiny_temperature():
    w = W.make([4] * 16, 3000, logit_std=3.0, temperature=0.01, q_mode="noise", q_sigma=0.5, seed=7,
               gen_seed=77, device="cuda")
    _say("T = 0.01")
    g, o = run_gpu(w, want_p=True), run_oracle(w)
    compare(g, o, w)
    compare_p(g, o, w)


def test_q_zero_at_draft_accepts():
    w = W.make([3] * 8, 2000, logit_std=2.0, temperature=1.0, q_mode="noise", q_sigma=0.5, seed=8,
               gen_seed=88, device="cuda")
    q = w.draft_probs.clone()
    q[torch.arange(w.D, device="cuda"), w.draft_token_ids.long()] = 0.0
    w.draft_probs = q
    _say("q(x*) = 0")
    g, o = run_gpu(w), run_oracle(w)
    compare(g, o, w)
    assert (o.num_accepted == 3).all()


def test_q_equal_p_accepts_all():
    B, K, V = 16, 5, 4000
    w = W.make([K] * B, V, logit_std=3.0, temperature=0.9, q_mode="none", draft_mode="uniform", seed=9,
               gen_seed=99, device="cuda")
    rows = W.draft_rows(w.num_draft).cuda()
    q = torch.softmax(w.logits.float()[rows] / 0.9, dim=-1)
    ids = torch.multinomial(q, 1, generator=torch.Generator("cuda").manual_seed(5)).view(-1).to(torch.int32)
    w.draft_probs, w.draft_token_ids = q.contiguous(), ids
    _say("q = p")
    g, o = run_gpu(w), run_oracle(w)
    compare(g, o, w)
    assert (o.num_accepted[~o.near_tie] == K).all()


def test_disjoint_supports():
    torch.manual_seed(10)
    V, B = 512, 64
    l = torch.randn(V) * 2
    l[V // 2:] = -1e4
    rows = l.repeat(2 * B, 1).to(torch.bfloat16)
    qrow = torch.zeros(V)
    qrow[V // 2:] = torch.softmax(torch.randn(V // 2), 0)
    q = qrow.repeat(B, 1)
    drafts = torch.multinomial(q, 1, generator=torch.Generator().manual_seed(1)).view(-1)
    w = _custom(rows, q, drafts, [1] * B, [1.0] * B, seed=11)
    _say("disjoint supports")
    g, o = run_gpu(w), run_oracle(w)
    compare(g, o, w)
    assert (o.num_accepted == 0).all()


def test_masked_logits_minus_inf():
    torch.manual_seed(12)
    w = W.make([3] * 12, 1000, logit_std=2.0, temperature=1.0, q_mode="noise", q_sigma=0.5, seed=12,
               gen_seed=120, device="cuda")
    lg = w.logits.clone()
    lg[:, 500:] = float("-inf")
    w.logits = lg
    rows = W.draft_rows(w.num_draft).cuda()
    q = torch.softmax(lg.float()[rows] + 0.3 * torch.randn(w.D, 1000, device="cuda"), -1)
    w.draft_probs = q.contiguous()
    w.draft_token_ids = torch.multinomial(q, 1).view(-1).to(torch.int32)
    _say("-inf logits")
    g, o = run_gpu(w), run_oracle(w)
    compare(g, o, w)
    assert (g.tokens[g.tokens >= 0] < 500).all()


def test_greedy_bf16_ties():
    B, K, V = 64, 4, 3001
    rng = np.random.default_rng(4)
    rows = torch.from_numpy((rng.standard_normal((B * (K + 1), V)) * 3).astype(np.float32)).to(torch.bfloat16).float()
    drafts = []
    for r in range(B * (K + 1)):
        a, b = sorted(rng.choice(V, 2, replace=False))
        rows[r, a] = rows[r, b] = rows[r].max()
    rows = rows.to(torch.bfloat16)
    for b in range(B):
        for j in range(K):
            r = rows[b * (K + 1) + j].float()
            m = r.max()
            idx = torch.nonzero(r == m).view(-1)
            drafts.append(int(idx[0]) if rng.random() < 0.7 else int(idx[-1]))
    w = _custom(rows, None, drafts, [K] * B, [0.0] * B)
    _say("greedy exact ties")
    for entry in (True, False):
        g, o = run_gpu(w, greedy_entry=entry), run_oracle(w, greedy_entry=entry)
        np.testing.assert_array_equal(g.tokens, o.tokens)
        np.testing.assert_array_equal(g.num_accepted, o.num_accepted)


def test_invalid_metadata_rows():
    torch.manual_seed(13)
    V = 100
    rows = torch.randn(8, V).to(torch.bfloat16)
    # request 0: K=2 valid; request 1: K=4 > max_k=3 (invalid); D = 6, B = 2 -> R = 8
    cu = [0, 2, 6]
    drafts = [1, 2, 3, 4, 5, 6]
    w = _custom(rows, None, drafts, [2, 4], [1.0, 1.0])
    w.cu_num_draft_tokens = torch.tensor(cu, dtype=torch.int32, device="cuda")
    _say("invalid metadata")
    out, n = rs.verify(w.logits, None, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature, seed=0, max_k=3)
    out, n = out.cpu().numpy(), n.cpu().numpy()
    assert n[1] == -1 and (out[1] == -1).all()
    assert 0 <= n[0] <= 2
    # a draft id outside [0, V)
    w2 = _custom(rows[:6], None, [1, 2, 3, 999], [2, 2], [1.0, 0.0])
    out, n = rs.verify(w2.logits, None, w2.draft_token_ids, w2.cu_num_draft_tokens, w2.temperature, seed=0, max_k=2)
    assert n.cpu()[1] == -1 and (out.cpu()[1] == -1).all() and n.cpu()[0] >= 0
    o = run_oracle(w2)
    assert o.num_accepted[1] == -1


@pytest.mark.parametrize("path", [0, 1, 2, 3])
def test_invalid_requests_every_path(path):
    """Requests made invalid by a draft id V at position 1, a draft id -7 at
    position 0 or a last offset beyond D get n = -1 and a -1 row on every
    path, at a vocabulary of three row chunks per row, and the valid requests
    beside them, one with K = 0, match the oracle."""
    g0 = torch.Generator().manual_seed(29)
    V, ks = 70001, [3, 2, 0, 2, 3]
    D, B = sum(ks), len(ks)
    rows = (torch.randn(D + B, V, generator=g0) * 3).to(torch.bfloat16)
    q = torch.softmax(rows[:D].float() + 0.5 * torch.randn(D, V, generator=g0), 1)
    drafts = torch.randint(0, V, (D,), generator=g0, dtype=torch.int32)
    drafts[3 + 1] = V   # request 1, position 1
    drafts[5] = -7      # request 3, position 0
    w = _custom(rows, q, drafts, ks, [1.0, 1.0, 0.7, 1.0, 1.0], seed=5)
    w.cu_num_draft_tokens = torch.tensor([0, 3, 5, 5, 7, 11], dtype=torch.int32, device="cuda")  # request 4: e > D
    _say(f"invalid requests, V={V}, path {path}")
    g, o = run_gpu(w, path=path), run_oracle(w)
    bad = [1, 3, 4]
    assert (o.num_accepted[bad] == -1).all() and (o.num_accepted[[0, 2]] >= 0).all()
    assert (g.num_accepted[bad] == -1).all() and (g.tokens[bad] == -1).all()
    compare(g, o, w)


# ------------------------------------------- 10^6 requests: parity + marginal = p
def test_million_requests_parity_and_marginal():
    V, B, T = 8, 1_000_000, 1.0
    rng = np.random.default_rng(21)
    l0 = (rng.standard_normal(V) * 1.5).astype(np.float32)
    l1 = (rng.standard_normal(V) * 1.5).astype(np.float32)
    qv = special.softmax(l0.astype(np.float64) + rng.standard_normal(V)).astype(np.float32)
    rows = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(np.stack([l0, l1]), (B, 2, V)).reshape(2 * B, V)))
    q = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(qv, (B, V))))
    drafts = rng.choice(V, size=B, p=qv.astype(np.float64) / qv.sum(dtype=np.float64))
    w = _custom(rows, q, drafts, [1] * B, [T] * B, seed=2025)
    _say("1e6 requests, V=8")
    g, o = run_gpu(w), run_oracle(w)
    rep = compare(g, o, w, max_flag_frac=1e-4)
    _say(f"flagged {rep['flagged']} of {rep['requests']}")
    p0 = special.softmax(l0.astype(np.float64) / T)
    counts = np.bincount(g.tokens[:, 0], minlength=V)
    assert stats.chisquare(counts, p0 * B).pvalue > 1e-3


# ------------------------------------------------ all-zero residual (q = 2p)
def _q_twice_p(ks, V, T, seed, logit_std=3.0, device="cuda"):
    """Draft rows q = 2 p (p = softmax(l / T) of the draft position's row, fp64
    then fp32): not normalised, which the boundary allows (q >= 0).  Drafts
    are drawn from p.  Every accept test is u < 1/2, and at every rejection
    max(0, p - q) is zero everywhere: the reading races over p instead."""
    w = W.make(ks, V, dtype=torch.bfloat16, logit_std=logit_std, temperature=T, q_mode="none",
               draft_mode="uniform", seed=seed, gen_seed=seed + 100, device=device)
    rows = W.draft_rows(w.num_draft).to(w.device)
    slot_req = torch.repeat_interleave(torch.arange(w.B), torch.tensor(w.num_draft)).to(w.device)
    Ts = w.temperature.double()[slot_req].clamp_min(1e-3)[:, None]
    p = torch.softmax(w.logits.double()[rows] / Ts, dim=-1)
    w.draft_probs = (2.0 * p).float().contiguous()
    g = torch.Generator(device=w.device).manual_seed(seed)
    w.draft_token_ids = torch.multinomial(p.float(), 1, generator=g).view(-1).to(torch.int32).contiguous()
    return w


@pytest.mark.parametrize("path", [0, 1, 2, 3])
def test_zero_residual_q_twice_p(path):
    w = _q_twice_p([4] * 40 + [0, 1, 7], 20011, ("uniform", 0.5, 1.3), seed=29)
    _say(f"q = 2p, B={w.B} V={w.V}, path {path}")
    g, o = run_gpu(w, path=path, want_p=True), run_oracle(w)
    zr = (o.flags & oracle.FLAG_ZERO_RESIDUAL) != 0
    assert zr.sum() >= 20  # about half of the requests reject at position 0 already
    rep = compare(g, o, w)
    compare_p(g, o, w)
    _say(f"zero-residual requests {int(zr.sum())}, flagged {rep['flagged']}")


def test_zero_residual_full_vocab_and_filtered():
    """q = 2p at V = 151936 (the fallback scans a whole row) on the automatic
    path and the phased path, then with top-k / top-p filtering (p' >= p on
    the kept tokens, so only some rows have a zero residual there)."""
    w = _q_twice_p([3] * 24 + [8] * 8, 151936, ("uniform", 0.4, 1.2), seed=31, logit_std=4.0)
    o = run_oracle(w)
    assert ((o.flags & oracle.FLAG_ZERO_RESIDUAL) != 0).sum() >= 10
    for path in (0, 2):
        _say(f"q = 2p, V=151936, path {path}")
        compare(run_gpu(w, path=path), o, w)
    wf = w.with_filters([0, 50, 2000, 20] * 8, [1.0, 0.9, 0.5, 0.99] * 8, name="q = 2p filtered")
    _say("q = 2p with top-k / top-p")
    gf, of = run_gpu(wf, want_p=True), run_oracle(wf)
    compare(gf, of, wf)
    compare_p(gf, of, wf)
