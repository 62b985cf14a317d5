"""GPU parity of top-k / top-p filtered verify (rs_verify_filtered through the
C ABI) against the CPU oracle on the same seeded inputs [第12章 投机解码：以小博大
§12.2.3; §12.9 (compute_probs)].  Same bar as the unfiltered path: token ids
and accepted counts bit-exact on every request the oracle does not flag as a
near tie (top-p boundary ties included), p'(x*) within 1e-5 relative, and the
full filtered distribution p' of small shapes within 1e-5 relative (exact
zeros where the filter drops a token).
"""
import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_rs_amd as rs
import rs_workloads as W
from parity import compare, compare_p, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

KS = [0, 1, 2, 20, 50, 1000, -5]   # plus V - 1, V, V + 3 per case
PS = [1.0, 0.0, 0.3, 0.8, 0.9, 0.95, 0.999, 1.5]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device (run the CPU suite with -m 'not gpu')")
    rs.load_library()


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _mixed_filters(w, seed):
    rng = np.random.default_rng(seed)
    ks = KS + [w.V - 1, w.V, w.V + 3]
    top_k = rng.choice(ks, size=w.B).astype(np.int32)
    top_p = rng.choice(PS, size=w.B).astype(np.float32)
    return w.with_filters(top_k.tolist(), top_p.tolist())


def _case(name, ks, V, dtype, q_mode, temp, seed, ties=False, std=3.0):
    w = W.make(ks, V, dtype=dtype, logit_std=std, temperature=temp, q_mode=q_mode, q_sigma=0.8,
               draft_mode="sample_q" if q_mode == "noise" else "argmax_mix", seed=seed, gen_seed=6000 + seed,
               device="cuda", name=name)
    if ties:  # few distinct logit values: ties at every threshold
        w.logits = (torch.round(w.logits.float() * 2) / 2).to(dtype).contiguous()
    return _mixed_filters(w, seed)


CASES = [
    ("bf16 q ragged V=32000", lambda: _case("bf16 q ragged V=32000", [3, 0, 5, 8, 1, 4, 6, 2] * 4, 32000,
                                             torch.bfloat16, "noise", ("uniform", 0.4, 1.3), 21)),
    ("fp32 q V=9001", lambda: _case("fp32 q V=9001", [4] * 20, 9001, torch.float32, "noise", 0.9, 22)),
    ("bf16 onehot mixed-greedy V=65537",
     lambda: _case("bf16 onehot mixed-greedy V=65537", [2, 5, 1, 3] * 6, 65537, torch.bfloat16, "none",
                   [0.0, 1.0, 0.7, -1.0] * 6, 23)),
    ("bf16 q ties V=4096", lambda: _case("bf16 q ties V=4096", [3] * 40, 4096, torch.bfloat16, "noise", 1.0, 24,
                                         ties=True)),
    ("fp32 onehot ties V=777", lambda: _case("fp32 onehot ties V=777", [2] * 30, 777, torch.float32, "none", 0.8,
                                             25, ties=True)),
    # Nearly flat targets: top-p keeps tens of thousands of tokens (selection
    # over the whole row).  Each token then moves the cumulative mass by
    # ~1e-5 of the total, so the top-p boundary falls within the 1e-6 near-tie
    # band of the target on ~10% of rows; the oracle flags those rows, and
    # only the unflagged ones must match.
    ("bf16 q flat V=151936", lambda: _case("bf16 q flat V=151936", [3] * 16, 151936, torch.bfloat16, "noise", 2.0,
                                           28, std=0.3)),
    ("fp32 q flat V=100000", lambda: _case("fp32 q flat V=100000", [2] * 12, 100000, torch.float32, "noise", 1.5,
                                           29, std=0.5)),
    # more than 4096 segment maxima per row (V > 2^19 bf16): thresholds come
    # from the selection over the whole row, with no bound from the maxima
    ("bf16 q V=600001", lambda: _case("bf16 q V=600001", [2, 0, 3, 1] * 3, 600001, torch.bfloat16, "noise",
                                      ("uniform", 0.5, 1.3), 30)),
    ("fp32 onehot V=300007", lambda: _case("fp32 onehot V=300007", [3, 1, 2] * 3, 300007, torch.float32, "none",
                                           [1.0, 0.0, 0.8] * 3, 31)),
]
MAX_FLAGGED = {"bf16 q flat V=151936": 4, "fp32 q flat V=100000": 4}


@pytest.mark.parametrize("name,build", CASES, ids=[c[0] for c in CASES])
def test_filtered_parity(name, build):
    w = build()
    _say(f"{name}: B={w.B} D={w.D} V={w.V}")
    g = run_gpu(w, want_p=True)
    o = run_oracle(w)
    rep = compare(g, o, w)
    worst = compare_p(g, o, w)
    _say(f"{name}: flagged {rep['flagged']}/{rep['requests']}, max p' rel err {worst:.3e}")
    assert rep["flagged"] <= MAX_FLAGGED.get(name, 1)


@pytest.mark.parametrize("n", [4, 5, 2])
def test_workload_with_filters(n):
    w = W.config(n, device="cuda").with_filters(50, 0.9)
    _say(f"workload {n} + top_k 50, top_p 0.9: B={w.B} V={w.V}")
    g = run_gpu(w, want_p=True)
    o = run_oracle(w)
    rep = compare(g, o, w)
    worst = compare_p(g, o, w)
    _say(f"workload {n} filtered: flagged {rep['flagged']}/{rep['requests']}, max p' rel err {worst:.3e}, "
         f"mean accepted {o.num_accepted.mean():.3f}")
    assert rep["flagged"] <= 1


@pytest.mark.parametrize("n,tp", [(4, 0.9), (5, 0.95), (3, 0.8)])
def test_top_p_alone_full_size(n, tp):
    # top-p without top-k at full size: most rows keep hundreds to thousands of
    # tokens, so their thresholds come from the whole-row selection (by exact
    # value for bf16 logits)
    w = W.config(n, device="cuda").with_filters(None, tp)
    _say(f"workload {n} + top_p {tp}: B={w.B} V={w.V}")
    g = run_gpu(w, want_p=True)
    o = run_oracle(w)
    rep = compare(g, o, w)
    worst = compare_p(g, o, w)
    _say(f"workload {n} top_p {tp}: flagged {rep['flagged']}/{rep['requests']}, max p' rel err {worst:.3e}")
    assert rep["flagged"] <= 2


def test_filtered_probs_match_oracle():
    w = _case("probs", [2, 0, 3, 1] * 3, 3000, torch.bfloat16, "noise", ("uniform", 0.5, 1.5), 26)
    g = run_gpu(w, want_probs=True)
    c = w.to("cpu")
    T = c.temperature.numpy()
    lg = c.logits.float().numpy().astype(np.float64)
    cu = c.cu_num_draft_tokens.numpy()
    for b in range(w.B):
        for j in range(w.num_draft[b] + 1):
            row = cu[b] + b + j
            want, tie = oracle.filtered_probs_row(lg[row], np.float32(T[b]), int(c.top_k[b]), float(c.top_p[b]))
            if tie:
                continue
            got = g.probs[row].astype(np.float64)
            zero = want == 0
            assert np.all(got[zero] == 0), (b, j)
            big = want > 2.0 ** -100
            np.testing.assert_allclose(got[big], want[big], rtol=1e-5, err_msg=f"b={b} j={j}")


@pytest.mark.parametrize("knobs", [dict(row_nv=1), dict(race_tpt=8), dict(phases=(-1,)), dict(phases=(2, 4)),
                                   dict(path=1), dict(path=3)])
def test_filtered_launch_shape_independent(knobs):
    w = _case("shape", [4, 7, 0, 3, 8] * 5, 20000, torch.bfloat16, "noise", 0.9, 27)
    a = run_gpu(w)
    b = run_gpu(w, **knobs)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.num_accepted, b.num_accepted)


def test_filtered_rerun_bit_identical():
    w = W.config(4, device="cuda", B=64).with_filters(50, 0.9)
    a, b = run_gpu(w), run_gpu(w)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.num_accepted, b.num_accepted)


def test_filters_off_equal_unfiltered():
    w = W.config(4, device="cuda", B=32)
    off = w.with_filters([0, -1, w.V, w.V + 9] * 8, [1.0, 0.0, 2.0, -0.5] * 8)
    a, b = run_gpu(w), run_gpu(off)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.num_accepted, b.num_accepted)


def test_signed_zeros_at_threshold():
    # thresholds inside a large group of zeros of both signs: -0 and +0 are
    # one value, so every zero is kept and counted in the kept mass
    w = W.make([2] * 40, 4096, dtype=torch.bfloat16, temperature=1.0, q_mode="noise", q_sigma=0.8,
               draft_mode="sample_q", seed=31, gen_seed=6031, device="cuda", name="signed zeros")
    rng = np.random.default_rng(31)
    base = np.full(4096, -6.0, np.float32)
    base[:8] = 4.0
    base[8:1508] = 0.0
    base[1508:3008] = -0.0
    rows = np.stack([rng.permutation(base) for _ in range(w.logits.shape[0])])
    w.logits = torch.from_numpy(rows).to(torch.bfloat16).to(w.logits.device).contiguous()
    top_k = rng.choice([0, 8, 9, 500, 2000, 3008, 3009, 4095], size=w.B)
    top_p = rng.choice([1.0, 0.5, 0.9, 0.99, 0.999], size=w.B)
    w = w.with_filters(top_k.tolist(), top_p.tolist())
    _say(f"signed zeros: B={w.B} V={w.V}")
    o = run_oracle(w)
    for _ in range(3):  # ties of equal values once raced here: repeat
        g = run_gpu(w, want_p=True)
        rep = compare(g, o, w)
        compare_p(g, o, w)
        assert rep["flagged"] == 0


def test_top_k_one_is_greedy_like():
    # top-k = 1 leaves only the argmax (and its exact ties): every emitted
    # extra token is a row maximum of its logits
    w = W.config(2, device="cuda").with_filters(1, None)
    g = run_gpu(w)
    c = w.to("cpu")
    lg = c.logits.float().numpy()
    cu = c.cu_num_draft_tokens.numpy()
    for b in range(w.B):
        n = int(g.num_accepted[b])
        row = cu[b] + b + n
        assert lg[row, g.tokens[b, n]] == lg[row].max()
