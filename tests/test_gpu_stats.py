"""GPU parity of the acceptance counters (rs_accept_stats_accumulate through
the C ABI) against the oracle's definition [第12章 投机解码：以小博大 §12.7.5;
投机解码（Speculative Decoding）端到端深挖 §13]: integer counters must match
exactly, accumulated over several verify steps, on ragged batches with
invalid and zero-draft requests and on batches spanning several workgroups.
"""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_rs_amd as rs
import rs_workloads as W
from oracle import stats

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device (run the CPU suite with -m 'not gpu')")
    rs.load_library()


def _verify(w):
    out, n = rs.verify(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                       seed=w.seed, max_k=w.max_k)
    return n


@pytest.mark.parametrize("n", [3, 4, 5])
def test_counters_match_oracle_over_steps(n):
    print(f"[gpu-case] stats workload {n}", flush=True)
    counters = torch.zeros(rs.STATS_COUNTERS, dtype=torch.int64, device="cuda")
    want = None
    for copy in range(3):  # three verify steps
        w = W.config(n, device="cuda", copy=copy)
        nacc = _verify(w)
        rs.accept_stats_accumulate(nacc, w.cu_num_draft_tokens, counters)
        want = stats.accumulate(want, nacc.cpu().numpy(), w.cu_num_draft_tokens.cpu().numpy())
    torch.cuda.synchronize()
    got = counters.cpu().numpy()
    np.testing.assert_array_equal(got, stats.to_array(want))
    assert rs.accept_rate(counters) == pytest.approx(stats.accept_rate(want), rel=1e-15)
    assert rs.accept_length(counters) == pytest.approx(stats.accept_length(want), rel=1e-15)
    print(f"[gpu-case] workload {n}: alpha {rs.accept_rate(counters):.4f} tau {rs.accept_length(counters):.4f}",
          flush=True)


def test_invalid_zero_draft_and_large_batch():
    rng = np.random.default_rng(5)
    B = 3000
    ks = rng.integers(0, 9, size=B)
    cu = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    n = np.array([rng.integers(0, k + 1) for k in ks], np.int32)
    n[rng.random(B) < 0.05] = -1
    nt, cut = torch.tensor(n, device="cuda"), torch.tensor(cu, device="cuda")
    counters = rs.accept_stats_accumulate(nt, cut)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(counters.cpu().numpy(), stats.to_array(stats.accumulate(None, n, cu)))


def test_max_positions():
    # K = 32 drafts, all accepted: every position counter moves
    B = 70
    cu = (np.arange(B + 1) * 32).astype(np.int32)
    n = np.full(B, 32, np.int32)
    counters = rs.accept_stats_accumulate(torch.tensor(n, device="cuda"), torch.tensor(cu, device="cuda"))
    torch.cuda.synchronize()
    got = counters.cpu().numpy()
    np.testing.assert_array_equal(got, stats.to_array(stats.accumulate(None, n, cu)))
    assert (got[rs.STATS_SCALARS:] == B).all()
