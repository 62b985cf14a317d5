"""GPU parity of the batched n-gram proposer (rs_ngram_propose through the C
ABI) against the oracle [第12章 投机解码：以小博大 §12.4.4]: proposals, counts
and prefix sums bit-exact (integer work), on ragged batches of repetitive
contexts, short and empty contexts, k capped by max_model_len, and a
proposer -> rs_verify pipeline checked end to end against the oracles.
"""
import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_rs_amd as rs
import rs_workloads as W
from parity import GpuResult, compare
from oracle import ngram

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device (run the CPU suite with -m 'not gpu')")
    rs.load_library()


def _check(flat, cu, min_n, max_n, k, mml):
    d, n, c = rs.ngram_propose(flat, cu, min_n=min_n, max_n=max_n, k=k, max_model_len=mml)
    torch.cuda.synchronize()
    f, cuh = flat.cpu().numpy(), cu.cpu().numpy()
    ctxs = [f[cuh[b]:cuh[b + 1]] for b in range(len(cuh) - 1)]
    want, wcnt = ngram.propose_batch(ctxs, min_n, max_n, k, mml)
    n, c, d = n.cpu().numpy(), c.cpu().numpy(), d.cpu().numpy()
    np.testing.assert_array_equal(n, wcnt)
    np.testing.assert_array_equal(c, np.concatenate([[0], np.cumsum(wcnt)]))
    for b in range(len(ctxs)):
        np.testing.assert_array_equal(d[c[b]:c[b + 1]], want[b, :wcnt[b]])
    return wcnt


@pytest.mark.parametrize("B,length,vocab,min_n,max_n,k", [
    (64, 4096, 151936, 3, 8, 5),      # the pages' n-gram settings on 4K contexts
    (200, (1, 900), 50, 1, 4, 7),     # tiny vocabulary: many matches, ragged lengths
    (37, (0, 3000), 32000, 2, 64, 32),
])
def test_ngram_parity(B, length, vocab, min_n, max_n, k):
    flat, cu = W.make_contexts(B, length, vocab, seed=B, device="cuda")
    print(f"[gpu-case] ngram B={B} len={length} vocab={vocab}", flush=True)
    cnt = _check(flat, cu, min_n, max_n, k, 1 << 40)
    assert cnt.sum() > 0


def test_ngram_max_model_len_and_edges():
    ctx = [[1, 2, 3, 4, 2, 3], [7, 8, 9, 1, 8, 9, 2, 7, 8, 9], [5, 5], [], [1, 2, 3, 4]]
    flat = torch.tensor([t for c in ctx for t in c], dtype=torch.int32, device="cuda")
    cu = torch.tensor(np.concatenate([[0], np.cumsum([len(c) for c in ctx])]), dtype=torch.int32, device="cuda")
    for mml in (1 << 40, 11, 10, 7):
        _check(flat, cu, 1, 3, 4, mml)


def test_proposer_then_verify():
    # n-gram drafts (no draft distribution) verified against bf16 target logits
    B, V = 32, 32000
    flat, cu = W.make_contexts(B, 2048, V, seed=5, device="cuda")
    d, n, c = rs.ngram_propose(flat, cu, min_n=3, max_n=8, k=6)
    D = int(c[-1])
    drafts = d[:D].contiguous()
    g = torch.Generator(device="cuda").manual_seed(12)
    logits = (torch.randn(D + B, V, generator=g, device="cuda") * 3).to(torch.bfloat16)
    T = torch.full((B,), 0.9, device="cuda")
    out, acc = rs.verify(logits, None, drafts, c, T, seed=21, max_k=6)
    torch.cuda.synchronize()
    o = oracle.verify(logits.cpu(), None, drafts.cpu(), c.cpu(), T.cpu(), 21, 6)
    w = W.Workload("ngram drafts", logits, None, drafts, c, T, 21, n.cpu().tolist())
    compare(GpuResult(out.cpu().numpy(), acc.cpu().numpy()), o, w)


def test_preallocated_outputs_and_workspace():
    """Outputs and workspace passed in (poisoned first) give the allocating
    call's results, on a call and on a smaller one after it; with no request
    cu_num_draft_tokens is [0]; short buffers are refused."""
    dev = torch.device("cuda")
    out = (torch.full((64 * 8,), -7, dtype=torch.int32, device=dev), torch.full((64,), -7, dtype=torch.int32, device=dev),
           torch.full((65,), -7, dtype=torch.int32, device=dev))
    ws = torch.full((64 * 8,), -7, dtype=torch.int32, device=dev)
    for B, L in ((64, 1500), (23, (0, 700))):
        flat, cu = W.make_contexts(B, L, 500, seed=B + 1, device="cuda")
        print(f"[gpu-case] ngram preallocated B={B}", flush=True)
        d0, n0, c0 = rs.ngram_propose(flat, cu, min_n=2, max_n=6, k=8)
        d1, n1, c1 = rs.ngram_propose(flat, cu, min_n=2, max_n=6, k=8, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert d1.data_ptr() == out[0].data_ptr() and c1.numel() == B + 1 and n1.numel() == B
        np.testing.assert_array_equal(n1.cpu().numpy(), n0.cpu().numpy())
        np.testing.assert_array_equal(c1.cpu().numpy(), c0.cpu().numpy())
        D = int(c0[-1])
        np.testing.assert_array_equal(d1[:D].cpu().numpy(), d0[:D].cpu().numpy())
    empty_cu = torch.zeros(1, dtype=torch.int32, device=dev)
    _, n2, c2 = rs.ngram_propose(torch.zeros(0, dtype=torch.int32, device=dev), empty_cu, min_n=1, max_n=2, k=3,
                                 out=out, workspace=ws)
    torch.cuda.synchronize()
    assert n2.numel() == 0 and c2.cpu().tolist() == [0]
    flat, cu = W.make_contexts(64, 100, 50, seed=9, device="cuda")
    with pytest.raises(ValueError):
        rs.ngram_propose(flat, cu, min_n=1, max_n=2, k=9, out=out, workspace=ws)
    with pytest.raises(ValueError):
        rs.ngram_propose(flat, cu, min_n=1, max_n=2, k=8, out=out, workspace=ws[:10])
