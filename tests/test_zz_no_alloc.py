"""rs_verify_noalloc, the verify entry point for callers that cannot allocate
(it takes no workspace; its scratch is the library's fixed per-GPU array),
through the C ABI against rs_verify on the same inputs: identical tokens and
counts, on two calls in a row with the second smaller, so the second call runs
on scratch the first one left behind; on forced paths; and a size beyond the
fixed scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import rejection_sampling_verify_rs_amd as rs
import rs_workloads as W
from parity import GpuResult, compare, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device (run the CPU suite with -m 'not gpu')")
    rs.load_library()


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _with_workspace(w, path=0):
    dbg = rs.Debug(sampling_path=path) if path else None
    out, n = rs.verify(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                       seed=w.seed, max_k=w.max_k, debug=dbg)
    torch.cuda.synchronize()
    return out.cpu().numpy(), n.cpu().numpy()


def _outputs(w):
    return (torch.full((w.B, w.max_k + 1), -7, dtype=torch.int32, device="cuda"),
            torch.full((w.B,), -7, dtype=torch.int32, device="cuda"))


def test_two_calls_in_a_row_second_smaller():
    big = W.config(4, device="cuda")          # B=256 K=8 V=151936: 2.9 MB of scratch
    small = W.config(5, device="cuda", B=40)  # B=40 K=3 V=129280
    for w in (big, small):
        assert rs.workspace_size(w.B, w.D, w.max_k, w.V, w.logits.dtype) <= rs.NOALLOC_SCRATCH_BYTES
    refs = [_with_workspace(big), _with_workspace(small)]
    for rep in range(2):
        _say(f"noalloc: workload 4 then a smaller workload 5 batch, back to back (round {rep})")
        outs = []
        for w in (big, small):  # no synchronisation between the two calls
            out, n = _outputs(w)
            rs.verify_noalloc(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                              seed=w.seed, max_k=w.max_k, out=out, num_accepted=n)
            outs.append((out, n))
        torch.cuda.synchronize()
        for (out, n), (ro, rn) in zip(outs, refs):
            np.testing.assert_array_equal(out.cpu().numpy(), ro)
            np.testing.assert_array_equal(n.cpu().numpy(), rn)
    # and the small call against the oracle
    out, n = outs[1]
    compare(GpuResult(out.cpu().numpy(), n.cpu().numpy()), run_oracle(small), small)


@pytest.mark.parametrize("path", [1, 2, 3])
def test_forced_paths_after_a_larger_call(path):
    big = W.config(4, device="cuda", B=96)
    small = W.make([0, 3, 5, 1, 8, 2], 40013, temperature=[1.0, 0.0, 0.7, 1.3, 0.9, -1.0], q_mode="noise",
                   q_sigma=0.8, seed=77, gen_seed=7700, device="cuda")
    ref = _with_workspace(small, path)
    _say(f"noalloc: B=96 workload 4 then a ragged B=6 batch on path {path}")
    o1, n1 = _outputs(big)
    rs.verify_noalloc(big.logits, big.draft_probs, big.draft_token_ids, big.cu_num_draft_tokens, big.temperature,
                      seed=big.seed, max_k=big.max_k, out=o1, num_accepted=n1)
    o2, n2 = _outputs(small)
    rs.verify_noalloc(small.logits, small.draft_probs, small.draft_token_ids, small.cu_num_draft_tokens,
                      small.temperature, seed=small.seed, max_k=small.max_k, out=o2, num_accepted=n2,
                      debug=rs.Debug(sampling_path=path))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o2.cpu().numpy(), ref[0])
    np.testing.assert_array_equal(n2.cpu().numpy(), ref[1])
    np.testing.assert_array_equal(o1.cpu().numpy(), _with_workspace(big)[0])


def test_size_beyond_the_scratch_is_refused_before_any_launch():
    lib = rs.load_library()
    B, K, V = 1024, 8, 151936  # needs 11.6 MB
    assert rs.workspace_size(B, B * K, K, V) > rs.NOALLOC_SCRATCH_BYTES
    dummy = 0x10000  # never dereferenced: the size check comes first
    st = lib.rs_verify_noalloc(dummy, 1, None, dummy, dummy, dummy, B, B * K, K, V, 0, dummy, dummy, None, None)
    assert st == rs.RS_ERR_WORKSPACE
    assert b"RS_NOALLOC_SCRATCH_BYTES" in lib.rs_status_string(st)
