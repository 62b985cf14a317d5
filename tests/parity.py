"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same tensors, then compare.

Bar (see the design notes): token ids and accepted counts bit-exact on every
request the oracle does not flag as a near tie (decision margin < 1e-6
relative); flagged requests only need valid output.  p(x*) within 1e-5
relative of the oracle's fp64 value.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import oracle
import rejection_sampling_verify_rs_amd as rs
import rs_workloads as W

P_RTOL = 1e-5


@dataclass
class GpuResult:
    tokens: np.ndarray
    num_accepted: np.ndarray
    p_draft: Optional[np.ndarray] = None
    probs: Optional[np.ndarray] = None


def run_gpu(w: W.Workload, *, greedy_entry: bool = False, want_p: bool = False, want_probs: bool = False,
            row_nv: int = 0, race_tpt: int = 0, path: int = 0, phases=()) -> GpuResult:
    dev = torch.device("cuda")
    w = w.to(dev)
    if greedy_entry:
        out, n = rs.verify_greedy(w.logits, w.draft_token_ids, w.cu_num_draft_tokens, max_k=w.max_k)
        torch.cuda.synchronize()
        return GpuResult(out.cpu().numpy(), n.cpu().numpy())
    dbg = None
    if want_p or want_probs or row_nv or race_tpt or path or phases:
        dbg = rs.Debug(row_vectors_per_thread=row_nv, race_tokens_per_thread=race_tpt, sampling_path=path,
                       phase_ends=tuple(phases))
        if want_p:
            dbg.draft_target_prob = torch.full((max(w.D, 1),), float("nan"), dtype=torch.float64, device=dev)
        if want_probs:
            dbg.probs = torch.full((w.D + w.B, w.V), float("nan"), dtype=torch.float32, device=dev)
    out, n = rs.verify(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                       seed=w.seed, max_k=w.max_k, debug=dbg, top_k=w.top_k, top_p=w.top_p)
    torch.cuda.synchronize()
    r = GpuResult(out.cpu().numpy(), n.cpu().numpy())
    if want_p:
        r.p_draft = dbg.draft_target_prob.cpu().numpy()[: w.D]
    if want_probs:
        r.probs = dbg.probs.cpu().numpy()
    return r


def run_oracle(w: W.Workload, *, greedy_entry: bool = False) -> oracle.OracleResult:
    w = w.to("cpu")
    if greedy_entry:
        return oracle.verify_greedy(w.logits, w.draft_token_ids, w.cu_num_draft_tokens, w.max_k)
    return oracle.verify(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                         w.seed, w.max_k, top_k=w.top_k, top_p=w.top_p)


def compare(g: GpuResult, o: oracle.OracleResult, w: W.Workload, *, max_flag_frac: Optional[float] = None) -> dict:
    """Assert the parity bar; return a small report."""
    flagged = o.near_tie
    ok = ~flagged
    bad = np.nonzero(ok & ((g.num_accepted != o.num_accepted) | (g.tokens != o.tokens).any(axis=1)))[0]
    if bad.size:
        b = int(bad[0])
        raise AssertionError(
            f"{bad.size} unflagged request(s) differ, first b={b}: gpu n={g.num_accepted[b]} "
            f"tokens={g.tokens[b].tolist()} oracle n={o.num_accepted[b]} tokens={o.tokens[b].tolist()} "
            f"flags={int(o.flags[b])}")
    # flagged requests: only validity
    ks = np.asarray(w.num_draft)
    for b in np.nonzero(flagged)[0]:
        n = int(g.num_accepted[b])
        assert 0 <= n <= ks[b]
        row = g.tokens[b]
        assert 0 <= row[n] < w.V and (row[n + 1:] == -1).all()
    frac = float(flagged.mean()) if flagged.size else 0.0
    if max_flag_frac is not None:
        assert frac <= max_flag_frac, f"flagged fraction {frac} > {max_flag_frac}"
    return {"requests": int(flagged.size), "flagged": int(flagged.sum()), "flag_frac": frac}


def compare_p(g: GpuResult, o: oracle.OracleResult, w: Optional[W.Workload] = None) -> float:
    """p(x*) at every position the oracle evaluated, within P_RTOL relative.  Returns the max rel error.

    With the workload w, positions of requests whose top-p boundary is a near
    tie (FLAG_TOPP_TIE: the cumulative mass just above the boundary value lies
    within the tie margin of top_p times the mass) are left out: the kept set,
    and with it S' and p'(x*), then has two valid values, like the tokens of
    any flagged request."""
    have = ~np.isnan(o.p_draft)
    if w is not None:
        cu = w.cu_num_draft_tokens.cpu().numpy().astype(np.int64)
        slot_req = np.repeat(np.arange(cu.size - 1), np.diff(cu))
        have &= ((o.flags & oracle.FLAG_TOPP_TIE) == 0)[slot_req]
    if not have.any():
        return 0.0
    pg, po = g.p_draft[have], o.p_draft[have]
    tiny = po < 2.0 ** -100
    rel = np.abs(pg[~tiny] - po[~tiny]) / po[~tiny]
    assert np.all(np.abs(pg[tiny]) <= 2.0 ** -99)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= P_RTOL, f"p(x*) relative error {worst}"
    return worst
