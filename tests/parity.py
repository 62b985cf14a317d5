"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same tensors, then compare.

Bar: token ids and accepted counts bit-exact on every request the oracle does
not flag as a near tie (decision margin < 1e-6 relative).  A flagged request
must still be valid and agree with the oracle on every decision that is not
the near tie (check_flagged / compare_tree).  p(x*) within 1e-5 relative of
the oracle's fp64 value.
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


def _logit(w, row: int, x: int) -> float:
    return float(w.logits[row, x].float().item())


def check_flagged(tokens: np.ndarray, num_accepted: np.ndarray, o: oracle.OracleResult, w: W.Workload,
                  b: int) -> None:
    """Validity of a request the oracle flags as a near tie.  Several outputs
    are correct there, but every invalid one must still fail:
      - 0 <= n <= K_b, the first n tokens are the request's drafts, then one
        token in [0, V) with a finite target logit at row n, then -1;
      - unless an accept test or the top-p boundary is the near tie, n is the
        oracle's n (the accept decisions themselves are not in doubt);
      - then, if the race is the near tie, the token is the oracle's winner or
        one of its near-tied alternatives; otherwise it is the oracle's token."""
    cu = w.cu_num_draft_tokens
    s, e = int(cu[b]), int(cu[b + 1])
    K = e - s
    n = int(num_accepted[b])
    row = tokens[b]
    where = f"flagged request b={b} (flags {int(o.flags[b])}): gpu n={n} tokens={row.tolist()} " \
            f"oracle n={int(o.num_accepted[b])} tokens={o.tokens[b].tolist()}"
    assert 0 <= n <= K, where
    drafts = w.draft_token_ids[s:s + n].cpu().numpy()
    assert (row[:n] == drafts).all(), where
    assert (row[n + 1:] == -1).all(), where
    tok = int(row[n])
    assert 0 <= tok < w.V, where
    assert _logit(w, s + b + n, tok) > float("-inf"), where
    f = int(o.flags[b])
    if f & (oracle.FLAG_ACCEPT_TIE | oracle.FLAG_TOPP_TIE):
        return
    assert n == int(o.num_accepted[b]), where
    if f & oracle.FLAG_RACE_TIE:
        if not f & oracle.FLAG_CAND_OVERFLOW:
            assert tok in set(int(c) for c in o.cand[b] if c >= 0), where + f" candidates={o.cand[b].tolist()}"
    else:
        assert tok == int(o.tokens[b, n]), where


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
    fl = np.nonzero(flagged)[0]
    if fl.size:
        wc = w.to("cpu") if fl.size > 64 else w
        for b in fl:
            check_flagged(g.tokens, g.num_accepted, o, wc, int(b))
    frac = float(flagged.mean()) if flagged.size else 0.0
    if max_flag_frac is not None:
        assert frac <= max_flag_frac, f"flagged fraction {frac} > {max_flag_frac}"
    return {"requests": int(flagged.size), "flagged": int(flagged.sum()), "flag_frac": frac}


def compare_tree(out: np.ndarray, path: np.ndarray, n: np.ndarray, o, tw, max_depth: int) -> int:
    """Tree verify against the oracle: bit-exact on unflagged requests; on a
    flagged one, a valid walk (each accepted node a child of the previous one,
    its token emitted, then one token in [0, V), then -1), the oracle's depth
    and path unless an accept coin is the near tie, and then the oracle's
    token or, for a race near tie, one of its near-tied alternatives.
    Returns the number of flagged requests."""
    ok = ~o.near_tie
    bad = np.nonzero(ok & ((n != o.num_accepted) | (out != o.tokens).any(1) | (path != o.path).any(1)))[0]
    if bad.size:
        b = int(bad[0])
        raise AssertionError(f"{bad.size} unflagged requests differ; b={b}: gpu n={n[b]} out={out[b].tolist()} "
                             f"path={path[b].tolist()} oracle n={o.num_accepted[b]} out={o.tokens[b].tolist()} "
                             f"path={o.path[b].tolist()} flags={o.flags[b]}")
    cu = tw.cu_num_nodes.cpu().numpy()
    toks = tw.node_tokens.cpu().numpy()
    pars = tw.node_parents.cpu().numpy()
    for b in np.nonzero(~ok)[0]:
        b = int(b)
        s, e = int(cu[b]), int(cu[b + 1])
        d = int(n[b])
        where = f"flagged tree request b={b} (flags {int(o.flags[b])}): gpu d={d} out={out[b].tolist()} " \
                f"path={path[b].tolist()} oracle d={int(o.num_accepted[b])} out={o.tokens[b].tolist()}"
        assert 0 <= d <= max_depth, where
        prev = -1
        for i in range(d):
            node = int(path[b, i])
            assert 0 <= node < e - s and int(pars[s + node]) == prev, where
            assert int(out[b, i]) == int(toks[s + node]), where
            prev = node
        assert (path[b, d:] == -1).all() and (out[b, d + 1:] == -1).all(), where
        tok = int(out[b, d])
        assert 0 <= tok < tw.V, where
        f = int(o.flags[b])
        if f & oracle.FLAG_ACCEPT_TIE:
            continue
        assert d == int(o.num_accepted[b]) and (path[b] == o.path[b]).all(), where
        if f & oracle.FLAG_RACE_TIE:
            if not f & oracle.FLAG_CAND_OVERFLOW:
                assert tok in set(int(c) for c in o.cand[b] if c >= 0), where + f" candidates={o.cand[b].tolist()}"
        else:
            assert tok == int(o.tokens[b, d]), where
    return int((~ok).sum())


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
