"""n-gram (prompt lookup) draft proposer -- CPU oracle.

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's
CPU baseline use this module; the product path never imports it.

What it computes [第12章 投机解码：以小博大 §12.4.4 (the n-gram proposer:
pattern matching over the request's own context, longer n-grams first, up to
k tokens copied after the match)]:
  k_eff = min(k, max_model_len - len(context)); no proposal if k_eff <= 0;
  for n = max_n, max_n - 1, ..., min_n:
      pattern = the last n tokens of the context;
      find the leftmost start s of an occurrence of the pattern that ends
      before the pattern itself begins (s + n <= len(context) - n);
      if found, propose context[s + n : s + n + k_eff] (fewer tokens when the
      context ends first) and stop;
  no proposal if no n matches.
The pages implement the search with KMP; the leftmost occurrence is a plain
definition, so the oracle scans start positions in order (numpy compares a
window per start).
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np


def propose(context: Sequence[int], min_n: int, max_n: int, k: int, max_model_len: int) -> List[int]:
    ctx = np.asarray(context, dtype=np.int64)
    N = int(ctx.shape[0])
    k_eff = min(k, max_model_len - N)
    if k_eff <= 0:
        return []
    for n in range(max_n, min_n - 1, -1):
        if n <= 0 or 2 * n > N:
            continue
        pattern = ctx[N - n:]
        last = N - 2 * n  # largest start whose occurrence ends before the pattern
        for s in range(0, last + 1):
            if np.array_equal(ctx[s:s + n], pattern):
                return ctx[s + n: s + n + k_eff].tolist()
    return []


def propose_batch(contexts: Sequence[Sequence[int]], min_n: int, max_n: int, k: int, max_model_len: int):
    """Per request: (padded drafts [B, k] int32 with -1, counts [B])."""
    B = len(contexts)
    out = np.full((B, k), -1, np.int32)
    cnt = np.zeros(B, np.int32)
    for b, c in enumerate(contexts):
        d = propose(c, min_n, max_n, k, max_model_len)
        out[b, :len(d)] = d
        cnt[b] = len(d)
    return out, cnt
