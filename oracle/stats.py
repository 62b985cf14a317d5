"""Acceptance statistics of verify steps (CPU oracle).

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's
CPU baseline use this module; the product path never imports it.

Definitions, by page title and section:
  - counters a serving engine exports per verify step [第12章 投机解码：以小博大
    §12.7.5]: the number of draft proposals (requests that proposed at least
    one draft; a count of proposals, not of tokens), the number of draft
    tokens proposed, the number of draft tokens accepted, and the number of
    accepted tokens per draft position (position j counts the requests whose
    first j + 1 drafts were all accepted);
  - acceptance rate alpha = accepted / proposed draft tokens (bonus excluded)
    and acceptance length tau = emitted tokens / verify count, where every
    verify emits its accepted drafts plus one extra token
    [投机解码（Speculative Decoding）端到端深挖 §13, and its worked example].
Reading: one verify is one request in one verify step; requests whose output
is invalid (num_accepted = -1) are not counted.

Plain Python loops over the requests (the inputs are per-request integers).
"""
from __future__ import annotations

import numpy as np

MAX_POS = 32

NAMES = ("num_drafts", "num_draft_tokens", "num_accepted_tokens", "num_emitted_tokens", "num_verifies")


def accumulate(counters, num_accepted, cu_num_draft_tokens):
    """Add one verify step to the running counters (dict of ints plus
    'accepted_per_pos' list of MAX_POS ints); returns the updated dict."""
    c = dict(counters) if counters else {k: 0 for k in NAMES}
    per_pos = list(c.get("accepted_per_pos", [0] * MAX_POS))
    n = [int(x) for x in np.asarray(num_accepted).reshape(-1)]
    cu = [int(x) for x in np.asarray(cu_num_draft_tokens).reshape(-1)]
    for b in range(len(n)):
        if n[b] < 0:
            continue  # invalid request: nothing was verified
        k = cu[b + 1] - cu[b]
        if k > 0:
            c["num_drafts"] += 1
        c["num_draft_tokens"] += k
        c["num_accepted_tokens"] += n[b]
        c["num_emitted_tokens"] += n[b] + 1
        c["num_verifies"] += 1
        for j in range(n[b]):
            per_pos[j] += 1
    c["accepted_per_pos"] = per_pos
    return c


def accept_rate(c) -> float:
    """alpha = accepted draft tokens / proposed draft tokens."""
    return c["num_accepted_tokens"] / c["num_draft_tokens"] if c["num_draft_tokens"] else float("nan")


def accept_length(c) -> float:
    """tau = emitted tokens / verifies (accepted drafts plus the extra token per verify)."""
    return c["num_emitted_tokens"] / c["num_verifies"] if c["num_verifies"] else float("nan")


def to_array(c) -> np.ndarray:
    """Counters in the library's layout: 5 scalars then MAX_POS per-position counts (int64)."""
    return np.array([c[k] for k in NAMES] + list(c["accepted_per_pos"]), np.int64)
