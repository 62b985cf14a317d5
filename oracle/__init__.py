"""CPU oracle for the batched speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``rejection_sampling_verify_rs_amd``) never imports it, and this package
never imports the product path: the two share nothing but the seeded input
generators, which hold none of the method's arithmetic.

The arithmetic lives in ``rs_oracle.c`` (plain C, fp64); this module builds it
with gcc and marshals numpy/torch CPU arrays into it.  See the header of
``rs_oracle.c`` for what is computed and which passage of the pages each step
follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "librs_oracle.so")

FLAG_ACCEPT_TIE = 1
FLAG_RACE_TIE = 2
FLAG_ZERO_RESIDUAL = 4
FLAG_INVALID = 8
FLAG_TOPP_TIE = 16
FLAG_CAND_OVERFLOW = 32
# A zero residual (FLAG_ZERO_RESIDUAL) is an exact decision: the oracle adds
# FLAG_RACE_TIE when the perturbation could flip it.
NEAR_TIE_FLAGS = FLAG_ACCEPT_TIE | FLAG_RACE_TIE | FLAG_TOPP_TIE
# near-tied race alternatives reported per request (the winner first, -1 padded)
NCAND = 8

DEFAULT_EPS = 1e-6

_lib = None


def build() -> str:
    """Compile rs_oracle.c into librs_oracle.so (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fopenmp", "-ffp-contract=off",
           "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, u64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
    lib.rso_verify.argtypes = [P, i32, P, P, P, P, i32, i32, i32, i32, u64, i32, f64, P, P, P, P, P, i32]
    lib.rso_verify.restype = ctypes.c_int
    lib.rso_verify_filtered.argtypes = [P, i32, P, P, P, P, P, P, i32, i32, i32, i32, u64, i32, f64, P, P, P, P,
                                        P, i32]
    lib.rso_verify_filtered.restype = ctypes.c_int
    lib.rso_filtered_probs_row.argtypes = [P, i32, f64, i32, f64, f64, P, P, P]
    lib.rso_filtered_probs_row.restype = None
    lib.rso_verify_tree.argtypes = [P, i32, P, P, P, P, P, i32, i32, i32, i32, i32, u64, f64, P, P, P, P, P, i32]
    lib.rso_verify_tree.restype = ctypes.c_int
    lib.rso_probs.argtypes = [P, i32, P, P, i32, i32, P]
    lib.rso_probs.restype = ctypes.c_int
    lib.rso_softmax_row.argtypes = [P, i32, f64, P]
    lib.rso_softmax_row.restype = None
    lib.rso_philox_many.argtypes = [i64, P, P, P]
    lib.rso_philox_many.restype = None
    lib.rso_accept_uniforms.argtypes = [u64, P, P, i64, P]
    lib.rso_accept_uniforms.restype = None
    lib.rso_race_exponentials.argtypes = [u64, i32, i32, i32, i64, P]
    lib.rso_race_exponentials.restype = None
    lib.rso_race_uniform.argtypes = [u64, i32, i32, i32]
    lib.rso_race_uniform.restype = f64
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _to_numpy(t, dtype=None) -> np.ndarray:
    """torch CPU tensor or array-like -> contiguous numpy array."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            t = t.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(t)
    if dtype is not None:
        a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _logits_arg(logits):
    """Return (array, dtype code): raw bf16 bits as uint16 (code 1) or fp32 (code 0)."""
    a = _to_numpy(logits)
    if a.dtype == np.uint16:
        return a, 1
    return np.ascontiguousarray(a, dtype=np.float32), 0


@dataclass
class OracleResult:
    tokens: np.ndarray        # [B, max_k + 1] int32, -1 padded
    num_accepted: np.ndarray  # [B] int32
    flags: np.ndarray         # [B] int32, FLAG_* bits
    p_draft: np.ndarray       # [D] float64, p(x*) where evaluated, NaN elsewhere
    cand: np.ndarray          # [B, NCAND] int32: the race winner, then its near-tied alternatives, -1 padded

    @property
    def near_tie(self) -> np.ndarray:
        return (self.flags & NEAR_TIE_FLAGS) != 0


def verify(logits, draft_probs, draft_token_ids, cu_num_draft_tokens, temperature, seed: int,
           max_k: int, *, greedy_only: bool = False, eps: float = DEFAULT_EPS,
           threads: int = 0, top_k=None, top_p=None) -> OracleResult:
    """Run the oracle on one batch (see rs_oracle.c, rso_verify_filtered).
    top_k [B] int32 / top_p [B] float32 (or None) filter the target
    distribution of random requests."""
    lib = _load()
    lg, code = _logits_arg(logits)
    V = int(lg.shape[-1])
    ids = _to_numpy(draft_token_ids, np.int32)
    cu = _to_numpy(cu_num_draft_tokens, np.int32)
    B = int(cu.shape[0]) - 1
    D = int(ids.shape[0])
    T = None if temperature is None else _to_numpy(temperature, np.float32)
    q = None if draft_probs is None else _to_numpy(draft_probs, np.float32)
    if lg.size != (D + B) * V:
        raise ValueError(f"logits hold {lg.size} values, expected (D + B) * V = {(D + B) * V}")
    if q is not None and q.size != D * V:
        raise ValueError("draft_probs must be [D, V]")
    tk = None if top_k is None else _to_numpy(top_k, np.int32)
    tp = None if top_p is None else _to_numpy(top_p, np.float32)
    if (tk is not None and tk.size != B) or (tp is not None and tp.size != B):
        raise ValueError("top_k / top_p must have B entries")
    out = np.empty((B, max_k + 1), np.int32)
    nacc = np.empty(B, np.int32)
    flags = np.empty(B, np.int32)
    pd = np.empty(D, np.float64)
    cand = np.empty((B, NCAND), np.int32)
    rc = lib.rso_verify_filtered(_ptr(lg), code, _ptr(q), _ptr(ids), _ptr(cu), _ptr(T), _ptr(tk), _ptr(tp),
                                 B, D, max_k, V, int(seed) & ((1 << 64) - 1), int(greedy_only), float(eps),
                                 _ptr(out), _ptr(nacc), _ptr(flags), _ptr(pd), _ptr(cand), int(threads))
    if rc != 0:
        raise RuntimeError("oracle rejected its arguments")
    return OracleResult(out, nacc, flags, pd, cand)


@dataclass
class TreeResult:
    tokens: np.ndarray        # [B, max_depth + 1] int32, -1 padded
    path: np.ndarray          # [B, max_depth] accepted node indices (request-local), -1 padded
    num_accepted: np.ndarray  # [B] int32
    flags: np.ndarray         # [B] int32
    cand: np.ndarray          # [B, NCAND] int32: the stop race's winner, then near-tied alternatives

    @property
    def near_tie(self) -> np.ndarray:
        return (self.flags & NEAR_TIE_FLAGS) != 0


def verify_tree(logits, node_tokens, node_parents, cu_num_nodes, temperature, seed: int, max_nodes: int,
                max_depth: int, *, draft_probs=None, eps: float = DEFAULT_EPS, threads: int = 0) -> TreeResult:
    """Tree verify (rs_oracle.c, rso_verify_tree): request b's rows start at
    cu[b] + b (row 0 the root position, row 1 + i node i).  draft_probs
    (optional, fp32, one row per tree position like the logits): the extra
    token after a stop at node c comes from max(0, p - q_c) when c has
    children (a childless node's extra token follows p)."""
    lib = _load()
    lg, code = _logits_arg(logits)
    V = int(lg.shape[-1])
    q = None if draft_probs is None else _to_numpy(draft_probs, np.float32)
    tok = _to_numpy(node_tokens, np.int32)
    par = _to_numpy(node_parents, np.int32)
    cu = _to_numpy(cu_num_nodes, np.int32)
    T = _to_numpy(temperature, np.float32)
    B = int(cu.shape[0]) - 1
    N = int(tok.shape[0])
    if lg.size != (N + B) * V:
        raise ValueError("logits must hold N + B rows")
    if q is not None and q.size != (N + B) * V:
        raise ValueError("draft_probs must hold N + B rows")
    out = np.empty((B, max_depth + 1), np.int32)
    path = np.empty((B, max(max_depth, 0)), np.int32)
    nacc = np.empty(B, np.int32)
    flags = np.empty(B, np.int32)
    cand = np.empty((B, NCAND), np.int32)
    rc = lib.rso_verify_tree(_ptr(lg), code, None if q is None else _ptr(q), _ptr(tok), _ptr(par), _ptr(cu),
                             _ptr(T), B, N, int(max_nodes),
                             int(max_depth), V, int(seed) & ((1 << 64) - 1), float(eps), _ptr(out), _ptr(path),
                             _ptr(nacc), _ptr(flags), _ptr(cand), int(threads))
    if rc != 0:
        raise RuntimeError("oracle rejected its arguments")
    return TreeResult(out, path, nacc, flags, cand)


def verify_greedy(logits, draft_token_ids, cu_num_draft_tokens, max_k: int,
                  threads: int = 0) -> OracleResult:
    return verify(logits, None, draft_token_ids, cu_num_draft_tokens, None, 0, max_k,
                  greedy_only=True, threads=threads)


def probs(logits, cu_num_draft_tokens, temperature) -> np.ndarray:
    """p = softmax(l / T_b) for every row, fp64 [R, V]; NaN rows for greedy requests."""
    lib = _load()
    lg, code = _logits_arg(logits)
    V = int(lg.shape[-1])
    cu = _to_numpy(cu_num_draft_tokens, np.int32)
    T = _to_numpy(temperature, np.float32)
    B = int(cu.shape[0]) - 1
    R = lg.size // V
    out = np.empty((R, V), np.float64)
    if lib.rso_probs(_ptr(lg), code, _ptr(cu), _ptr(T), B, V, _ptr(out)) != 0:
        raise RuntimeError("oracle rejected its arguments")
    return out


def softmax_row(l: np.ndarray, T: float) -> np.ndarray:
    lib = _load()
    l = np.ascontiguousarray(l, dtype=np.float64)
    p = np.empty_like(l)
    lib.rso_softmax_row(_ptr(l), int(l.shape[0]), float(T), _ptr(p))
    return p


def filtered_probs_row(l: np.ndarray, T: float, top_k: int = 0, top_p: float = 1.0,
                       eps: float = DEFAULT_EPS):
    """Target distribution p' of one row after temperature, top-k and top-p
    (rso_filtered_probs_row).  Returns (p' [V] fp64, near_tie)."""
    lib = _load()
    l = np.ascontiguousarray(l, dtype=np.float64)
    p = np.empty_like(l)
    scratch = np.empty_like(l)
    tie = ctypes.c_int(0)
    lib.rso_filtered_probs_row(_ptr(l), int(l.shape[0]), float(T), int(top_k), float(top_p), float(eps), _ptr(p),
                               _ptr(scratch), ctypes.byref(tie))
    return p, bool(tie.value)


def philox(ctr, key) -> np.ndarray:
    """Philox4x32-10 of each row: ctr [n, 4] uint32, key [n, 2] uint32 -> [n, 4] uint32."""
    lib = _load()
    c = np.ascontiguousarray(ctr, dtype=np.uint32).reshape(-1, 4)
    k = np.ascontiguousarray(key, dtype=np.uint32).reshape(-1, 2)
    assert c.shape[0] == k.shape[0]
    out = np.empty_like(c)
    lib.rso_philox_many(c.shape[0], _ptr(c), _ptr(k), _ptr(out))
    return out


def accept_uniforms(seed: int, b, j) -> np.ndarray:
    lib = _load()
    b = np.ascontiguousarray(b, dtype=np.int32)
    j = np.ascontiguousarray(j, dtype=np.int32)
    u = np.empty(b.shape[0], np.float64)
    lib.rso_accept_uniforms(int(seed), _ptr(b), _ptr(j), b.shape[0], _ptr(u))
    return u


def race_exponentials(seed: int, b: int, j: int, x0: int, n: int) -> np.ndarray:
    lib = _load()
    e = np.empty(n, np.float64)
    lib.rso_race_exponentials(int(seed), int(b), int(j), int(x0), int(n), _ptr(e))
    return e


def race_uniform(seed: int, b: int, j: int, x: int) -> float:
    return _load().rso_race_uniform(int(seed), int(b), int(j), int(x))
