"""MI355X-native batched speculative-sampling verify.

A thin ctypes binding over ``librs_verify.so`` (the C ABI declared in
``include/rs_verify.h``).  It only marshals arguments: every step of the verify
path runs in the library's HIP kernels on the caller's current HIP stream.
PyTorch provides device memory and the stream.

If the library has not been built this module raises on first use; build it
with ``python -m rejection_sampling_verify_rs_amd.build``.  There is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

__all__ = ["verify", "verify_greedy", "verify_noalloc", "workspace_size", "NOALLOC_SCRATCH_BYTES", "Debug",
           "RsVerifyError", "load_library", "accept_stats_accumulate", "accept_rate", "accept_length", "verify_tree", "MAX_SPEC_LEN",
           "MAX_TREE_NODES", "STATS_COUNTERS", "ngram_propose",
           "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librs_verify.so")
MAX_SPEC_LEN = 32
MAX_TREE_NODES = 64
STATS_SCALARS = 5
STATS_COUNTERS = STATS_SCALARS + MAX_SPEC_LEN
NOALLOC_SCRATCH_BYTES = 8 << 20  # RS_NOALLOC_SCRATCH_BYTES

RS_OK, RS_ERR_INVALID_ARG, RS_ERR_UNSUPPORTED, RS_ERR_WORKSPACE, RS_ERR_HIP = range(5)
RS_F32, RS_BF16 = 0, 1
_DTYPE = {torch.float32: RS_F32, torch.bfloat16: RS_BF16}

_lib = None


class RsVerifyError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class _RsDebug(ctypes.Structure):
    _fields_ = [
        ("draft_target_prob", ctypes.c_void_p),
        ("probs", ctypes.c_void_p),
        ("events", ctypes.c_void_p),
        ("num_events", ctypes.c_int32),
        ("kernels_launched", ctypes.c_void_p),
        ("row_vectors_per_thread", ctypes.c_int32),
        ("race_tokens_per_thread", ctypes.c_int32),
        ("sampling_path", ctypes.c_int32),
        ("phase_ends", ctypes.c_int32 * 3),
        ("path_taken", ctypes.c_void_p),
    ]


def load_library(path: str = LIB_PATH):
    """Load librs_verify.so once; raise loudly if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m rejection_sampling_verify_rs_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    lib.rs_verify_workspace_size.argtypes = [i32, i32, i32, i32, ctypes.c_int]
    lib.rs_verify_workspace_size.restype = sz
    lib.rs_verify_filtered_workspace_size.argtypes = [i32, i32, i32, i32, ctypes.c_int]
    lib.rs_verify_filtered_workspace_size.restype = sz
    lib.rs_verify.argtypes = [P, ctypes.c_int, P, P, P, P, i32, i32, i32, i32, u64, P, P, P, sz, P, P]
    lib.rs_verify.restype = ctypes.c_int
    lib.rs_verify_noalloc.argtypes = [P, ctypes.c_int, P, P, P, P, i32, i32, i32, i32, u64, P, P, P, P]
    lib.rs_verify_noalloc.restype = ctypes.c_int
    lib.rs_verify_filtered.argtypes = [P, ctypes.c_int, P, P, P, P, P, P, i32, i32, i32, i32, u64, P, P, P, sz, P,
                                       P]
    lib.rs_verify_filtered.restype = ctypes.c_int
    lib.rs_verify_greedy.argtypes = [P, ctypes.c_int, P, P, i32, i32, i32, i32, P, P, P, sz, P]
    lib.rs_verify_greedy.restype = ctypes.c_int
    lib.rs_verify_tree.argtypes = [P, ctypes.c_int, P, P, P, P, P, i32, i32, i32, i32, i32, u64, P, P, P, P, sz, P]
    lib.rs_verify_tree_workspace_size.argtypes = [i32, i32]
    lib.rs_verify_tree_workspace_size.restype = sz
    lib.rs_verify_tree.restype = ctypes.c_int
    lib.rs_ngram_propose.argtypes = [P, P, i32, i32, i32, i32, i32, ctypes.c_int64, P, P, P, P, sz, P]
    lib.rs_ngram_propose.restype = ctypes.c_int
    lib.rs_accept_stats_accumulate.argtypes = [P, P, i32, P, P]
    lib.rs_accept_stats_accumulate.restype = ctypes.c_int
    lib.rs_accept_rate.argtypes = [P]
    lib.rs_accept_rate.restype = ctypes.c_double
    lib.rs_accept_length.argtypes = [P]
    lib.rs_accept_length.restype = ctypes.c_double
    lib.rs_status_string.argtypes = [ctypes.c_int]
    lib.rs_status_string.restype = ctypes.c_char_p
    lib.rs_abi_version.argtypes = []
    lib.rs_abi_version.restype = i32
    _lib = lib
    return lib


def _check(status: int):
    if status != RS_OK:
        msg = load_library().rs_status_string(status).decode()
        raise RsVerifyError(status, msg)


def workspace_size(batch: int, total_draft_tokens: int, max_k: int, vocab: int,
                   dtype: torch.dtype = torch.bfloat16, filtered: bool = False) -> int:
    """Workspace bytes for rs_verify / rs_verify_greedy, or for rs_verify_filtered
    with top-k / top-p (filtered=True)."""
    if dtype not in _DTYPE:
        raise ValueError(f"unsupported logits dtype {dtype}")
    lib = load_library()
    f = lib.rs_verify_filtered_workspace_size if filtered else lib.rs_verify_workspace_size
    return int(f(batch, total_draft_tokens, max_k, vocab, _DTYPE[dtype]))


@dataclass
class Debug:
    """Optional parity / profiling outputs (see rs_debug in include/rs_verify.h)."""
    draft_target_prob: Optional[torch.Tensor] = None  # [D] float64
    probs: Optional[torch.Tensor] = None              # [R, V] float32
    events: Optional[Sequence[torch.cuda.Event]] = None  # [0] before the first kernel, [k] after the k-th
    row_vectors_per_thread: int = 0
    race_tokens_per_thread: int = 0
    sampling_path: int = 0          # 0 automatic, 1 per-request, 2 phased split, 3 stream
    phase_ends: Sequence[int] = ()   # () automatic, (-1,) one phase, else positions where phases end
    kernels_launched: Optional[int] = None  # set after the call
    path_taken: Optional[int] = None        # set after the call: 1, 2 or 3

    def _struct(self, stream) -> Tuple[_RsDebug, object]:
        d = _RsDebug()
        d.draft_target_prob = self.draft_target_prob.data_ptr() if self.draft_target_prob is not None else None
        d.probs = self.probs.data_ptr() if self.probs is not None else None
        count = ctypes.c_int32(0)
        path = ctypes.c_int32(0)
        keep = [count, path]
        if self.events is not None:
            for e in self.events:  # torch creates the HIP event on first record
                if e.cuda_event == 0:
                    e.record(stream)
            arr = (ctypes.c_void_p * len(self.events))(*[e.cuda_event for e in self.events])
            keep.append(arr)
            d.events = ctypes.cast(arr, ctypes.c_void_p)
            d.num_events = len(self.events)
        d.kernels_launched = ctypes.cast(ctypes.pointer(count), ctypes.c_void_p)
        d.path_taken = ctypes.cast(ctypes.pointer(path), ctypes.c_void_p)
        d.row_vectors_per_thread = int(self.row_vectors_per_thread)
        d.race_tokens_per_thread = int(self.race_tokens_per_thread)
        d.sampling_path = int(self.sampling_path)
        ends = list(self.phase_ends)[:3]
        for i, v in enumerate(ends):
            d.phase_ends[i] = int(v)
        return d, keep


def _dev_tensor(t: torch.Tensor, name: str, dtype, device) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _common(target_logits, draft_token_ids, cu_num_draft_tokens, max_k, out, num_accepted, workspace,
            stream, filtered=False):
    if not isinstance(target_logits, torch.Tensor) or target_logits.device.type != "cuda":
        raise ValueError("target_logits must be a CUDA (HIP) tensor")
    dev = target_logits.device
    if target_logits.dtype not in _DTYPE:
        raise TypeError(f"target_logits must be float32 or bfloat16, got {target_logits.dtype}")
    _dev_tensor(target_logits, "target_logits", None, dev)
    _dev_tensor(draft_token_ids, "draft_token_ids", torch.int32, dev)
    _dev_tensor(cu_num_draft_tokens, "cu_num_draft_tokens", torch.int32, dev)
    if target_logits.dim() < 2:
        raise ValueError("target_logits must be [R, V] or [B, K+1, V]")
    V = int(target_logits.shape[-1])
    B = int(cu_num_draft_tokens.numel()) - 1
    D = int(draft_token_ids.numel())
    if B < 0:
        raise ValueError("cu_num_draft_tokens needs B + 1 entries")
    if target_logits.numel() != (D + B) * V:
        raise ValueError(f"target_logits has {target_logits.numel() // max(V, 1)} rows, expected D + B = {D + B}")
    if max_k is None:
        raise ValueError("max_k (max drafts per request) is required")
    if out is None:
        out = torch.empty((B, max_k + 1), dtype=torch.int32, device=dev)
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    _dev_tensor(out, "out", torch.int32, dev)
    _dev_tensor(num_accepted, "num_accepted", torch.int32, dev)
    if out.numel() != B * (max_k + 1) or num_accepted.numel() != B:
        raise ValueError("out must hold B * (max_k + 1) and num_accepted B int32 values")
    if workspace is None:
        n = workspace_size(B, D, max_k, V, target_logits.dtype, filtered) if B > 0 else 0
        workspace = torch.empty((max(n, 1),), dtype=torch.uint8, device=dev)
    _dev_tensor(workspace, "workspace", torch.uint8, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return dev, B, D, V, out, num_accepted, workspace, stream


def verify(target_logits: torch.Tensor, draft_probs: Optional[torch.Tensor], draft_token_ids: torch.Tensor,
           cu_num_draft_tokens: torch.Tensor, temperature: torch.Tensor, *, seed: int, max_k: int,
           out: Optional[torch.Tensor] = None, num_accepted: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, debug: Optional[Debug] = None,
           stream: Optional[torch.cuda.Stream] = None, top_k: Optional[torch.Tensor] = None,
           top_p: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Batched verify.  Returns (output_token_ids [B, max_k+1], num_accepted [B]).

    With top_k ([B] int32) and / or top_p ([B] float32) it calls
    rs_verify_filtered (target distribution filtered per request), else
    rs_verify."""
    lib = load_library()
    dev, B, D, V, out, num_accepted, workspace, stream = _common(
        target_logits, draft_token_ids, cu_num_draft_tokens, max_k, out, num_accepted, workspace, stream,
        filtered=top_k is not None or top_p is not None)
    _dev_tensor(temperature, "temperature", torch.float32, dev)
    if temperature.numel() != B:
        raise ValueError("temperature must have B entries")
    if draft_probs is not None:
        _dev_tensor(draft_probs, "draft_probs", torch.float32, dev)
        if draft_probs.numel() != D * V:
            raise ValueError("draft_probs must be [D, V]")
    for t, name, dt in ((top_k, "top_k", torch.int32), (top_p, "top_p", torch.float32)):
        if t is not None:
            _dev_tensor(t, name, dt, dev)
            if t.numel() != B:
                raise ValueError(f"{name} must have B entries")
    dbg, keep = (None, None)
    if debug is not None:
        dbg, keep = debug._struct(stream)
    head = (target_logits.data_ptr(), _DTYPE[target_logits.dtype],
            draft_probs.data_ptr() if draft_probs is not None else None,
            draft_token_ids.data_ptr() if D > 0 else None, cu_num_draft_tokens.data_ptr(), temperature.data_ptr())
    tail = (B, D, int(max_k), V, int(seed) & ((1 << 64) - 1), out.data_ptr(), num_accepted.data_ptr(),
            workspace.data_ptr(), workspace.numel(), ctypes.byref(dbg) if dbg is not None else None,
            ctypes.c_void_p(stream.cuda_stream))
    if top_k is None and top_p is None:
        status = lib.rs_verify(*head, *tail)
    else:
        status = lib.rs_verify_filtered(*head, top_k.data_ptr() if top_k is not None else None,
                                        top_p.data_ptr() if top_p is not None else None, *tail)
    if debug is not None:
        debug.kernels_launched = int(keep[0].value)
        debug.path_taken = int(keep[1].value)
    del keep
    _check(status)
    return out, num_accepted


def verify_noalloc(target_logits: torch.Tensor, draft_probs: Optional[torch.Tensor], draft_token_ids: torch.Tensor,
                   cu_num_draft_tokens: torch.Tensor, temperature: torch.Tensor, *, seed: int, max_k: int,
                   out: torch.Tensor, num_accepted: torch.Tensor, debug: Optional[Debug] = None,
                   stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """rs_verify_noalloc: rs_verify with the library's own fixed scratch and no
    workspace argument, for callers that cannot allocate.  The caller passes
    the outputs (out [B, max_k+1] int32, num_accepted [B] int32); this binding
    allocates nothing either.  Calls that overlap on one GPU race on the
    shared scratch."""
    lib = load_library()
    if not isinstance(target_logits, torch.Tensor) or target_logits.device.type != "cuda":
        raise ValueError("target_logits must be a CUDA (HIP) tensor")
    if target_logits.dtype not in _DTYPE:
        raise TypeError(f"target_logits must be float32 or bfloat16, got {target_logits.dtype}")
    dev = target_logits.device
    _dev_tensor(target_logits, "target_logits", None, dev)
    _dev_tensor(draft_token_ids, "draft_token_ids", torch.int32, dev)
    _dev_tensor(cu_num_draft_tokens, "cu_num_draft_tokens", torch.int32, dev)
    _dev_tensor(temperature, "temperature", torch.float32, dev)
    _dev_tensor(out, "out", torch.int32, dev)
    _dev_tensor(num_accepted, "num_accepted", torch.int32, dev)
    V = int(target_logits.shape[-1])
    B = int(cu_num_draft_tokens.numel()) - 1
    D = int(draft_token_ids.numel())
    if B < 0 or target_logits.numel() != (D + B) * V or temperature.numel() != B:
        raise ValueError("expected target_logits [D + B, V], temperature [B], cu_num_draft_tokens [B + 1]")
    if out.numel() != B * (max_k + 1) or num_accepted.numel() != B:
        raise ValueError("out must hold B * (max_k + 1) and num_accepted B int32 values")
    if draft_probs is not None:
        _dev_tensor(draft_probs, "draft_probs", torch.float32, dev)
        if draft_probs.numel() != D * V:
            raise ValueError("draft_probs must be [D, V]")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    dbg, keep = (None, None)
    if debug is not None:
        dbg, keep = debug._struct(stream)
    status = lib.rs_verify_noalloc(
        target_logits.data_ptr(), _DTYPE[target_logits.dtype],
        draft_probs.data_ptr() if draft_probs is not None else None, draft_token_ids.data_ptr() if D > 0 else None,
        cu_num_draft_tokens.data_ptr(), temperature.data_ptr(), B, D, int(max_k), V, int(seed) & ((1 << 64) - 1),
        out.data_ptr(), num_accepted.data_ptr(), ctypes.byref(dbg) if dbg is not None else None,
        ctypes.c_void_p(stream.cuda_stream))
    if debug is not None:
        debug.kernels_launched = int(keep[0].value)
        debug.path_taken = int(keep[1].value)
    del keep
    _check(status)
    return out, num_accepted


def verify_greedy(target_logits: torch.Tensor, draft_token_ids: torch.Tensor, cu_num_draft_tokens: torch.Tensor,
                  *, max_k: int, out: Optional[torch.Tensor] = None, num_accepted: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Greedy argmax-match verify (rs_verify_greedy)."""
    lib = load_library()
    dev, B, D, V, out, num_accepted, workspace, stream = _common(
        target_logits, draft_token_ids, cu_num_draft_tokens, max_k, out, num_accepted, workspace, stream)
    status = lib.rs_verify_greedy(
        target_logits.data_ptr(), _DTYPE[target_logits.dtype], draft_token_ids.data_ptr() if D > 0 else None,
        cu_num_draft_tokens.data_ptr(), B, D, int(max_k), V, out.data_ptr(), num_accepted.data_ptr(),
        workspace.data_ptr(), workspace.numel(), ctypes.c_void_p(stream.cuda_stream))
    _check(status)
    return out, num_accepted


def accept_stats_accumulate(num_accepted: torch.Tensor, cu_num_draft_tokens: torch.Tensor,
                            counters: Optional[torch.Tensor] = None,
                            stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Add one verify step to the running acceptance counters
    (rs_accept_stats_accumulate); counters is an int64 [STATS_COUNTERS] device
    tensor (created zeroed when None).  Returns counters."""
    lib = load_library()
    if not isinstance(num_accepted, torch.Tensor) or num_accepted.device.type != "cuda":
        raise ValueError("num_accepted must be a CUDA (HIP) tensor")
    dev = num_accepted.device
    _dev_tensor(num_accepted, "num_accepted", torch.int32, dev)
    _dev_tensor(cu_num_draft_tokens, "cu_num_draft_tokens", torch.int32, dev)
    B = int(num_accepted.numel())
    if cu_num_draft_tokens.numel() != B + 1:
        raise ValueError("cu_num_draft_tokens needs B + 1 entries")
    if counters is None:
        counters = torch.zeros(STATS_COUNTERS, dtype=torch.int64, device=dev)
    _dev_tensor(counters, "counters", torch.int64, dev)
    if counters.numel() != STATS_COUNTERS:
        raise ValueError(f"counters must hold {STATS_COUNTERS} int64 values")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _check(lib.rs_accept_stats_accumulate(num_accepted.data_ptr(), cu_num_draft_tokens.data_ptr(), B,
                                          counters.data_ptr(), ctypes.c_void_p(stream.cuda_stream)))
    return counters


def _host_counters(counters) -> "torch.Tensor":
    c = counters.detach().to("cpu", torch.int64).contiguous()
    if c.numel() != STATS_COUNTERS:
        raise ValueError(f"counters must hold {STATS_COUNTERS} int64 values")
    return c


def accept_rate(counters) -> float:
    """alpha = accepted / proposed draft tokens (rs_accept_rate on a host copy)."""
    c = _host_counters(counters)
    return float(load_library().rs_accept_rate(c.data_ptr()))


def accept_length(counters) -> float:
    """tau = emitted tokens / verifies (rs_accept_length on a host copy)."""
    c = _host_counters(counters)
    return float(load_library().rs_accept_length(c.data_ptr()))


def verify_tree(target_logits: torch.Tensor, node_tokens: torch.Tensor, node_parents: torch.Tensor,
                cu_num_nodes: torch.Tensor, temperature: torch.Tensor, *, seed: int, max_nodes: int, max_depth: int,
                draft_probs: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                accepted_nodes: Optional[torch.Tensor] = None, num_accepted: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None):
    """Tree verify (rs_verify_tree).  draft_probs (optional, fp32, one row per
    tree position like target_logits): the extra token after a stop comes from
    max(0, p - q) of the stop node's row.  Returns (output_token_ids
    [B, max_depth+1], accepted_nodes [B, max_depth], num_accepted [B])."""
    lib = load_library()
    if not isinstance(target_logits, torch.Tensor) or target_logits.device.type != "cuda":
        raise ValueError("target_logits must be a CUDA (HIP) tensor")
    dev = target_logits.device
    if target_logits.dtype not in _DTYPE:
        raise TypeError(f"target_logits must be float32 or bfloat16, got {target_logits.dtype}")
    _dev_tensor(target_logits, "target_logits", None, dev)
    for t, name in ((node_tokens, "node_tokens"), (node_parents, "node_parents"), (cu_num_nodes, "cu_num_nodes")):
        _dev_tensor(t, name, torch.int32, dev)
    _dev_tensor(temperature, "temperature", torch.float32, dev)
    V = int(target_logits.shape[-1])
    B = int(cu_num_nodes.numel()) - 1
    N = int(node_tokens.numel())
    if B < 0 or node_parents.numel() != N or temperature.numel() != B:
        raise ValueError("node_parents needs N entries, temperature B, cu_num_nodes B + 1")
    if target_logits.numel() != (N + B) * V:
        raise ValueError(f"target_logits must hold N + B = {N + B} rows")
    if draft_probs is not None:
        _dev_tensor(draft_probs, "draft_probs", torch.float32, dev)
        if draft_probs.numel() != (N + B) * V:
            raise ValueError(f"draft_probs must hold N + B = {N + B} rows of V")
    if out is None:
        out = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    if accepted_nodes is None:
        accepted_nodes = torch.empty((B, max_depth), dtype=torch.int32, device=dev)
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    for t, name, n in ((out, "out", B * (max_depth + 1)), (accepted_nodes, "accepted_nodes", B * max_depth),
                       (num_accepted, "num_accepted", B)):
        _dev_tensor(t, name, torch.int32, dev)
        if t.numel() != n:
            raise ValueError(f"{name} must hold {n} int32 values")
    if workspace is None:
        workspace = torch.empty((max(int(lib.rs_verify_tree_workspace_size(B, V)), 1),), dtype=torch.uint8,
                                device=dev)
    _dev_tensor(workspace, "workspace", torch.uint8, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _check(lib.rs_verify_tree(
        target_logits.data_ptr(), _DTYPE[target_logits.dtype],
        draft_probs.data_ptr() if draft_probs is not None else None, node_tokens.data_ptr() if N > 0 else None,
        node_parents.data_ptr() if N > 0 else None, cu_num_nodes.data_ptr(), temperature.data_ptr(), B, N,
        int(max_nodes), int(max_depth), V, int(seed) & ((1 << 64) - 1), out.data_ptr(),
        accepted_nodes.data_ptr() if max_depth > 0 else None, num_accepted.data_ptr(), workspace.data_ptr(),
        workspace.numel(), ctypes.c_void_p(stream.cuda_stream)))
    return out, accepted_nodes, num_accepted


def ngram_propose(context_token_ids: torch.Tensor, cu_context: torch.Tensor, *, min_n: int, max_n: int, k: int,
                  max_model_len: int = 1 << 62, out: Optional[tuple] = None, workspace: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None):
    """n-gram drafts (rs_ngram_propose).  Returns (draft_token_ids packed [B * k],
    num_draft_tokens [B], cu_num_draft_tokens [B + 1]); the first
    cu_num_draft_tokens[-1] drafts are valid.  out: optional preallocated
    (draft_token_ids, num_draft_tokens, cu_num_draft_tokens) int32 tensors of
    at least B * k, B and B + 1 elements; workspace: optional int32 scratch of
    at least B * k elements (with both, a call allocates nothing)."""
    lib = load_library()
    if not isinstance(context_token_ids, torch.Tensor) or context_token_ids.device.type != "cuda":
        raise ValueError("context_token_ids must be a CUDA (HIP) tensor")
    dev = context_token_ids.device
    _dev_tensor(context_token_ids, "context_token_ids", torch.int32, dev)
    _dev_tensor(cu_context, "cu_context", torch.int32, dev)
    B = int(cu_context.numel()) - 1
    if B < 0:
        raise ValueError("cu_context needs B + 1 entries")
    if out is None:
        drafts = torch.empty(max(B * k, 1), dtype=torch.int32, device=dev)
        num = torch.empty(max(B, 1), dtype=torch.int32, device=dev)[:B]
        # the pack kernel writes every prefix sum; with no request nothing runs, so cu = [0] here
        cu = torch.zeros(1, dtype=torch.int32, device=dev) if B == 0 else torch.empty(B + 1, dtype=torch.int32,
                                                                                          device=dev)
    else:
        drafts, num, cu = out
        for t, name, need in ((drafts, "draft_token_ids", B * k), (num, "num_draft_tokens", B),
                              (cu, "cu_num_draft_tokens", B + 1)):
            _dev_tensor(t, name, torch.int32, dev)
            if t.numel() < need:
                raise ValueError(f"{name} needs at least {need} elements")
        if B == 0:
            cu[:1].zero_()
    if workspace is None:
        ws = torch.empty(max(B * k, 1), dtype=torch.int32, device=dev)
    else:
        ws = workspace
        _dev_tensor(ws, "workspace", torch.int32, dev)
        if ws.numel() < B * k:
            raise ValueError(f"workspace needs at least {B * k} int32 elements")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    T = int(context_token_ids.numel())
    _check(lib.rs_ngram_propose(context_token_ids.data_ptr() if T > 0 else None, cu_context.data_ptr(), B, T,
                                int(min_n), int(max_n), int(k), int(max_model_len), drafts.data_ptr(),
                                num.data_ptr() if B > 0 else None, cu.data_ptr(), ws.data_ptr(),
                                ws.numel() * 4, ctypes.c_void_p(stream.cuda_stream)))
    return drafts[: B * k], num[:B], cu[: B + 1]
