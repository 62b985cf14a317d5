"""C-ABI checks that need no GPU: the library loads, exports every function
include/rs_verify.h declares, and rejects bad arguments on the host before any
HIP call (NULL pointers, sizes, max_k > 32 [第12章 §12.5.4 MAX_SPEC_LEN],
dtype, alignment, workspace)."""
import ctypes
import os
import re
import subprocess

import pytest

import rejection_sampling_verify_rs_amd as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rs_verify.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rs_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return rs.load_library()


def test_header_declares_the_boundary():
    assert _declared_functions() == ["rs_abi_version", "rs_accept_length", "rs_accept_rate",
                                     "rs_accept_stats_accumulate", "rs_ngram_propose", "rs_status_string",
                                     "rs_verify",
                                     "rs_verify_filtered", "rs_verify_filtered_workspace_size", "rs_verify_greedy",
                                     "rs_verify_noalloc", "rs_verify_tree", "rs_verify_tree_workspace_size",
                                     "rs_verify_workspace_size"]


def test_library_exports_every_declared_symbol(lib):
    nm = subprocess.run(["nm", "-D", "--defined-only", rs.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (rs_\w+)", nm))
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    assert lib.rs_abi_version() == 2


def test_status_codes_as_documented(lib):
    """The status codes the header declares (RS_ERR_WORKSPACE = 3 and
    RS_ERR_HIP = 4: a workspace error is reported apart from a launch
    failure), their strings and the binding's constants."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    enum = dict((k, int(v)) for k, v in re.findall(r"\b(RS_(?:OK|ERR_[A-Z_]+))\s*=\s*(\d+)", src))
    assert enum == {"RS_OK": 0, "RS_ERR_INVALID_ARG": 1, "RS_ERR_UNSUPPORTED": 2, "RS_ERR_WORKSPACE": 3,
                    "RS_ERR_HIP": 4}
    for name, code in enum.items():
        assert lib.rs_status_string(code).decode().split(":")[0] == name
        assert getattr(rs, name) == code


def test_status_strings(lib):
    for code in range(5):
        assert lib.rs_status_string(code).decode().startswith("RS_")
    assert b"unknown" in lib.rs_status_string(99)


def test_workspace_size(lib):
    n = rs.workspace_size(256, 2048, 8, 151936)
    assert n > 0 and n % 256 == 0
    assert rs.workspace_size(256, 2048, 8, 151936, __import__("torch").float32) > 0
    assert lib.rs_verify_workspace_size(1, 0, 0, 1, 1) > 0
    assert lib.rs_verify_workspace_size(0, 0, 4, 10, 1) == 0      # empty batch needs nothing
    assert lib.rs_verify_workspace_size(-1, 0, 4, 10, 1) == 0
    assert lib.rs_verify_workspace_size(2, 0, 33, 10, 1) == 0     # max_k > 32
    assert lib.rs_verify_workspace_size(2, 9, 4, 10, 1) == 0      # D > B * max_k
    assert lib.rs_verify_workspace_size(2, 4, 4, 0, 1) == 0       # V < 1
    assert lib.rs_verify_workspace_size(2, 4, 4, 10, 5) == 0      # dtype
    # grows with the batch
    assert rs.workspace_size(512, 4096, 8, 151936) > n
    # the filtered entry point adds one fp32 maximum per 4096-byte row segment
    nf = rs.workspace_size(256, 2048, 8, 151936, filtered=True)
    assert nf >= n + 2304 * 5 * 256 * 4
    assert lib.rs_verify_filtered_workspace_size(2, 9, 4, 10, 1) == 0


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# The calls below pass non-NULL dummy addresses that are never valid device
# memory.  Each call must fail validation on the host; they are skipped on a
# GPU machine so a validation bug can never launch a kernel on them.
needs_no_gpu = pytest.mark.skipif(_gpu_present(), reason="host-validation tests use dummy pointers")

DUMMY = 0x10000  # 16-byte aligned, never dereferenced


def _call(lib, **kw):
    a = dict(logits=DUMMY, dtype=1, q=None, draft=DUMMY, cu=DUMMY, T=DUMMY, B=2, D=4, max_k=2, V=100, seed=0,
             out=DUMMY, nacc=DUMMY, ws=DUMMY, ws_bytes=1 << 30, dbg=None, stream=None)
    a.update(kw)
    return lib.rs_verify(a["logits"], a["dtype"], a["q"], a["draft"], a["cu"], a["T"], a["B"], a["D"], a["max_k"],
                         a["V"], a["seed"], a["out"], a["nacc"], a["ws"], a["ws_bytes"], a["dbg"], a["stream"])


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), rs.RS_ERR_INVALID_ARG),
    (dict(D=-1), rs.RS_ERR_INVALID_ARG),
    (dict(V=0), rs.RS_ERR_INVALID_ARG),
    (dict(max_k=-1), rs.RS_ERR_INVALID_ARG),
    (dict(max_k=33, D=4), rs.RS_ERR_INVALID_ARG),
    (dict(D=5), rs.RS_ERR_INVALID_ARG),                 # D > B * max_k
    (dict(dtype=2), rs.RS_ERR_UNSUPPORTED),
    (dict(logits=None), rs.RS_ERR_INVALID_ARG),
    (dict(cu=None), rs.RS_ERR_INVALID_ARG),
    (dict(T=None), rs.RS_ERR_INVALID_ARG),
    (dict(out=None), rs.RS_ERR_INVALID_ARG),
    (dict(nacc=None), rs.RS_ERR_INVALID_ARG),
    (dict(draft=None), rs.RS_ERR_INVALID_ARG),
    (dict(logits=DUMMY + 1), rs.RS_ERR_UNSUPPORTED),    # bf16 needs 2-byte alignment
    (dict(logits=DUMMY + 2, dtype=0), rs.RS_ERR_UNSUPPORTED),  # fp32 needs 4-byte alignment
    (dict(q=DUMMY + 2), rs.RS_ERR_UNSUPPORTED),
    (dict(cu=DUMMY + 1), rs.RS_ERR_UNSUPPORTED),
    (dict(ws=None), rs.RS_ERR_WORKSPACE),
    (dict(ws=DUMMY + 8), rs.RS_ERR_WORKSPACE),
    (dict(ws_bytes=16), rs.RS_ERR_WORKSPACE),
])
def test_host_validation_rejects(lib, kw, status):
    assert _call(lib, **kw) == status


@needs_no_gpu
def test_empty_batch_is_a_no_op(lib):
    assert _call(lib, B=0, D=0, logits=None, out=None, nacc=None, ws=None) == rs.RS_OK


@needs_no_gpu
def test_debug_knobs_validated(lib):
    d = rs._RsDebug()
    d.row_vectors_per_thread = 3
    assert _call(lib, dbg=ctypes.byref(d)) == rs.RS_ERR_INVALID_ARG
    d.row_vectors_per_thread = 0
    d.race_tokens_per_thread = 12
    assert _call(lib, dbg=ctypes.byref(d)) == rs.RS_ERR_INVALID_ARG
    d.race_tokens_per_thread = 0
    d.sampling_path = 4
    assert _call(lib, dbg=ctypes.byref(d)) == rs.RS_ERR_INVALID_ARG
    d.sampling_path = 0
    d.num_events = 3  # events array missing
    assert _call(lib, dbg=ctypes.byref(d)) == rs.RS_ERR_INVALID_ARG


@needs_no_gpu
def test_noalloc_entry_validation(lib):
    """rs_verify_noalloc: the argument checks of rs_verify, and a call whose
    workspace would exceed the library's fixed scratch is refused, all before
    any HIP call."""
    f = lib.rs_verify_noalloc
    ok = dict(logits=DUMMY, dtype=1, q=None, draft=DUMMY, cu=DUMMY, T=DUMMY, B=2, D=4, max_k=2, V=100, seed=0,
              out=DUMMY, nacc=DUMMY)

    def g(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["logits"], a["dtype"], a["q"], a["draft"], a["cu"], a["T"], a["B"], a["D"], a["max_k"], a["V"],
                 a["seed"], a["out"], a["nacc"], None, None)

    assert g(max_k=40) == rs.RS_ERR_INVALID_ARG
    assert g(cu=None) == rs.RS_ERR_INVALID_ARG
    assert g(dtype=7) == rs.RS_ERR_UNSUPPORTED
    assert g(B=0, D=0) == rs.RS_OK
    B, K, V = 1024, 8, 151936
    assert rs.workspace_size(B, B * K, K, V) > rs.NOALLOC_SCRATCH_BYTES >= rs.workspace_size(512, 512 * K, K, V)
    assert g(B=B, D=B * K, max_k=K, V=V) == rs.RS_ERR_WORKSPACE


@needs_no_gpu
def test_greedy_entry_validation(lib):
    f = lib.rs_verify_greedy
    ok = dict(logits=DUMMY, dtype=1, draft=DUMMY, cu=DUMMY, B=2, D=4, max_k=2, V=100, out=DUMMY, nacc=DUMMY, ws=DUMMY,
              ws_bytes=1 << 30)

    def g(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["logits"], a["dtype"], a["draft"], a["cu"], a["B"], a["D"], a["max_k"], a["V"], a["out"],
                 a["nacc"], a["ws"], a["ws_bytes"], None)

    assert g(max_k=40) == rs.RS_ERR_INVALID_ARG
    assert g(cu=None) == rs.RS_ERR_INVALID_ARG
    assert g(ws_bytes=0) == rs.RS_ERR_WORKSPACE
    assert g(B=0, D=0) == rs.RS_OK


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(3, 10)
    with pytest.raises(ValueError):
        rs.verify(x, None, torch.zeros(2, dtype=torch.int32), torch.tensor([0, 2], dtype=torch.int32),
                  torch.ones(1), seed=0, max_k=2)


def _call_filtered(lib, **kw):
    a = dict(logits=DUMMY, dtype=1, q=None, draft=DUMMY, cu=DUMMY, T=DUMMY, top_k=DUMMY, top_p=DUMMY, B=2, D=4,
             max_k=2, V=100, seed=0, out=DUMMY, nacc=DUMMY, ws=DUMMY, ws_bytes=1 << 30, dbg=None, stream=None)
    a.update(kw)
    return lib.rs_verify_filtered(a["logits"], a["dtype"], a["q"], a["draft"], a["cu"], a["T"], a["top_k"],
                                  a["top_p"], a["B"], a["D"], a["max_k"], a["V"], a["seed"], a["out"], a["nacc"],
                                  a["ws"], a["ws_bytes"], a["dbg"], a["stream"])


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(V=1 << 20), rs.RS_ERR_UNSUPPORTED),            # fixed-point top-p masses need V < 2^20
    (dict(V=1 << 20, top_k=None), rs.RS_ERR_UNSUPPORTED),
    (dict(top_k=DUMMY + 2), rs.RS_ERR_UNSUPPORTED),      # int32 alignment
    (dict(top_p=DUMMY + 1), rs.RS_ERR_UNSUPPORTED),
    (dict(max_k=33, D=4), rs.RS_ERR_INVALID_ARG),
    (dict(T=None), rs.RS_ERR_INVALID_ARG),
    (dict(ws_bytes=16), rs.RS_ERR_WORKSPACE),
])
def test_filtered_entry_validation(lib, kw, status):
    assert _call_filtered(lib, **kw) == status


@needs_no_gpu
def test_filtered_entry_empty_batch(lib):
    assert _call_filtered(lib, B=0, D=0, logits=None, out=None, nacc=None, ws=None) == rs.RS_OK


@needs_no_gpu
def test_stats_entry_validation(lib):
    f = lib.rs_accept_stats_accumulate
    assert f(DUMMY, DUMMY, -1, DUMMY, None) == rs.RS_ERR_INVALID_ARG
    assert f(None, DUMMY, 4, DUMMY, None) == rs.RS_ERR_INVALID_ARG
    assert f(DUMMY, None, 4, DUMMY, None) == rs.RS_ERR_INVALID_ARG
    assert f(DUMMY, DUMMY, 4, None, None) == rs.RS_ERR_INVALID_ARG
    assert f(DUMMY, DUMMY, 4, DUMMY + 4, None) == rs.RS_ERR_UNSUPPORTED
    assert f(None, None, 0, None, None) == rs.RS_OK


def test_stats_host_helpers(lib):
    import json
    import numpy as np
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "accept_stats_worked_example.json")))
    c = np.zeros(rs.STATS_COUNTERS, np.int64)
    c[1] = g["verifies"] * g["K"]
    c[2] = g["accepted_total"]
    c[3] = g["completion_tokens"]
    c[4] = g["verifies"]
    p = c.ctypes.data_as(ctypes.c_void_p)
    assert lib.rs_accept_rate(p) == g["accept_rate"]
    assert lib.rs_accept_length(p) == g["accept_length"]
    import math
    assert math.isnan(lib.rs_accept_rate(np.zeros(rs.STATS_COUNTERS, np.int64).ctypes.data_as(ctypes.c_void_p)))
    assert math.isnan(lib.rs_accept_length(None))


def _call_tree(lib, **kw):
    a = dict(logits=DUMMY, dtype=1, tok=DUMMY, par=DUMMY, cu=DUMMY, T=DUMMY, B=2, N=10, max_nodes=8, max_depth=4,
             V=100, seed=0, out=DUMMY, path=DUMMY, nacc=DUMMY, ws=DUMMY, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.rs_verify_tree(a["logits"], a["dtype"], a.get("q"), a["tok"], a["par"], a["cu"], a["T"], a["B"], a["N"],
                              a["max_nodes"], a["max_depth"], a["V"], a["seed"], a["out"], a["path"], a["nacc"],
                              a["ws"], a["wsb"], a["stream"])


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), rs.RS_ERR_INVALID_ARG),
    (dict(max_nodes=65, max_depth=4), rs.RS_ERR_INVALID_ARG),   # RS_MAX_TREE_NODES = 64
    (dict(max_depth=9), rs.RS_ERR_INVALID_ARG),                 # deeper than max_nodes
    (dict(N=17), rs.RS_ERR_INVALID_ARG),                        # N > B * max_nodes
    (dict(V=0), rs.RS_ERR_INVALID_ARG),
    (dict(dtype=3), rs.RS_ERR_UNSUPPORTED),
    (dict(tok=None), rs.RS_ERR_INVALID_ARG),
    (dict(path=None), rs.RS_ERR_INVALID_ARG),
    (dict(T=None), rs.RS_ERR_INVALID_ARG),
    (dict(logits=DUMMY + 1), rs.RS_ERR_UNSUPPORTED),
    (dict(par=DUMMY + 2), rs.RS_ERR_UNSUPPORTED),
    (dict(q=DUMMY + 8), rs.RS_ERR_UNSUPPORTED),                 # draft rows must be 16-byte aligned
    (dict(ws=None), rs.RS_ERR_WORKSPACE),
    (dict(wsb=8), rs.RS_ERR_WORKSPACE),
])
def test_tree_entry_validation(lib, kw, status):
    assert _call_tree(lib, **kw) == status


@needs_no_gpu
def test_tree_entry_empty_batch(lib):
    assert _call_tree(lib, B=0, N=0, logits=None, out=None, nacc=None) == rs.RS_OK


@needs_no_gpu
def test_ngram_entry_validation(lib):
    f = lib.rs_ngram_propose

    def g(**kw):
        a = dict(ctx=DUMMY, cu=DUMMY, B=2, T=100, mn=2, mx=4, k=5, mml=1 << 40, d=DUMMY, n=DUMMY, c=DUMMY, ws=DUMMY,
                 wsb=1 << 20)
        a.update(kw)
        return f(a["ctx"], a["cu"], a["B"], a["T"], a["mn"], a["mx"], a["k"], a["mml"], a["d"], a["n"], a["c"],
                 a["ws"], a["wsb"], None)

    assert g(B=-1) == rs.RS_ERR_INVALID_ARG
    assert g(mn=0) == rs.RS_ERR_INVALID_ARG
    assert g(mx=1) == rs.RS_ERR_INVALID_ARG          # max_n < min_n
    assert g(mx=65) == rs.RS_ERR_INVALID_ARG         # RS_NGRAM_MAX_N = 64
    assert g(k=33) == rs.RS_ERR_INVALID_ARG          # RS_MAX_SPEC_LEN = 32
    assert g(cu=None) == rs.RS_ERR_INVALID_ARG
    assert g(ctx=DUMMY + 2) == rs.RS_ERR_UNSUPPORTED
    assert g(wsb=2 * 5 * 4 - 1) == rs.RS_ERR_WORKSPACE
    assert g(ws=None) == rs.RS_ERR_WORKSPACE
    assert g(B=0, ctx=None, cu=None, d=None, n=None, c=None, ws=None) == rs.RS_OK
