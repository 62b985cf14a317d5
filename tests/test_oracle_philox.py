"""Pins of the oracle's random stream (Philox4x32-10 and the u / E mappings).

The pages name no generator; the stream is Philox4x32-10 from its published
definition, so the oracle's implementation is pinned against (a) the
published known-answer vectors, (b) an independent library implementation
(rocRAND's host engine, compiled here from its header), and (c) the
distributions the verify rule needs: u ~ U[0, 1) on a 24-bit grid and
E = -ln U ~ Exp(1).
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(t, 16) for t in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_known_answer_vectors():
    for ctr, key, expect in _kat():
        got = oracle.philox([ctr], [key])[0]
        assert [int(v) for v in got] == expect


def _rocrand_binary(tmp):
    cxx = shutil.which("amdclang++") or "/opt/rocm/bin/amdclang++"
    if not os.path.exists(cxx) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND header or amdclang++ not available")
    exe = os.path.join(tmp, "rr")
    subprocess.run([cxx, "-x", "c++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(HERE, "rocrand_philox_check.cpp"), "-o", exe], check=True)
    return exe


def test_matches_rocrand_host_engine():
    rng = np.random.default_rng(12345)
    n = 2000
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64)
    ctr[:, 1] %= 2**30  # the rocRAND helper encodes c1 through a 64-bit offset
    key = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64)
    # the counter layouts the verify step uses: (0, j, b, 0) and (x >> 2, j, b, 1)
    ctr[:100, 0] = 0
    ctr[:100, 3] = 0
    ctr[100:200, 3] = 1
    ctr[:200, 1] %= 33
    with tempfile.TemporaryDirectory() as tmp:
        exe = _rocrand_binary(tmp)
        inp = "\n".join(" ".join(f"{int(v):x}" for v in list(c) + list(k)) for c, k in zip(ctr, key))
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    ref = np.array([[int(t, 16) for t in line.split()] for line in out.strip().splitlines()], np.uint64)
    got = oracle.philox(ctr.astype(np.uint32), key.astype(np.uint32)).astype(np.uint64)
    assert ref.shape == (n, 4)
    np.testing.assert_array_equal(got, ref)


def test_accept_uniform_grid_and_distribution():
    b = np.repeat(np.arange(20000, dtype=np.int32), 10)
    j = np.tile(np.arange(10, dtype=np.int32), 20000)
    u = oracle.accept_uniforms(77, b, j)
    # exactly representable on the 2^-24 grid in [0, 1)
    k = u * 2**24
    assert np.all(k == np.floor(k)) and np.all(u >= 0) and np.all(u < 1)
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    # word 0 of Philox((0, j, b, 0), seed) >> 8
    w = oracle.philox([[0, 3, 5, 0]], [[77, 0]])[0]
    assert oracle.accept_uniforms(77, [5], [3])[0] == (int(w[0]) >> 8) / 2**24


def test_race_exponential_grid_and_distribution():
    e = oracle.race_exponentials(2024, 7, 3, 0, 200000)
    assert np.all(np.isfinite(e)) and np.all(e > 0)
    assert stats.kstest(e, "expon").pvalue > 1e-3
    assert abs(e.mean() - 1.0) < 5 * 1.0 / np.sqrt(e.size)
    # U = ((w >> 9) + 1/2) 2^-23 with w = word (x & 3) of Philox((x >> 2, j, b, 1), seed)
    for x in (0, 1, 2, 3, 4, 151935):
        w = oracle.philox([[x >> 2, 3, 7, 1]], [[2024, 0]])[0]
        U = ((int(w[x & 3]) >> 9) + 0.5) / 2**23
        assert oracle.race_uniform(2024, 7, 3, x) == U
        assert e[x] == pytest.approx(-np.log(U), rel=1e-15) if x < e.size else True


def test_streams_differ_by_request_position_and_tag():
    u1 = oracle.accept_uniforms(1, [0, 0, 1], [0, 1, 0])
    assert len(set(u1.tolist())) == 3
    # seed high word feeds the key
    a = oracle.accept_uniforms(1, [0], [0])[0]
    b = oracle.accept_uniforms(1 + (1 << 32), [0], [0])[0]
    assert a != b
