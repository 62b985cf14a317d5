"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle (plain C) with gcc's -fsanitize=address,undefined, driven
  through every entry on small seeded inputs (tests/sanitize/oracle_driver.c).
- The library's host side (argument validation, launch planning, workspace
  sizes, counter helpers, status strings) built with hipcc, the sanitizers on
  the host pass only, driven through every entry point with pointers that are
  never dereferenced (tests/sanitize/abi_driver.cpp).  None of its calls
  reaches a HIP call, so it needs no GPU.

Builds are cached under the system temporary directory by a hash of their
sources, so only the first run after a change pays the compile (~1 minute for
the library, whose device pass is built at -O0 here)."""
import hashlib
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
REPORTS = ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:", "UndefinedBehaviorSanitizer")


def _hash(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _build(name, sources, deps, cmd_of):
    out_dir = os.path.join(tempfile.gettempdir(), "rs_verify_host_sanitizers")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, f"{name}_{_hash(sources + deps)}")
    if not os.path.exists(exe):
        tmp = exe + f".tmp{os.getpid()}"
        r = subprocess.run(cmd_of(tmp), capture_output=True, text=True)
        if r.returncode != 0:
            raise AssertionError(f"sanitizer build of {name} failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, exe)
    return exe


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=SAN_ENV, timeout=600)
    text = r.stdout + r.stderr
    assert r.returncode == 0 and not any(s in text for s in REPORTS), text
    return text


def test_oracle_under_asan_ubsan():
    src = [os.path.join(ROOT, "oracle", "rs_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")]
    exe = _build("oracle_driver", src, [], lambda out: [
        "gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
        "-fno-sanitize-recover=all", *src, "-o", out, "-lm"])
    assert "ok" in _run(exe)


@pytest.mark.slow
def test_library_host_side_under_asan_ubsan():
    csrc = os.path.join(ROOT, "rejection_sampling_verify_rs_amd", "csrc")
    deps = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)) + [os.path.join(ROOT, "include", "rs_verify.h")]
    src = [os.path.join(csrc, "rs_verify.hip"), os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")]
    hipcc = next((c for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc") if c and os.path.exists(c)), "hipcc")
    exe = _build("abi_driver", src, deps, lambda out: [
        hipcc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-Xarch_device", "-O0",
        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=all",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), *src, "-o", out])
    assert "ok" in _run(exe)
