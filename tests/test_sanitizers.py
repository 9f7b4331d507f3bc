"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The host bookkeeping (host_cache.cpp: slot pool and compressed radix tree)
and the C oracle (attn_oracle.c) are compiled by g++ / gcc with
-fsanitize=address,undefined (host code only: no GPU code is involved), and
a child Python process with the ASan runtime preloaded runs the existing CPU
tests against those builds: the random-operation comparison of the
bookkeeping with the brute-force model, the batched calls, the allocator
cases, and the oracle's pins that need no other library (hand cases, the two
evaluation orders, probability rows, the state merge, prefix reuse, argument
checks).  Any sanitizer report aborts the child and fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "tests", "_build")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime():
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        return None
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime() is None, reason="gcc with the ASan runtime is not available")
def test_host_code_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    host = os.path.join(OUT, "libsgl_host_san.so")
    orc = os.path.join(OUT, "liboracle_san.so")
    subprocess.run(["g++", "-std=c++17", "-shared", "-fPIC", *SAN, "-I" + os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "prefix_shared_paged_amd", "csrc", "host_cache.cpp"), "-o", host],
                   check=True)
    subprocess.run(["gcc", "-std=c11", "-shared", "-fPIC", *SAN, os.path.join(ROOT, "oracle", "attn_oracle.c"),
                    "-o", orc, "-lpthread", "-lm"], check=True)
    env = dict(os.environ)
    pre = [_runtime()] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else [])
    env.update(LD_PRELOAD=":".join(pre), SGL_ATTN_LIBRARY=host, ORACLE_LIBRARY=orc,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_host_cache.py"),
           os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", "not sdpa"]
    res = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = "\n".join((res.stdout + res.stderr).splitlines()[-40:])
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail
    assert " passed" in res.stdout, tail
