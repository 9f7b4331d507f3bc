"""The C-ABI library loads, exports every function include/sgl_attn.h declares,
and rejects bad arguments before any GPU work (these calls never reach HIP,
so they run without a GPU)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

import prefix_shared_paged_amd as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgl_attn.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(sgl_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for n in ["sgl_kv_pool_alloc", "sgl_build_req_to_token", "sgl_extend_attn", "sgl_decode_attn",
              "sgl_cascade_decode_attn"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = sp.load()
    names = declared_functions()
    assert names, "no declarations found"
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(sp.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", sp.lib_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (sgl_\w+)", out))
    assert set(names) <= exported


def test_header_compiles_as_c():
    src = ('#include "sgl_attn.h"\n#include "sgl_probe.h"\n'
           'int main(void) { return sgl_abi_version() > 0 ? 0 : 1; }\n')
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I",
                          os.path.dirname(HEADER), "-x", "c", "-"], input=src, text=True,
                         capture_output=True)
    assert res.returncode == 0, res.stderr


def test_status_strings():
    assert sp.status_string(0) == "SGL_OK"
    assert sp.status_string(3) == "SGL_ERR_OOM"
    assert sp.status_string(99) == "SGL_ERR_UNKNOWN"


def _fake(n=1):
    # host buffers used only as non-null pointers: every call below fails its
    # argument checks before any pointer is dereferenced or any kernel enqueued
    return ctypes.cast(ctypes.create_string_buffer(64 * n), ctypes.c_void_p)


def test_device_calls_reject_bad_arguments_before_gpu_work():
    lib = sp.load()
    p = _fake()
    # unsupported head_dim
    assert lib.sgl_extend_attn(sp.SGL_BF16, p, None, None, p, p, 16, p, 1, 8, p, p, p, 1, 4, 4,
                               8, 8, 96, 0.1, p, None, None, 0, None) == sp.SGL_ERR_UNSUPPORTED
    # Hq not a multiple of Hkv
    assert lib.sgl_decode_attn(sp.SGL_BF16, p, None, None, p, p, 16, p, 1, 8, p, p, 1, 8, 12, 8,
                               128, 0.1, p, None, p, 1 << 20, None) == sp.SGL_ERR_UNSUPPORTED
    # unsupported dtype
    assert lib.sgl_decode_attn(7, p, None, None, p, p, 16, p, 1, 8, p, p, 1, 8, 8, 8, 128, 0.1, p,
                               None, p, 1 << 20, None) == sp.SGL_ERR_UNSUPPORTED
    # missing q
    assert lib.sgl_extend_attn(sp.SGL_BF16, None, None, None, p, p, 16, p, 1, 8, p, p, p, 1, 4, 4,
                               8, 8, 128, 0.1, p, None, None, 0, None) == sp.SGL_ERR_INVALID
    # k_new without v_new
    assert lib.sgl_extend_attn(sp.SGL_BF16, p, p, None, p, p, 16, p, 1, 8, p, p, p, 1, 4, 4, 8, 8,
                               128, 0.1, p, None, None, 0, None) == sp.SGL_ERR_INVALID
    # workspace too small
    need = lib.sgl_decode_workspace_size(4, 1000, 32, 8, 128)
    assert need > 0
    assert lib.sgl_decode_attn(sp.SGL_BF16, p, None, None, p, p, 16, p, 4, 1000, p, p, 4, 1000, 32,
                               8, 128, 0.1, p, None, p, need - 1, None) == sp.SGL_ERR_WORKSPACE
    # cascade: group larger than supported (1024 requests x 8 heads > 4096 rows)
    assert lib.sgl_cascade_decode_attn(sp.SGL_BF16, p, None, None, p, p, 16, p, 16, 100, p, p, p, p,
                                       1024, 1, 100, 1024, 50, 64, 8, 128, 0.1, p, None, p, 1 << 24,
                                       None) == sp.SGL_ERR_UNSUPPORTED
    # cascade: prefix bound larger than the context bound
    assert lib.sgl_cascade_decode_attn(sp.SGL_BF16, p, None, None, p, p, 16, p, 4, 100, p, p, p, p, 4,
                                       1, 100, 4, 101, 32, 8, 128, 0.1, p, None, p, 1 << 24,
                                       None) == sp.SGL_ERR_INVALID
    # r2t build: prefix slots without offsets
    assert lib.sgl_build_req_to_token(p, 4, 8, p, 1, p, None, p, p, None, None) == sp.SGL_ERR_INVALID
    # device index check: missing counter, negative bounds; empty batch is a no-op
    assert lib.sgl_count_bad_slots(p, 4, 8, p, p, 1, 8, 16, None, None) == sp.SGL_ERR_INVALID
    assert lib.sgl_count_bad_slots(p, 4, 8, p, p, 1, -1, 16, p, None) == sp.SGL_ERR_INVALID
    assert lib.sgl_count_bad_slots(p, 4, 8, p, p, 0, 8, 16, p, None) == sp.SGL_OK
    # empty batches are a no-op
    assert lib.sgl_decode_attn(sp.SGL_BF16, p, None, None, p, p, 16, p, 1, 8, p, p, 0, 8, 32, 8, 128,
                               0.1, p, None, None, 0, None) == sp.SGL_OK
    # FP8 KV: fp32 queries are not supported
    assert lib.sgl_decode_attn_fp8kv(sp.SGL_F32, p, None, None, p, p, p, p, 16, p, 1, 8, p, p, 1, 8, 32,
                                     8, 128, 0.1, p, None, p, 1 << 20, None) == sp.SGL_ERR_UNSUPPORTED
    # FP8 KV: missing per-head factors
    assert lib.sgl_decode_attn_fp8kv(sp.SGL_BF16, p, None, None, p, p, None, p, 16, p, 1, 8, p, p, 1, 8,
                                     32, 8, 128, 0.1, p, None, p, 1 << 20, None) == sp.SGL_ERR_INVALID
    assert lib.sgl_cascade_decode_attn_fp8kv(sp.SGL_BF16, p, None, None, p, p, p, None, 16, p, 4, 100, p,
                                             p, p, p, 4, 1, 100, 4, 50, 32, 8, 128, 0.1, p, None, p,
                                             1 << 24, None) == sp.SGL_ERR_INVALID
    assert lib.sgl_store_kv_fp8(sp.SGL_BF16, p, p, 4, p, p, p, 16, 8, 128, None, p,
                                None) == sp.SGL_ERR_INVALID
    # FP8 KV: unsupported head_dim
    assert lib.sgl_store_kv_fp8(sp.SGL_BF16, p, p, 4, p, p, p, 16, 8, 96, p, p,
                                None) == sp.SGL_ERR_UNSUPPORTED
    # FP8 KV: empty store is a no-op
    assert lib.sgl_store_kv_fp8(sp.SGL_F32, p, p, 0, p, p, p, 16, 8, 128, p, p, None) == sp.SGL_OK
    # host tier: row bytes not a positive multiple of 16, negative count, K/V pairing, alignment, nulls
    pf, wb = lib.sgl_hicache_prefetch, lib.sgl_hicache_write_back
    q = _fake(4)
    mis = ctypes.c_void_p(q.value + 8)
    assert pf(q, q, 8, q, q, 4, q, q, 8, 15, None) == sp.SGL_ERR_INVALID
    assert pf(q, q, 8, q, q, 4, q, q, 8, 0, None) == sp.SGL_ERR_INVALID
    assert pf(q, q, 8, q, q, -1, q, q, 8, 16, None) == sp.SGL_ERR_INVALID
    assert pf(q, q, 8, q, q, 4, q, None, 8, 16, None) == sp.SGL_ERR_INVALID
    assert pf(mis, None, 8, q, q, 4, q, None, 8, 16, None) == sp.SGL_ERR_INVALID
    assert pf(q, None, 8, None, q, 4, q, None, 8, 16, None) == sp.SGL_ERR_INVALID
    assert wb(q, q, 8, q, q, 4, q, q, 0, 16, None) == sp.SGL_ERR_INVALID
    assert wb(q, None, 8, q, q, 4, q, q, 8, 16, None) == sp.SGL_ERR_INVALID
    assert wb(q, q, 8, q, q, 0, q, q, 8, 16, None) == sp.SGL_OK
    assert pf(None, None, 8, None, None, 0, None, None, 8, 16, None) == sp.SGL_OK
    # measurement helpers: bad sizes, counts and pointers
    assert lib.sgl_probe_copy(q, _fake(4), 24, None) == sp.SGL_ERR_INVALID
    assert lib.sgl_probe_copy(q, _fake(4), -16, None) == sp.SGL_ERR_INVALID
    assert lib.sgl_probe_copy(mis, _fake(4), 16, None) == sp.SGL_ERR_INVALID
    assert lib.sgl_probe_copy(q, None, 16, None) == sp.SGL_ERR_INVALID
    assert lib.sgl_probe_copy(q, ctypes.c_void_p(q.value + 16), 64, None) == sp.SGL_ERR_INVALID
    assert lib.sgl_probe_copy(None, None, 0, None) == sp.SGL_OK
    assert lib.sgl_probe_mfma_bf16(0, 1, 1.0, q, None) == sp.SGL_ERR_INVALID
    assert lib.sgl_probe_mfma_bf16(1, 0, 1.0, q, None) == sp.SGL_ERR_INVALID
    assert lib.sgl_probe_mfma_bf16(1, 1, 1.0, None, None) == sp.SGL_ERR_INVALID


def test_workspace_sizes_grow_with_the_problem():
    lib = sp.load()
    a = lib.sgl_decode_workspace_size(256, 8192, 32, 8, 128)
    b = lib.sgl_decode_workspace_size(256, 4096, 32, 8, 128)
    assert a > b > 0
    c = lib.sgl_cascade_workspace_size(256, 16, 8192, 16, 4096, 32, 8, 128)
    assert c > a
    # the extend workload's grid (4096 workgroups) needs no key splits
    assert lib.sgl_extend_workspace_size(64, 16384, 256, 2304, 32, 8, 128) == 0
    # a few new tokens per request (split-K path), and one long chunked-prefill
    # request whose 256-workgroup grid gets key splits
    assert lib.sgl_extend_workspace_size(64, 256, 4, 8300, 32, 8, 128) > 0
    assert lib.sgl_extend_workspace_size(1, 512, 512, 33000, 64, 8, 128) > 0
    assert lib.sgl_extend_workspace_size(1, 512, 512, 4096, 64, 8, 128) == 0


def test_bytes_per_token_accounting():
    # 'SGLang 深度拆解' (chenxutan.com) section 4.3: K and V of one token of
    # Llama3.1-70B in bf16 take 2 x 80 layers x 8 KV heads x 128 dims x 2 bytes
    # = 327,680 bytes, and a 4096-token prompt about 1.25 GB.
    from prefix_shared_paged_amd.accounting import kv_bytes_per_token
    assert kv_bytes_per_token(Hkv=8, D=128, elt=2, layers=80) == 327680
    assert abs(4096 * kv_bytes_per_token(8, 128, 2, 80) / 2 ** 30 - 1.25) < 1e-9


def test_set_validate_modes():
    """The validation switch is host state only: it returns the previous mode
    and rejects modes outside {-1, 0, 1} without changing anything."""
    import prefix_shared_paged_amd as sp
    lib = sp.load()
    prev = lib.sgl_set_validate(1)
    try:
        assert lib.sgl_set_validate(0) == 1
        assert lib.sgl_set_validate(5) == -2
        assert lib.sgl_set_validate(-1) == 0
    finally:
        lib.sgl_set_validate(prev)
