"""Paged prefix-shared attention for MI355X (gfx950): Python binding.

Thin ctypes marshalling over the C ABI of libsgl_attn.so (declared in
include/sgl_attn.h); every step of the attention path runs in the library's
HIP kernels.  PyTorch only provides device memory and the current stream.
The names follow the C functions without the ``sgl_`` prefix.

If the library is missing it is built (hipcc) on first use; if that fails the
import of the entry points raises -- there is no fallback implementation.
"""
import ctypes
import os

import numpy as np

from . import build as _build

SGL_OK, SGL_ERR_INVALID, SGL_ERR_UNSUPPORTED, SGL_ERR_OOM, SGL_ERR_HIP, SGL_ERR_WORKSPACE = range(6)
SGL_F32, SGL_BF16 = 0, 1

_lib = None


class SglError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


class OutOfSlots(SglError):
    pass


def lib_path() -> str:
    return _build.LIB


def load():
    """Load libsgl_attn.so (building it first if it does not exist).

    SGL_ATTN_LIBRARY=<path> loads another build of the same sources instead;
    the sanitizer check of the host bookkeeping uses it for a host-only build
    (only the symbols that build exports are bound: the device entry points
    are absent from it and raise AttributeError when called)."""
    global _lib
    if _lib is not None:
        return _lib
    alt = os.environ.get("SGL_ATTN_LIBRARY")
    if alt:
        lib = ctypes.CDLL(alt)
    else:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "sgl_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "sgl_abi_version": (ctypes.c_int, []),
        "sgl_set_validate": (ctypes.c_int, [ctypes.c_int]),
        "sgl_kv_pool_create": (ctypes.c_int, [I64, I32, P, P]),
        "sgl_kv_pool_destroy": (ctypes.c_int, [P]),
        "sgl_kv_pool_alloc": (ctypes.c_int, [P, I64, I32, I64, P]),
        "sgl_kv_pool_free": (ctypes.c_int, [P, P, I64]),
        "sgl_kv_pool_available": (I64, [P]),
        "sgl_radix_create": (ctypes.c_int, [I32, P]),
        "sgl_radix_destroy": (ctypes.c_int, [P]),
        "sgl_radix_match": (ctypes.c_int, [P, P, I64, P, P, P]),
        "sgl_radix_insert": (ctypes.c_int, [P, P, P, I64, P, P]),
        "sgl_radix_lock": (ctypes.c_int, [P, ctypes.c_uint64, I32]),
        "sgl_radix_evict": (ctypes.c_int, [P, I64, P, P]),
        "sgl_radix_stats": (ctypes.c_int, [P, P, P]),
        "sgl_radix_match_batch": (ctypes.c_int, [P, P, P, I32, I32, P, P, P]),
        "sgl_radix_insert_batch": (ctypes.c_int, [P, P, P, P, I32, P, P]),
        "sgl_radix_lock_batch": (ctypes.c_int, [P, P, I32, I32]),
        "sgl_kv_pool_alloc_batch": (ctypes.c_int, [P, P, P, P, I32, P]),
        "sgl_build_req_to_token": (ctypes.c_int, [P, I64, I64, P, I32, P, P, P, P, P, P]),
        "sgl_count_bad_slots": (ctypes.c_int, [P, I64, I64, P, P, I32, I32, I64, P, P]),
        "sgl_store_kv": (ctypes.c_int, [ctypes.c_int, P, P, I64, P, P, P, I64, I32, I32, P]),
        "sgl_extend_attn": (ctypes.c_int, [ctypes.c_int, P, P, P, P, P, I64, P, I64, I64, P, P, P,
                                           I32, I64, I32, I32, I32, I32, F, P, P, P, SZ, P]),
        "sgl_extend_workspace_size": (SZ, [I32, I64, I32, I64, I32, I32, I32]),
        "sgl_decode_attn": (ctypes.c_int, [ctypes.c_int, P, P, P, P, P, I64, P, I64, I64, P, P,
                                           I32, I32, I32, I32, I32, F, P, P, P, SZ, P]),
        "sgl_decode_workspace_size": (SZ, [I32, I32, I32, I32, I32]),
        "sgl_cascade_decode_attn": (ctypes.c_int, [ctypes.c_int, P, P, P, P, P, I64, P, I64, I64, P,
                                                   P, P, P, I32, I32, I32, I32, I32, I32, I32, I32,
                                                   F, P, P, P, SZ, P]),
        "sgl_cascade_workspace_size": (SZ, [I32, I32, I32, I32, I32, I32, I32, I32]),
        "sgl_cascade_decode_attn_static": (ctypes.c_int, [ctypes.c_int, P, P, P, P, P, I64, P, I64, I64, P,
                                                          P, P, P, I32, I32, I32, I32, I32, I32, I32, I32,
                                                          F, P, P, P]),
        "sgl_static_scratch_bytes": (SZ, []),
        "sgl_store_kv_fp8": (ctypes.c_int, [ctypes.c_int, P, P, I64, P, P, P, I64, I32, I32, P, P, P]),
        "sgl_decode_attn_fp8kv": (ctypes.c_int, [ctypes.c_int, P, P, P, P, P, P, P, I64, P, I64, I64,
                                                 P, P, I32, I32, I32, I32, I32, F, P, P, P, SZ, P]),
        "sgl_cascade_decode_attn_fp8kv": (ctypes.c_int, [ctypes.c_int, P, P, P, P, P, P, P, I64, P,
                                                         I64, I64, P, P, P, P, I32, I32, I32, I32,
                                                         I32, I32, I32, I32, F, P, P, P, SZ, P]),
        "sgl_mla_decode_attn": (ctypes.c_int, [P, P, P, I64, P, I64, I64, P, P, I32, I32, I32, I32, I32, F,
                                               P, P, P, SZ, P]),
        "sgl_mla_decode_workspace_size": (SZ, [I32, I32, I32, I32]),
        "sgl_mla_cascade_decode_attn": (ctypes.c_int, [P, P, P, I64, P, I64, I64, P, P, P, P, I32, I32, I32,
                                                       I32, I32, I32, I32, I32, F, P, P, P, SZ, P]),
        "sgl_mla_cascade_workspace_size": (SZ, [I32, I32, I32, I32, I32, I32, I32]),
        "sgl_hicache_prefetch": (ctypes.c_int, [P, P, I64, P, P, I64, P, P, I64, I64, P]),
        "sgl_hicache_write_back": (ctypes.c_int, [P, P, I64, P, P, I64, P, P, I64, I64, P]),
        "sgl_probe_mfma_bf16": (ctypes.c_int, [I32, I32, F, P, P]),
        "sgl_probe_copy": (ctypes.c_int, [P, P, I64, P]),
    }
    for name, (res, args) in sig.items():
        if alt and not hasattr(lib, name):
            continue
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


EXPORTS = ["sgl_status_string", "sgl_abi_version", "sgl_set_validate", "sgl_kv_pool_create", "sgl_kv_pool_destroy",
           "sgl_kv_pool_alloc", "sgl_kv_pool_free", "sgl_kv_pool_available", "sgl_radix_create",
           "sgl_radix_destroy", "sgl_radix_match", "sgl_radix_insert", "sgl_radix_lock",
           "sgl_radix_evict", "sgl_radix_stats", "sgl_radix_match_batch", "sgl_radix_insert_batch",
           "sgl_radix_lock_batch", "sgl_kv_pool_alloc_batch", "sgl_build_req_to_token", "sgl_count_bad_slots",
           "sgl_store_kv",
           "sgl_extend_attn", "sgl_extend_workspace_size", "sgl_decode_attn",
           "sgl_decode_workspace_size", "sgl_cascade_decode_attn", "sgl_cascade_workspace_size",
           "sgl_cascade_decode_attn_static", "sgl_static_scratch_bytes",
           "sgl_store_kv_fp8", "sgl_decode_attn_fp8kv", "sgl_cascade_decode_attn_fp8kv",
           "sgl_mla_decode_attn", "sgl_mla_decode_workspace_size", "sgl_mla_cascade_decode_attn",
           "sgl_mla_cascade_workspace_size", "sgl_hicache_prefetch", "sgl_hicache_write_back",
           "sgl_probe_mfma_bf16", "sgl_probe_copy"]


def status_string(status: int) -> str:
    return load().sgl_status_string(status).decode()


def set_validate(mode: int) -> int:
    """Index validation of the device calls: 1 on, 0 off, -1 follow
    SGL_ATTN_VALIDATE.  Returns the previous mode."""
    prev = load().sgl_set_validate(int(mode))
    if prev == -2:
        raise ValueError(f"validation mode must be -1, 0 or 1, not {mode}")
    return prev


def _check(fn, status):
    if status == SGL_ERR_OOM:
        raise OutOfSlots(fn, status)
    if status != SGL_OK:
        raise SglError(fn, status)


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


# ---------------------------------------------------------------------------
# host objects
# ---------------------------------------------------------------------------
class KVPool:
    """Slot pool: FIFO free list of pages (sgl_kv_pool_*)."""

    def __init__(self, num_slots, page_size=1, init_order=None):
        lib = load()
        self._h = ctypes.c_void_p()
        order = None if init_order is None else _i32(init_order)
        _check("sgl_kv_pool_create", lib.sgl_kv_pool_create(
            num_slots, page_size, _np_ptr(order) if order is not None else None, ctypes.byref(self._h)))
        self.num_slots = num_slots
        self.page_size = page_size

    @property
    def handle(self):
        return self._h

    def alloc(self, n, cur_len=0, last_slot=-1):
        out = np.empty(int(n), np.int32)
        _check("sgl_kv_pool_alloc", load().sgl_kv_pool_alloc(self._h, cur_len, last_slot, n, _np_ptr(out)))
        return out

    def alloc_batch(self, n, cur_len, last_slot):
        """Batched alloc (all or nothing); returns (flat slots, offsets)."""
        n = np.ascontiguousarray(n, np.int64)
        cur = np.ascontiguousarray(cur_len, np.int64)
        last = _i32(last_slot)
        off = np.zeros(n.size + 1, np.int64)
        np.cumsum(n, out=off[1:])
        out = np.empty(max(int(off[-1]), 1), np.int32)
        _check("sgl_kv_pool_alloc_batch", load().sgl_kv_pool_alloc_batch(
            self._h, _np_ptr(cur), _np_ptr(last), _np_ptr(n), n.size, _np_ptr(out)))
        return out[:off[-1]], off

    def free(self, slots):
        s = _i32(slots)
        _check("sgl_kv_pool_free", load().sgl_kv_pool_free(self._h, _np_ptr(s), s.size))

    def available(self):
        return int(load().sgl_kv_pool_available(self._h))

    def close(self):
        if self._h:
            load().sgl_kv_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class RadixTree:
    """Prefix cache: compressed radix tree with ref counts and LRU (sgl_radix_*)."""

    def __init__(self, page_size=1):
        self._h = ctypes.c_void_p()
        _check("sgl_radix_create", load().sgl_radix_create(page_size, ctypes.byref(self._h)))
        self.page_size = page_size

    def match(self, tokens):
        """Return (matched_len, slots[:matched_len], node_handle)."""
        t = _i32(tokens)
        out = np.empty(max(t.size, 1), np.int32)
        n = ctypes.c_int64()
        node = ctypes.c_uint64()
        _check("sgl_radix_match", load().sgl_radix_match(self._h, _np_ptr(t), t.size, _np_ptr(out),
                                                         ctypes.byref(n), ctypes.byref(node)))
        return int(n.value), out[:n.value].copy(), int(node.value)

    def insert(self, tokens, slots, pool=None):
        t, s = _i32(tokens), _i32(slots)
        if t.size != s.size:
            raise ValueError("tokens and slots differ in length")
        cached = ctypes.c_int64()
        _check("sgl_radix_insert", load().sgl_radix_insert(
            self._h, _np_ptr(t), _np_ptr(s), t.size, pool.handle if pool is not None else None,
            ctypes.byref(cached)))
        return int(cached.value)

    def lock(self, node, delta):
        _check("sgl_radix_lock", load().sgl_radix_lock(self._h, node, delta))

    def match_batch(self, tokens, off, lock=False):
        """Batched match over CSR tokens; returns (slots CSR on the same off, lens, nodes)."""
        t = _i32(tokens)
        off = np.ascontiguousarray(off, np.int64)
        B = off.size - 1
        slots = np.empty(max(t.size, 1), np.int32)
        lens = np.empty(B, np.int64)
        nodes = np.empty(B, np.uint64)
        _check("sgl_radix_match_batch", load().sgl_radix_match_batch(
            self._h, _np_ptr(t), _np_ptr(off), B, int(bool(lock)), _np_ptr(slots), _np_ptr(lens),
            _np_ptr(nodes)))
        return slots, lens, nodes

    def insert_batch(self, tokens, slots, off, pool=None):
        t, s = _i32(tokens), _i32(slots)
        off = np.ascontiguousarray(off, np.int64)
        B = off.size - 1
        cached = np.empty(B, np.int64)
        _check("sgl_radix_insert_batch", load().sgl_radix_insert_batch(
            self._h, _np_ptr(t), _np_ptr(s), _np_ptr(off), B, pool.handle if pool is not None else None,
            _np_ptr(cached)))
        return cached

    def lock_batch(self, nodes, delta):
        nd = np.ascontiguousarray(nodes, np.uint64)
        _check("sgl_radix_lock_batch", load().sgl_radix_lock_batch(self._h, _np_ptr(nd), nd.size, delta))

    def evict(self, n_tokens, pool):
        freed = ctypes.c_int64()
        _check("sgl_radix_evict", load().sgl_radix_evict(self._h, n_tokens, pool.handle, ctypes.byref(freed)))
        return int(freed.value)

    def stats(self):
        c, e = ctypes.c_int64(), ctypes.c_int64()
        _check("sgl_radix_stats", load().sgl_radix_stats(self._h, ctypes.byref(c), ctypes.byref(e)))
        return int(c.value), int(e.value)

    def close(self):
        if self._h:
            load().sgl_radix_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# device operations (torch tensors on the GPU)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dev_ptr(t, name, dtype=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return SGL_F32
    if t.dtype == torch.bfloat16:
        return SGL_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def build_req_to_token(r2t, req_rows, new_slots, new_off, prefix_slots=None, prefix_off=None,
                       new_col0=None, stream=None):
    torch = _torch()
    _check("sgl_build_req_to_token", load().sgl_build_req_to_token(
        _dev_ptr(r2t, "r2t", torch.int32), r2t.shape[0], r2t.shape[1],
        _dev_ptr(req_rows, "req_rows", torch.int32), req_rows.numel(),
        _dev_ptr(prefix_slots, "prefix_slots", torch.int32, True),
        _dev_ptr(prefix_off, "prefix_off", torch.int64, True),
        _dev_ptr(new_slots, "new_slots", torch.int32), _dev_ptr(new_off, "new_off", torch.int64),
        _dev_ptr(new_col0, "new_col0", torch.int32, True), _stream(stream)))


def count_bad_slots(r2t, req_rows, seq_lens, max_seq_len, num_slots, count, stream=None):
    """Adds to count (a device uint32 tensor of one element, zeroed by the
    caller) the out-of-range slot ids of the requests' rows, stream-ordered."""
    torch = _torch()
    if count.numel() != 1:
        raise ValueError("count: one int32 element (read as uint32)")
    _check("sgl_count_bad_slots", load().sgl_count_bad_slots(
        _dev_ptr(r2t, "r2t", torch.int32), r2t.shape[0], r2t.shape[1], _dev_ptr(req_rows, "req_rows", torch.int32),
        _dev_ptr(seq_lens, "seq_lens", torch.int32), req_rows.numel(), int(max_seq_len), int(num_slots),
        _dev_ptr(count, "count", torch.int32), _stream(stream)))


def store_kv(k_new, v_new, slots, k_pool, v_pool, stream=None):
    torch = _torch()
    n, Hkv, D = k_new.shape
    _check("sgl_store_kv", load().sgl_store_kv(
        _dtype_code(k_new), _dev_ptr(k_new, "k_new", k_new.dtype), _dev_ptr(v_new, "v_new", k_new.dtype), n,
        _dev_ptr(slots, "slots", torch.int32), _dev_ptr(k_pool, "k_pool", k_new.dtype),
        _dev_ptr(v_pool, "v_pool", k_new.dtype), k_pool.shape[0], Hkv, D, _stream(stream)))


def extend_workspace_size(batch, n_tokens, max_extend_len, row_stride, Hq, Hkv, D):
    return int(load().sgl_extend_workspace_size(batch, n_tokens, max_extend_len, row_stride, Hq, Hkv, D))


def extend_attn(q, k_pool, v_pool, r2t, req_rows, prefix_lens, q_off, max_extend_len, k_new=None,
                v_new=None, scale=None, o=None, lse=None, workspace=None, stream=None):
    """Extend attention; q [n_tokens, Hq, D], pools [S, Hkv, D]; returns o."""
    torch = _torch()
    n_tokens, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if o is None:
        o = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    ws_n = extend_workspace_size(req_rows.numel(), n_tokens, max_extend_len, r2t.shape[1], Hq, Hkv, D)
    if ws_n and workspace is None:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=q.device)
    _check("sgl_extend_attn", load().sgl_extend_attn(
        _dtype_code(q), _dev_ptr(q, "q", q.dtype), _dev_ptr(k_new, "k_new", q.dtype, True),
        _dev_ptr(v_new, "v_new", q.dtype, True), _dev_ptr(k_pool, "k_pool", q.dtype),
        _dev_ptr(v_pool, "v_pool", q.dtype), k_pool.shape[0], _dev_ptr(r2t, "r2t", torch.int32),
        r2t.shape[0], r2t.shape[1], _dev_ptr(req_rows, "req_rows", torch.int32),
        _dev_ptr(prefix_lens, "prefix_lens", torch.int32), _dev_ptr(q_off, "q_off", torch.int64),
        req_rows.numel(), n_tokens, max_extend_len, Hq, Hkv, D, scale, _dev_ptr(o, "o", q.dtype),
        _dev_ptr(lse, "lse", torch.float32, True), _dev_ptr(workspace, "workspace", None, True),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream)))
    return o


def decode_workspace_size(batch, max_seq_len, Hq, Hkv, D):
    return int(load().sgl_decode_workspace_size(batch, max_seq_len, Hq, Hkv, D))


def cascade_workspace_size(batch, G, max_seq_len, max_group_size, max_prefix_len, Hq, Hkv, D):
    return int(load().sgl_cascade_workspace_size(batch, G, max_seq_len, max_group_size, max_prefix_len,
                                                 Hq, Hkv, D))


def decode_attn(q, k_pool, v_pool, r2t, req_rows, seq_lens, max_seq_len, k_new=None, v_new=None,
                scale=None, o=None, lse=None, workspace=None, stream=None):
    """Decode attention; q [batch, Hq, D]; seq_lens include the current token; returns o."""
    torch = _torch()
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if o is None:
        o = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    ws_n = decode_workspace_size(B, max_seq_len, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    _check("sgl_decode_attn", load().sgl_decode_attn(
        _dtype_code(q), _dev_ptr(q, "q", q.dtype), _dev_ptr(k_new, "k_new", q.dtype, True),
        _dev_ptr(v_new, "v_new", q.dtype, True), _dev_ptr(k_pool, "k_pool", q.dtype),
        _dev_ptr(v_pool, "v_pool", q.dtype), k_pool.shape[0], _dev_ptr(r2t, "r2t", torch.int32),
        r2t.shape[0], r2t.shape[1], _dev_ptr(req_rows, "req_rows", torch.int32),
        _dev_ptr(seq_lens, "seq_lens", torch.int32), B, max_seq_len, Hq, Hkv, D, scale,
        _dev_ptr(o, "o", q.dtype), _dev_ptr(lse, "lse", torch.float32, True),
        _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))
    return o


def cascade_decode_attn(q, k_pool, v_pool, r2t, req_rows, seq_lens, group_ptr, group_prefix_len,
                        max_seq_len, max_group_size, max_prefix_len, k_new=None, v_new=None,
                        scale=None, o=None, lse=None, workspace=None, stream=None):
    """Cascade decode: groups share a prefix read once per group; returns o."""
    torch = _torch()
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = group_prefix_len.numel()
    if o is None:
        o = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    ws_n = cascade_workspace_size(B, G, max_seq_len, max_group_size, max_prefix_len, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    _check("sgl_cascade_decode_attn", load().sgl_cascade_decode_attn(
        _dtype_code(q), _dev_ptr(q, "q", q.dtype), _dev_ptr(k_new, "k_new", q.dtype, True),
        _dev_ptr(v_new, "v_new", q.dtype, True), _dev_ptr(k_pool, "k_pool", q.dtype),
        _dev_ptr(v_pool, "v_pool", q.dtype), k_pool.shape[0], _dev_ptr(r2t, "r2t", torch.int32),
        r2t.shape[0], r2t.shape[1], _dev_ptr(req_rows, "req_rows", torch.int32),
        _dev_ptr(seq_lens, "seq_lens", torch.int32), _dev_ptr(group_ptr, "group_ptr", torch.int32),
        _dev_ptr(group_prefix_len, "group_prefix_len", torch.int32), B, G, max_seq_len,
        max_group_size, max_prefix_len, Hq, Hkv, D, scale, _dev_ptr(o, "o", q.dtype),
        _dev_ptr(lse, "lse", torch.float32, True), _dev_ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return o


# ---------------------------------------------------------------------------
# FP8 (e4m3fn) KV cache: uint8 code pools [S, Hkv, D] with float32 per-head
# factors k_scale / v_scale [Hkv] (code c of head kv stands for value(c) * scale[kv])
# ---------------------------------------------------------------------------
def _check_fp8_pools(k_pool, v_pool, k_scale, v_scale, Hkv, D):
    if tuple(k_pool.shape[1:]) != (Hkv, D) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_pool / v_pool must both be [num_slots, Hkv, D]")
    if k_scale.numel() != Hkv or v_scale.numel() != Hkv:
        raise ValueError("k_scale / v_scale must hold one factor per KV head")


def static_scratch_bytes():
    return int(load().sgl_static_scratch_bytes())


def cascade_decode_attn_static(q, k_pool, v_pool, r2t, req_rows, seq_lens, group_ptr, group_prefix_len,
                               max_seq_len, max_group_size, max_prefix_len, k_new=None, v_new=None,
                               scale=None, o=None, lse=None, stream=None):
    """Cascade decode whose split states live in the library's static device
    scratch (no workspace, no device allocation by the library); returns o."""
    torch = _torch()
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = group_prefix_len.numel()
    if o is None:
        o = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    _check("sgl_cascade_decode_attn_static", load().sgl_cascade_decode_attn_static(
        _dtype_code(q), _dev_ptr(q, "q", q.dtype), _dev_ptr(k_new, "k_new", q.dtype, True),
        _dev_ptr(v_new, "v_new", q.dtype, True), _dev_ptr(k_pool, "k_pool", q.dtype),
        _dev_ptr(v_pool, "v_pool", q.dtype), k_pool.shape[0], _dev_ptr(r2t, "r2t", torch.int32),
        r2t.shape[0], r2t.shape[1], _dev_ptr(req_rows, "req_rows", torch.int32),
        _dev_ptr(seq_lens, "seq_lens", torch.int32), _dev_ptr(group_ptr, "group_ptr", torch.int32),
        _dev_ptr(group_prefix_len, "group_prefix_len", torch.int32), B, G, max_seq_len,
        max_group_size, max_prefix_len, Hq, Hkv, D, scale, _dev_ptr(o, "o", q.dtype),
        _dev_ptr(lse, "lse", torch.float32, True), _stream(stream)))
    return o


def store_kv_fp8(k_new, v_new, slots, k_pool, v_pool, k_scale, v_scale, stream=None):
    """Quantise K/V rows [n, Hkv, D] (fp32 or bf16) into the code pools at slots."""
    torch = _torch()
    n, Hkv, D = k_new.shape
    _check_fp8_pools(k_pool, v_pool, k_scale, v_scale, Hkv, D)
    if tuple(v_new.shape) != tuple(k_new.shape) or slots.numel() != n:
        raise ValueError("v_new must match k_new and slots hold one slot per row")
    _check("sgl_store_kv_fp8", load().sgl_store_kv_fp8(
        _dtype_code(k_new), _dev_ptr(k_new, "k_new", k_new.dtype), _dev_ptr(v_new, "v_new", k_new.dtype), n,
        _dev_ptr(slots, "slots", torch.int32), _dev_ptr(k_pool, "k_pool", torch.uint8),
        _dev_ptr(v_pool, "v_pool", torch.uint8), k_pool.shape[0], Hkv, D,
        _dev_ptr(k_scale, "k_scale", torch.float32), _dev_ptr(v_scale, "v_scale", torch.float32),
        _stream(stream)))


def decode_attn_fp8kv(q, k_pool, v_pool, k_scale, v_scale, r2t, req_rows, seq_lens, max_seq_len,
                      k_new=None, v_new=None, scale=None, o=None, lse=None, workspace=None, stream=None):
    """decode_attn over an FP8 KV cache; q bf16 [batch, Hq, D]; returns o."""
    torch = _torch()
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    _check_fp8_pools(k_pool, v_pool, k_scale, v_scale, Hkv, D)
    if o is None:
        o = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    ws_n = decode_workspace_size(B, max_seq_len, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    _check("sgl_decode_attn_fp8kv", load().sgl_decode_attn_fp8kv(
        _dtype_code(q), _dev_ptr(q, "q", q.dtype), _dev_ptr(k_new, "k_new", q.dtype, True),
        _dev_ptr(v_new, "v_new", q.dtype, True), _dev_ptr(k_pool, "k_pool", torch.uint8),
        _dev_ptr(v_pool, "v_pool", torch.uint8), _dev_ptr(k_scale, "k_scale", torch.float32),
        _dev_ptr(v_scale, "v_scale", torch.float32), k_pool.shape[0], _dev_ptr(r2t, "r2t", torch.int32),
        r2t.shape[0], r2t.shape[1], _dev_ptr(req_rows, "req_rows", torch.int32),
        _dev_ptr(seq_lens, "seq_lens", torch.int32), B, max_seq_len, Hq, Hkv, D, scale,
        _dev_ptr(o, "o", q.dtype), _dev_ptr(lse, "lse", torch.float32, True),
        _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))
    return o


def cascade_decode_attn_fp8kv(q, k_pool, v_pool, k_scale, v_scale, r2t, req_rows, seq_lens, group_ptr,
                              group_prefix_len, max_seq_len, max_group_size, max_prefix_len, k_new=None,
                              v_new=None, scale=None, o=None, lse=None, workspace=None, stream=None):
    """cascade_decode_attn over an FP8 KV cache; returns o."""
    torch = _torch()
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    _check_fp8_pools(k_pool, v_pool, k_scale, v_scale, Hkv, D)
    G = group_prefix_len.numel()
    if o is None:
        o = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    ws_n = cascade_workspace_size(B, G, max_seq_len, max_group_size, max_prefix_len, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    _check("sgl_cascade_decode_attn_fp8kv", load().sgl_cascade_decode_attn_fp8kv(
        _dtype_code(q), _dev_ptr(q, "q", q.dtype), _dev_ptr(k_new, "k_new", q.dtype, True),
        _dev_ptr(v_new, "v_new", q.dtype, True), _dev_ptr(k_pool, "k_pool", torch.uint8),
        _dev_ptr(v_pool, "v_pool", torch.uint8), _dev_ptr(k_scale, "k_scale", torch.float32),
        _dev_ptr(v_scale, "v_scale", torch.float32), k_pool.shape[0], _dev_ptr(r2t, "r2t", torch.int32),
        r2t.shape[0], r2t.shape[1], _dev_ptr(req_rows, "req_rows", torch.int32),
        _dev_ptr(seq_lens, "seq_lens", torch.int32), _dev_ptr(group_ptr, "group_ptr", torch.int32),
        _dev_ptr(group_prefix_len, "group_prefix_len", torch.int32), B, G, max_seq_len,
        max_group_size, max_prefix_len, Hq, Hkv, D, scale, _dev_ptr(o, "o", q.dtype),
        _dev_ptr(lse, "lse", torch.float32, True), _dev_ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return o


# ---------------------------------------------------------------------------
# latent (MLA-style) decode: one latent row [576] per slot shared by all heads;
# scores over 576 dims, values = the first 512
# ---------------------------------------------------------------------------
MLA_DQK, MLA_DV = 576, 512


def mla_decode_workspace_size(batch, max_seq_len, Hq, Dv=MLA_DV):
    return int(load().sgl_mla_decode_workspace_size(batch, max_seq_len, Hq, Dv))


def mla_cascade_workspace_size(batch, G, max_seq_len, max_group_size, max_prefix_len, Hq, Dv=MLA_DV):
    return int(load().sgl_mla_cascade_workspace_size(batch, G, max_seq_len, max_group_size, max_prefix_len, Hq, Dv))


def _mla_out(q, o):
    torch = _torch()
    if o is None:
        o = torch.empty((q.shape[0], q.shape[1], MLA_DV), dtype=q.dtype, device=q.device)
    return o


def mla_decode_attn(q, kv_pool, r2t, req_rows, seq_lens, max_seq_len, kv_new=None, scale=None, o=None, lse=None,
                    workspace=None, stream=None):
    """Latent decode; q bf16 [batch, Hq, 576], kv_pool bf16 [S, 576]; returns o [batch, Hq, 512]."""
    torch = _torch()
    B, Hq, Dqk = q.shape
    o = _mla_out(q, o)
    if scale is None:
        scale = 1.0 / (192 ** 0.5)
    ws_n = mla_decode_workspace_size(B, max_seq_len, Hq)
    if workspace is None:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    _check("sgl_mla_decode_attn", load().sgl_mla_decode_attn(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(kv_new, "kv_new", torch.bfloat16, True),
        _dev_ptr(kv_pool, "kv_pool", torch.bfloat16), kv_pool.shape[0], _dev_ptr(r2t, "r2t", torch.int32),
        r2t.shape[0], r2t.shape[1], _dev_ptr(req_rows, "req_rows", torch.int32),
        _dev_ptr(seq_lens, "seq_lens", torch.int32), B, max_seq_len, Hq, Dqk, MLA_DV, scale,
        _dev_ptr(o, "o", torch.bfloat16), _dev_ptr(lse, "lse", torch.float32, True),
        _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))
    return o


def mla_cascade_decode_attn(q, kv_pool, r2t, req_rows, seq_lens, group_ptr, group_prefix_len, max_seq_len,
                            max_group_size, max_prefix_len, kv_new=None, scale=None, o=None, lse=None,
                            workspace=None, stream=None):
    """Latent cascade decode (each group's shared prefix read once per 64 query rows); returns o."""
    torch = _torch()
    B, Hq, Dqk = q.shape
    G = group_prefix_len.numel()
    o = _mla_out(q, o)
    if scale is None:
        scale = 1.0 / (192 ** 0.5)
    ws_n = mla_cascade_workspace_size(B, G, max_seq_len, max_group_size, max_prefix_len, Hq)
    if workspace is None:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    _check("sgl_mla_cascade_decode_attn", load().sgl_mla_cascade_decode_attn(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(kv_new, "kv_new", torch.bfloat16, True),
        _dev_ptr(kv_pool, "kv_pool", torch.bfloat16), kv_pool.shape[0], _dev_ptr(r2t, "r2t", torch.int32),
        r2t.shape[0], r2t.shape[1], _dev_ptr(req_rows, "req_rows", torch.int32),
        _dev_ptr(seq_lens, "seq_lens", torch.int32), _dev_ptr(group_ptr, "group_ptr", torch.int32),
        _dev_ptr(group_prefix_len, "group_prefix_len", torch.int32), B, G, max_seq_len, max_group_size,
        max_prefix_len, Hq, Dqk, MLA_DV, scale, _dev_ptr(o, "o", torch.bfloat16),
        _dev_ptr(lse, "lse", torch.float32, True), _dev_ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return o


def _tier_args(host_k, host_v, k_pool, v_pool):
    """Check a host tier against its pool; returns (host_k, host_v, k_pool, v_pool) pointers and row bytes."""
    if (host_v is None) != (v_pool is None):
        raise ValueError("host_v and v_pool go together (both or neither)")
    for h, p, name in ((host_k, k_pool, "k"), (host_v, v_pool, "v")):
        if h is None:
            continue
        if h.is_cuda or not h.is_pinned():
            raise ValueError(f"host_{name} must be a page-locked (pinned) CPU tensor")
        if not h.is_contiguous() or not p.is_contiguous():
            raise ValueError(f"host_{name} and the pool must be contiguous")
        if h.dtype != p.dtype or tuple(h.shape[1:]) != tuple(p.shape[1:]):
            raise ValueError(f"host_{name} rows must have the pool's row shape and dtype")
    if host_v is not None and (host_v.shape[0] != host_k.shape[0] or v_pool.shape[0] != k_pool.shape[0]):
        raise ValueError("K and V tiers (and pools) must have the same number of rows")
    row_bytes = k_pool[0].numel() * k_pool.element_size()
    hv = None if host_v is None else ctypes.c_void_p(host_v.data_ptr())
    return (ctypes.c_void_p(host_k.data_ptr()), hv, _dev_ptr(k_pool, "k_pool"),
            _dev_ptr(v_pool, "v_pool", None, True), row_bytes)


def hicache_prefetch(host_k, host_v, host_rows, slots, k_pool, v_pool=None, stream=None):
    """pool[slots[i]] <- host[host_rows[i]] (host tier -> GPU pool), for K and V (or one latent tier)."""
    torch = _torch()
    hk, hv, kp, vp, row_bytes = _tier_args(host_k, host_v, k_pool, v_pool)
    if host_rows.numel() != slots.numel():
        raise ValueError("host_rows and slots must have the same length")
    _check("sgl_hicache_prefetch", load().sgl_hicache_prefetch(
        hk, hv, host_k.shape[0], _dev_ptr(host_rows, "host_rows", torch.int64),
        _dev_ptr(slots, "slots", torch.int32), slots.numel(), kp, vp, k_pool.shape[0], row_bytes, _stream(stream)))


def hicache_write_back(k_pool, v_pool, slots, host_rows, host_k, host_v=None, stream=None):
    """host[host_rows[i]] <- pool[slots[i]] (GPU pool -> host tier); synchronise before reading the host tier."""
    torch = _torch()
    hk, hv, kp, vp, row_bytes = _tier_args(host_k, host_v, k_pool, v_pool)
    if host_rows.numel() != slots.numel():
        raise ValueError("host_rows and slots must have the same length")
    _check("sgl_hicache_write_back", load().sgl_hicache_write_back(
        kp, vp, k_pool.shape[0], _dev_ptr(slots, "slots", torch.int32), _dev_ptr(host_rows, "host_rows", torch.int64),
        slots.numel(), hk, hv, host_k.shape[0], row_bytes, _stream(stream)))


# ---------------------------------------------------------------------------
# measurement helpers (sgl_probe.h): the chip's sustained MFMA rate and copy
# bandwidth, reported beside the published peaks
# ---------------------------------------------------------------------------
PROBE_THREADS = 256


def probe_mfma_bf16(out, iters, x=1.0, stream=None):
    """Enqueue the dense bf16 MFMA probe over out.numel() // 256 workgroups;
    returns the floating-point operations the launch performs."""
    torch = _torch()
    n_wg = out.numel() // PROBE_THREADS
    _check("sgl_probe_mfma_bf16", load().sgl_probe_mfma_bf16(
        n_wg, int(iters), float(x), _dev_ptr(out, "out", torch.float32), _stream(stream)))
    return n_wg * 4 * int(iters) * 8 * 32768


def probe_copy(src, dst, stream=None):
    """Enqueue dst <- src (same byte size, 16-byte multiple); returns the bytes moved (read + written)."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst must have the same byte size")
    _check("sgl_probe_copy", load().sgl_probe_copy(_dev_ptr(src, "src"), _dev_ptr(dst, "dst"), nb, _stream(stream)))
    return 2 * nb
