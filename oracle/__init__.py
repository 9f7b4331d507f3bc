"""Oracle: plain, slow, obviously correct CPU reference for the hot path.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  The product package
(prefix_shared_paged_amd) never imports it and shares no code with it.

Contents
  attention(...)        fp64 softmax(q k^T / sqrt(D), causal) v over logical
                        per-request sequences (C library, attn_oracle.c)
  attention_probs(...)  explicit probability matrix of one request / head
  merge_states(...)     merge of two partial softmax states
  fp8                   OCP e4m3fn codes: decode, encode, per-head KV
                        quantisation (pure numpy, see fp8.py)
  radix_model           brute-force prefix cache + slot allocator model
                        (pure Python, see radix_model.py)
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        alt = os.environ.get("ORACLE_LIBRARY")   # another build of attn_oracle.c (the sanitizer check)
        if alt:
            lib = ctypes.CDLL(alt)
        else:
            if (not os.path.exists(_build.LIB)
                    or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
                _build.build()
            lib = ctypes.CDLL(_build.LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int32
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [i64, p, p, p, i64, p, p, p, i32, i32, i32,
                                         ctypes.c_double, p, i32, p, p, p, p, p, p,
                                         i32, i32]
        lib.oracle_attention_kv_scaled.restype = ctypes.c_int
        lib.oracle_attention_kv_scaled.argtypes = [i64, p, p, p, p, p, i64, p, p, p, i32, i32,
                                                   i32, ctypes.c_double, p, i32, p, p, p, p,
                                                   p, p, i32, i32]
        lib.oracle_attention_dv.restype = ctypes.c_int
        lib.oracle_attention_dv.argtypes = [i64, p, p, p, p, p, i64, p, p, p, i32, i32, i32, i32,
                                            ctypes.c_double, p, i32, p, p, p, p, p, p, i32, i32]
        lib.oracle_attention_probs.restype = ctypes.c_int
        lib.oracle_attention_probs.argtypes = [i64, p, i64, p, p, i32, i32, i32, i32,
                                               ctypes.c_double, p]
        lib.oracle_merge_states.restype = None
        lib.oracle_merge_states.argtypes = [i64, i32, p, p, p, p, p, p, p, p, p]
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def attention(K_list, V_list, row_req, row_pos, Q, Hq, Hkv, scale=None, heads=None,
              key_lo=None, key_hi=None, method=0, threads=None, kv_scale=None):
    """Attention of query rows over their request's logical sequence.

    K_list / V_list: per request float32 arrays [L_r, Hkv, D] and [L_r, Hkv, Dv]
      (logical order, position j is row j; Dv may differ from D: attention in
      a latent space whose scores use D dims and values Dv) -- or a single
      concatenated array plus offsets via ``kv_off`` in a tuple (K_cat, kv_off).
    row_req[i], row_pos[i]: request and absolute position of query row i.
    Q: float32 [n_rows, Hq, D].
    heads: optional list of q heads to evaluate (default all).
    key_lo / key_hi: optional per-row key range (intersected with j <= t).
    kv_scale: optional (k_scale, v_scale), each [Hkv]: the keys and values
      attended are K * k_scale[kv] and V * v_scale[kv] (a dequantised KV
      cache: K / V hold the decoded codes, see oracle.fp8), formed in fp64.
    Returns (O [n_rows, n_heads, Dv], M, Lsum, LSE [n_rows, n_heads]) in float64.
    """
    lib = _load()
    if isinstance(K_list, tuple):
        K, kv_off = K_list
        V, _ = V_list
    else:
        lens = [k.shape[0] for k in K_list]
        kv_off = np.zeros(len(lens) + 1, np.int64)
        kv_off[1:] = np.cumsum(lens)
        K = np.concatenate(K_list, axis=0) if K_list else np.zeros((0, Hkv, Q.shape[2]), np.float32)
        V = np.concatenate(V_list, axis=0) if V_list else np.zeros((0, Hkv, Q.shape[2]), np.float32)
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    Q = np.ascontiguousarray(Q, np.float32)
    kv_off = np.ascontiguousarray(kv_off, np.int64)
    D = Q.shape[2]
    Dv = V.shape[2]
    assert K.shape[1] == Hkv and K.shape[2] == D and Q.shape[1] == Hq
    assert V.shape[0] == K.shape[0] and V.shape[1] == Hkv
    row_req = np.ascontiguousarray(row_req, np.int64)
    row_pos = np.ascontiguousarray(row_pos, np.int64)
    n_rows = row_req.shape[0]
    if heads is not None:
        heads = np.ascontiguousarray(heads, np.int32)
        n_heads = heads.shape[0]
    else:
        n_heads = Hq
    if key_lo is not None:
        key_lo = np.ascontiguousarray(key_lo, np.int64)
    if key_hi is not None:
        key_hi = np.ascontiguousarray(key_hi, np.int64)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    O = np.zeros((n_rows, n_heads, Dv), np.float64)
    M = np.zeros((n_rows, n_heads), np.float64)
    Ls = np.zeros((n_rows, n_heads), np.float64)
    LSE = np.zeros((n_rows, n_heads), np.float64)
    ks = vs = None
    if kv_scale is not None:
        ks = np.ascontiguousarray(kv_scale[0], np.float64).reshape(-1)
        vs = np.ascontiguousarray(kv_scale[1], np.float64).reshape(-1)
        assert ks.shape[0] == Hkv and vs.shape[0] == Hkv
    rc = lib.oracle_attention_dv(len(kv_off) - 1, _ptr(kv_off), _ptr(K), _ptr(V),
                                 _ptr(ks), _ptr(vs), n_rows,
                                 _ptr(row_req), _ptr(row_pos), _ptr(Q), Hq, Hkv, D, Dv,
                                 float(scale), _ptr(heads), n_heads, _ptr(key_lo),
                                 _ptr(key_hi), _ptr(O), _ptr(M), _ptr(Ls), _ptr(LSE),
                                 int(method), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_attention: invalid arguments")
    return O, M, Ls, LSE


def attention_probs(K, pos, Q, Hq, Hkv, h, scale=None):
    """Explicit probability matrix P [n_q, L] of one request and q head h."""
    lib = _load()
    K = np.ascontiguousarray(K, np.float32)
    Q = np.ascontiguousarray(Q, np.float32)
    pos = np.ascontiguousarray(pos, np.int64)
    L, D = K.shape[0], K.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    P = np.zeros((pos.shape[0], L), np.float64)
    rc = lib.oracle_attention_probs(L, _ptr(K), pos.shape[0], _ptr(pos), _ptr(Q), Hq, Hkv,
                                    D, int(h), float(scale), _ptr(P))
    if rc != 0:
        raise ValueError("oracle_attention_probs: invalid arguments")
    return P


def merge_states(mA, lA, oA, mB, lB, oB):
    """Merge partial softmax states (m, l, o) over two disjoint key sets."""
    lib = _load()
    mA, lA, mB, lB = (np.ascontiguousarray(x, np.float64).reshape(-1) for x in (mA, lA, mB, lB))
    D = oA.shape[-1]
    oA = np.ascontiguousarray(oA, np.float64).reshape(-1, D)
    oB = np.ascontiguousarray(oB, np.float64).reshape(-1, D)
    n = mA.shape[0]
    mO = np.zeros(n, np.float64)
    lO = np.zeros(n, np.float64)
    oO = np.zeros((n, D), np.float64)
    lib.oracle_merge_states(n, D, _ptr(mA), _ptr(lA), _ptr(oA), _ptr(mB), _ptr(lB), _ptr(oB),
                            _ptr(mO), _ptr(lO), _ptr(oO))
    return mO, lO, oO
