"""Algorithmic work of the attention calls (what the method must do, not what
a kernel happens to move): the denominators of every throughput and
roofline figure.

  kv bytes per token = 2 (K and V) * layers * Hkv * D * element bytes
      ("SGLang 深度拆解" (chenxutan.com) section 4.3 prints this product for
      Llama3.1-70B in bf16: 2*80*8*128*2 = 327,680 bytes per token).
  extend FLOPs = 4 * D per unmasked (query token, key, query head) triple
      (2 for q.k, 2 for p*v); the masked triangle is not counted.
  decode bytes = every K/V row the method must read (flat: each request
      its whole context; cascade: a group's shared prefix once) + the
      req_to_token entries it reads + Q + O + the store of the current
      tokens' K/V when the call makes it (stored = tokens stored: their new
      K/V read and their pool rows written).  With an FP8 KV cache the K/V
      rows take 1 byte per element (kv element size) while Q, O and the
      stored tokens' inputs keep theirs (q_elt).
"""
import numpy as np


def kv_bytes_per_token(Hkv, D, elt, layers=1):
    return 2 * layers * Hkv * D * elt


def extend_flops(prefix_lens, extend_lens, Hq, D):
    P = np.asarray(prefix_lens, np.float64)
    E = np.asarray(extend_lens, np.float64)
    # sum over i in [0, E) of (P + i + 1) visible keys
    pairs = E * P + E * (E + 1) / 2
    return float(4 * D * Hq * pairs.sum())


def extend_bytes(prefix_lens, extend_lens, Hq, Hkv, D, elt, shared_prefix_groups=None):
    """Q + O + the new K/V written and read once + prefix K/V read once per
    distinct prefix + req_to_token entries."""
    P = np.asarray(prefix_lens, np.int64)
    E = np.asarray(extend_lens, np.int64)
    kv = kv_bytes_per_token(Hkv, D, elt)
    n_new = int(E.sum())
    prefix_tokens = int(P.sum()) if shared_prefix_groups is None else int(sum(shared_prefix_groups))
    return (2 * n_new * Hq * D * elt            # Q read, O written
            + 2 * n_new * kv                    # new K/V: stored, then read
            + prefix_tokens * kv                # cached prefix read
            + 4 * int((P + E).sum()))           # req_to_token entries


def _store_bytes(stored, Hkv, D, elt, q_elt):
    return int(stored) * (kv_bytes_per_token(Hkv, D, q_elt) + kv_bytes_per_token(Hkv, D, elt))


def decode_bytes_flat(seq_lens, Hq, Hkv, D, elt, q_elt=None, stored=0):
    L = np.asarray(seq_lens, np.int64)
    B = len(L)
    q_elt = elt if q_elt is None else q_elt
    return (int(L.sum()) * (kv_bytes_per_token(Hkv, D, elt) + 4) + 2 * B * Hq * D * q_elt
            + _store_bytes(stored, Hkv, D, elt, q_elt))


def decode_bytes_cascade(seq_lens, group_of, group_prefix, Hq, Hkv, D, elt, q_elt=None, stored=0):
    L = np.asarray(seq_lens, np.int64)
    gp = np.asarray(group_prefix, np.int64)
    g = np.asarray(group_of, np.int64)
    B = len(L)
    q_elt = elt if q_elt is None else q_elt
    tokens = int(gp.sum()) + int((L - gp[g]).sum())
    return (tokens * (kv_bytes_per_token(Hkv, D, elt) + 4) + 2 * B * Hq * D * q_elt
            + _store_bytes(stored, Hkv, D, elt, q_elt))


def decode_flops(seq_lens, Hq, D):
    return float(4 * D * Hq * np.asarray(seq_lens, np.float64).sum())
