"""Scenario drivers for the GPU parity tests.

Each driver sets up a paged KV cache on the GPU through the library (slot
pool, radix tree, req_to_token, KV store), runs one attention call, and
replays the same bookkeeping on the brute-force model (oracle/radix_model.py)
to produce the expected req_to_token rows.  Expected attention values come
from the fp64 oracle over the LOGICAL sequences drawn by workloads/.
"""
import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import oracle.fp8 as F8
import workloads as W
from oracle.radix_model import PrefixCache, SlotPool
from prefix_shared_paged_amd import (cascade_decode_attn, cascade_decode_attn_fp8kv, decode_attn,
                                     decode_attn_fp8kv, extend_attn)
from prefix_shared_paged_amd.paged_cache import PagedKVCache

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(x, dt):
    """float32 array holding exact values of dtype `dt` -> GPU tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").to(TORCH_DT[dt])


def dev_i(x, dtype=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(x)).to(dtype).to("cuda")


class Mirror:
    """The brute-force model fed with the same operations as the library."""

    def __init__(self, spec, order):
        self.pool = SlotPool(spec.num_slots, spec.page_size, order)
        self.tree = PrefixCache(spec.page_size)
        self.rows = {}

    def admit(self, row, toks):
        n, slots, _ = self.tree.match(toks)
        self.rows[row] = list(slots)
        return n

    def append(self, row, n):
        cur = self.rows[row]
        self.rows[row] = cur + self.pool.alloc(len(cur), cur[-1] if cur else -1, n)

    def insert(self, row, toks):
        self.tree.insert(toks, self.rows[row][:len(toks)], self.pool)
        self.tree.match(toks[:len(toks) // self.tree.p * self.tree.p])   # the driver re-matches

    def expected_r2t(self, num_rows, stride):
        t = np.full((num_rows, stride), -1, np.int32)
        for r, s in self.rows.items():
            t[r, :len(s)] = s
        return t


class GroupCase:
    """Prefix groups set up in a fresh cache; requests admitted on top."""

    def __init__(self, wl, order=None, max_rows=None, row_stride=None, creator_extend=False, fp8=False):
        """fp8: the pools hold e4m3fn codes with the workload's per-head factors."""
        self.wl = wl
        s = wl.spec
        self.order = W.pool_order(s) if order is None else order
        n_rows = max_rows or (wl.B + wl.G)
        stride = row_stride or int(max(wl.ctx_len.max(), wl.prefix_len.max())) + 1
        assert not (fp8 and creator_extend)
        self.fp8 = fp8
        self.kv_scale = W.fp8_scales(s) if fp8 else None
        self.cache = PagedKVCache(s.num_slots, s.page_size, s.Hkv, s.D, TORCH_DT[s.dtype], n_rows, stride,
                                  self.order, kv_scale=self.kv_scale)
        self.mirror = Mirror(s, self.order)
        self.prefix_kv = {}
        self.creator_out = []
        for g in range(wl.G):
            toks = wl.prefix_tokens(g)
            if len(toks) == 0:
                self.prefix_kv[g] = wl.prefix_kv(g)
                continue
            [st] = self.cache.admit([toks])
            assert st.matched == 0 and self.mirror.admit(st.row, toks) == 0
            self.cache.append([st], [len(toks)])
            self.mirror.append(st.row, len(toks))
            K, V = wl.prefix_kv(g)
            self.prefix_kv[g] = (K, V)
            if creator_extend:
                # the prefix itself goes through an extend with no cached prefix
                q = wl.queries(10 ** 6 + g, len(toks))
                o = extend_attn(dev(q, s.dtype), self.cache.k_pool, self.cache.v_pool, self.cache.r2t,
                                self.cache.rows_tensor([st]), dev_i([0]), dev_i([0, len(toks)], torch.int64),
                                len(toks), k_new=dev(K, s.dtype), v_new=dev(V, s.dtype))
                self.creator_out.append((g, q, o.float().cpu().numpy()))
            else:
                self.cache.store(dev(K, s.dtype), dev(V, s.dtype), st.slots)
            self.cache.insert(st)
            self.mirror.insert(st.row, list(toks))
            self.cache.release(st)
            self.mirror.rows.pop(st.row)
        self.req_rows = []
        self.full_suffix_kv = {}

    def admit_requests(self, n_suffix):
        """Admit every request with tokens prefix || suffix[:n_suffix[r]]."""
        wl = self.wl
        toks = [np.concatenate([wl.prefix_tokens(wl.grp[r]), wl.suffix_tokens(r, n=int(n_suffix[r]))])
                for r in range(wl.B)]
        rows = self.cache.admit(toks)
        for r, st in enumerate(rows):
            assert self.mirror.admit(st.row, list(toks[r])) == st.matched
            assert st.matched == wl.prefix_len[wl.grp[r]]
        self.rows = rows
        return rows

    def suffix_kv(self, r):
        if r not in self.full_suffix_kv:
            n = int(self.wl.ctx_len[r] - self.wl.prefix_len[self.wl.grp[r]])
            self.full_suffix_kv[r] = self.wl.suffix_kv(r, n)
        return self.full_suffix_kv[r]

    def logical_kv(self, r, n_suffix):
        Kp, Vp = self.prefix_kv[self.wl.grp[r]]
        Ks, Vs = self.suffix_kv(r)
        return np.concatenate([Kp, Ks[:n_suffix]]), np.concatenate([Vp, Vs[:n_suffix]])

    def check_r2t(self):
        got = self.cache.r2t.cpu().numpy()
        want = self.mirror.expected_r2t(*got.shape)
        for st in self.rows:
            np.testing.assert_array_equal(got[st.row, :len(st.slots)], want[st.row, :len(st.slots)])
            np.testing.assert_array_equal(got[st.row, :len(st.slots)], st.slots)


def run_extend(case, E, lse=True):
    """All requests extend E[r] new tokens over their cached group prefix."""
    wl = case.wl
    s = wl.spec
    rows = case.admit_requests(E)
    case.cache.append(rows, E)
    for st, e in zip(rows, E):
        case.mirror.append(st.row, int(e))
    q = [wl.queries(r, int(E[r])) for r in range(wl.B)]
    Kn = [case.suffix_kv(r)[0][:E[r]] for r in range(wl.B)]
    Vn = [case.suffix_kv(r)[1][:E[r]] for r in range(wl.B)]
    q_off = np.zeros(wl.B + 1, np.int64)
    q_off[1:] = np.cumsum(E)
    P = np.array([wl.prefix_len[wl.grp[r]] for r in range(wl.B)], np.int32)
    qd = dev(np.concatenate(q), s.dtype)
    lse_t = torch.empty((qd.shape[0], s.Hq), dtype=torch.float32, device="cuda") if lse else None
    o = extend_attn(qd, case.cache.k_pool, case.cache.v_pool, case.cache.r2t, case.cache.rows_tensor(rows),
                    dev_i(P), dev_i(q_off, torch.int64), int(max(E.max(), 1)),
                    k_new=dev(np.concatenate(Kn), s.dtype), v_new=dev(np.concatenate(Vn), s.dtype), lse=lse_t)
    torch.cuda.synchronize()
    return dict(o=o.float().cpu().numpy(), lse=None if lse_t is None else lse_t.cpu().numpy(), q=q,
                q_off=q_off, P=P, E=E)


def oracle_extend(case, res, rows_sample=None, heads=None):
    """Oracle for the extend rows (all, or a list of (request, i) pairs)."""
    wl = case.wl
    s = wl.spec
    reqs = range(wl.B) if rows_sample is None else sorted({r for r, _ in rows_sample})
    Ks, Vs, rr, pos, Q, idx = [], [], [], [], [], []
    for k, r in enumerate(reqs):
        E = int(res["E"][r])
        K, V = case.logical_kv(r, E)
        Ks.append(K)
        Vs.append(V)
        ii = range(E) if rows_sample is None else [i for rq, i in rows_sample if rq == r]
        for i in ii:
            rr.append(k)
            pos.append(int(res["P"][r]) + i)
            Q.append(res["q"][r][i])
            idx.append(int(res["q_off"][r]) + i)
    O, M, L, LSE = oracle.attention(Ks, Vs, rr, pos, np.stack(Q), s.Hq, s.Hkv, heads=heads)
    return np.array(idx), O, LSE


def run_decode(case, L, cascade, both=False, workspace=None):
    """All requests decode one token at position L[r]-1 (L includes it).
    cascade: use the cascade call; both: run the flat call first (it stores the
    current token's K/V), then the cascade call on the same rows.  workspace:
    the cascade call's workspace (else one sized for this call)."""
    wl = case.wl
    s = wl.spec
    P = np.array([wl.prefix_len[wl.grp[r]] for r in range(wl.B)], np.int64)
    rows = case.admit_requests(L - P)
    case.cache.append(rows, L - P)
    for st, n in zip(rows, L - P):
        case.mirror.append(st.row, int(n))
    # cached history of the suffix (all but the current token)
    for r, st in enumerate(rows):
        n_hist = int(L[r] - P[r] - 1)
        if n_hist > 0:
            Ks, Vs = case.suffix_kv(r)
            case.cache.store(dev(Ks[:n_hist], s.dtype), dev(Vs[:n_hist], s.dtype), st.slots[P[r]:L[r] - 1])
    kn = np.stack([case.suffix_kv(r)[0][L[r] - P[r] - 1] for r in range(wl.B)])
    vn = np.stack([case.suffix_kv(r)[1][L[r] - P[r] - 1] for r in range(wl.B)])
    q = np.stack([wl.queries(r, 1)[0] for r in range(wl.B)])
    req_rows = case.cache.rows_tensor(rows)
    qd = dev(q, s.dtype)
    out = dict(q=q, L=L, P=P)

    c = case.cache
    fp8_args = (c.k_pool, c.v_pool, c.k_scale, c.v_scale) if case.fp8 else (c.k_pool, c.v_pool)

    def flat(store):
        lse_t = torch.empty((wl.B, s.Hq), dtype=torch.float32, device="cuda")
        kw = dict(k_new=dev(kn, s.dtype), v_new=dev(vn, s.dtype)) if store else {}
        fn = decode_attn_fp8kv if case.fp8 else decode_attn
        o = fn(qd, *fp8_args, c.r2t, req_rows, dev_i(L), int(L.max()), lse=lse_t, **kw)
        return o, lse_t

    def casc(store):
        lse_t = torch.empty((wl.B, s.Hq), dtype=torch.float32, device="cuda")
        kw = dict(k_new=dev(kn, s.dtype), v_new=dev(vn, s.dtype)) if store else {}
        gptr = np.zeros(wl.G + 1, np.int32)
        gptr[1:] = np.cumsum(np.bincount(wl.grp, minlength=wl.G))
        fn = cascade_decode_attn_fp8kv if case.fp8 else cascade_decode_attn
        if workspace is not None:
            kw["workspace"] = workspace
        o = fn(qd, *fp8_args, c.r2t, req_rows, dev_i(L), dev_i(gptr), dev_i(wl.prefix_len), int(L.max()),
               int(np.diff(gptr).max()), int(wl.prefix_len.max()), lse=lse_t, **kw)
        return o, lse_t

    if both:
        o, l = flat(True)
        oc, lc = casc(False)
        torch.cuda.synchronize()
        out.update(o=o.float().cpu().numpy(), lse=l.cpu().numpy(), o_c=oc.float().cpu().numpy(),
                   lse_c=lc.cpu().numpy())
    else:
        o, l = casc(True) if cascade else flat(True)
        torch.cuda.synchronize()
        out.update(o=o.float().cpu().numpy(), lse=l.cpu().numpy())
    return out


_FP8_LOCK = threading.Lock()


def _fp8_logical_kv(case, r, n_suffix):
    """The oracle's own FP8 codes of request r's logical K/V, decoded exactly.
    Coding is elementwise (per-head factors), so a group's prefix is coded
    once and reused by its members."""
    deq = lambda x, sc: F8.decode(F8.quantize(x, sc)).astype(np.float32)
    cache = case.__dict__.setdefault("_fp8_prefix_codes", {})
    g = int(case.wl.grp[r])
    with _FP8_LOCK:
        if g not in cache:
            Kp, Vp = case.prefix_kv[g]
            cache[g] = (deq(Kp, case.kv_scale[0]), deq(Vp, case.kv_scale[1]))
    Ks, Vs = case.suffix_kv(r)
    return (np.concatenate([cache[g][0], deq(Ks[:n_suffix], case.kv_scale[0])]),
            np.concatenate([cache[g][1], deq(Vs[:n_suffix], case.kv_scale[1])]))


def oracle_decode(case, res, reqs=None, heads=None, batch=16):
    wl = case.wl
    s = wl.spec
    reqs = list(range(wl.B)) if reqs is None else list(reqs)
    Os, LSEs = [], []
    for b0 in range(0, len(reqs), batch):
        part = reqs[b0:b0 + batch]
        n_suf = [int(res["L"][r] - res["P"][r]) for r in part]
        if case.fp8:   # the coding runs in numpy, which releases the GIL: one thread per request
            for r in part:
                case.suffix_kv(r)
            with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
                KV = list(ex.map(lambda a: _fp8_logical_kv(case, *a), zip(part, n_suf)))
        else:
            KV = [case.logical_kv(r, n) for r, n in zip(part, n_suf)]
        Ks = [k for k, _ in KV]
        Vs = [v for _, v in KV]
        O, M, Ls, LSE = oracle.attention(Ks, Vs, np.arange(len(part)), [int(res["L"][r]) - 1 for r in part],
                                         res["q"][part], s.Hq, s.Hkv, heads=heads, kv_scale=case.kv_scale)
        Os.append(O)
        LSEs.append(LSE)
    return np.array(reqs), np.concatenate(Os), np.concatenate(LSEs)


def bf16_err(got, want):
    return float(np.max(np.abs(got.astype(np.float64) - want)))


def f32_rel_err(got, want):
    """max over (row, head) of ||o - r||_inf / ||r||_inf."""
    num = np.max(np.abs(got.astype(np.float64) - want), axis=-1)
    den = np.max(np.abs(want), axis=-1)
    return float(np.max(num / np.maximum(den, 1e-30)))


def many_rounds_workload(seed, Hq=16, Hkv=2, D=128):
    """A group whose prefix covers nearly all of a 9,000-key context beside a
    request with no prefix at all: max_seq_len - max_prefix_len is 10, so the
    suffix splits are 64 keys and a two-launch cascade's suffix grid holds 2
    split rounds, while the prefix-less request needs 141 -- each suffix
    workgroup then runs up to 70 later items, found 64 per ballot."""
    spec = W.Spec("many_rounds", "bf16", Hq, Hkv, D, 1, 1 << 15, 0.5, seed)
    members = [2, 1]
    prefixes = [8990, 0]
    grp = np.concatenate([np.full(m, g) for g, m in enumerate(members)]).astype(np.int64)
    sib = np.concatenate([np.arange(m) for m in members]).astype(np.int64)
    L = np.array([8995, 9000, 9000], np.int64)
    return W.GroupWorkload(spec, np.array(prefixes, np.int64), grp, sib, L)


def late_rounds_workload(seed, Hq=32, Hkv=8, D=128):
    """One group with a 4000-token prefix and short suffixes beside groups
    with short prefixes and suffixes of up to 4080 keys: max_seq_len -
    max_prefix_len is 96, so the one-grid cascade puts only the first few
    suffix split rounds before the prefix items, and the long suffixes' later
    splits run in the rounds dispatched after them."""
    spec = W.Spec("late_rounds", "bf16", Hq, Hkv, D, 1, 1 << 15, 0.5, seed)
    members = [3, 2, 1, 4]
    prefixes = [4000, 16, 0, 2000]
    grp = np.concatenate([np.full(m, g) for g, m in enumerate(members)]).astype(np.int64)
    sib = np.concatenate([np.arange(m) for m in members]).astype(np.int64)
    L = np.array([4001, 4050, 4096, 4096, 3000, 2500, 2001, 2600, 4000, 4096], np.int64)
    assert len(L) == len(grp)
    return W.GroupWorkload(spec, np.array(prefixes, np.int64), grp, sib, L)
