"""GPU parity for the multi-turn mix: sessions with a ~70% cached history,
chunked prefill (chunks of 512) interleaved with decode, page size 16,
64 query / 8 KV heads, bf16.

req_to_token: every allocation the runner makes (the setup of the cached
histories, every chunk append, every decode append) and every insert at
prefill completion is replayed on the brute-force slot pool and trie
(oracle/radix_model.py), and every session's req_to_token row is compared
bit-exactly with the model's slot list.  Attention: outputs are checked
against the fp64 oracle on sampled rows (the first, last and one random row
of every chunk, and every decode token) of every session, on one query head
per KV group."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.radix_model import PrefixCache, SlotPool
from prefix_shared_paged_amd.chunked import ChunkedRunner, plan_rounds
from prefix_shared_paged_amd.paged_cache import PagedKVCache

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").to(torch.bfloat16)


def st_decoded(runner, sid):
    return next(x.decoded for x in runner.sessions if x.sid == sid)


def run_multiturn(wl, check_sessions, rng_seed=0):
    s = wl.spec
    n = wl.n
    hist, cached = wl.hist, wl.cached
    rounds = plan_rounds(hist, cached, wl.chunk)
    max_dec = max(sum(1 for _, dl in rounds for i, _ in dl if i == sid) for sid in range(n))
    stride = int(hist.max()) + max_dec + 16
    order = W.pool_order(s)
    cache = PagedKVCache(s.num_slots, s.page_size, s.Hkv, s.D, torch.bfloat16, 2 * n, stride, order)
    model_pool, model_tree = SlotPool(s.num_slots, s.page_size, order), PrefixCache(s.page_size)
    toks = [W.tokens(s, W.T_TOK_PREFIX, int(hist[i]) + max_dec, i + 1, i) for i in range(n)]
    # earlier turns: the cached part of every session is already in the tree
    setup = cache.admit([t[:int(c)] for t, c in zip(toks, cached)])
    cache.append(setup, [int(c) for c in cached])
    for i, st in enumerate(setup):
        assert st.matched == 0
        K, V = wl.kv(i, 0, int(cached[i]))
        cache.store(_dev(K), _dev(V), st.slots)
        m_slots = model_pool.alloc(0, -1, int(cached[i]))
        assert list(st.slots) == m_slots            # same allocator decisions, bit-exact
        cache.insert(st)
        model_tree.insert(list(toks[i][:int(cached[i])]), m_slots, model_pool)
        cache.release(st)
    runner = ChunkedRunner(cache, wl.chunk)
    rows = runner.admit(list(range(n)), toks, hist)
    model_slots = {}
    for i, st in enumerate(rows):
        m, m_slots, _ = model_tree.match(list(toks[i]))
        assert st.matched == m == cached[i]
        assert list(st.slots) == m_slots
        model_slots[i] = list(m_slots)

    def model_append(sid, k):
        cur = model_slots[sid]
        cur += model_pool.alloc(len(cur), cur[-1] if cur else -1, k)

    def inputs(ext, dec):
        q = np.concatenate([wl.queries(i, lo, hi) for i, lo, hi in ext]) if ext else np.zeros((0, s.Hq, s.D))
        kv = [wl.kv(i, lo, hi) for i, lo, hi in ext]
        k = np.concatenate([a for a, _ in kv]) if kv else np.zeros((0, s.Hkv, s.D))
        v = np.concatenate([b for _, b in kv]) if kv else np.zeros((0, s.Hkv, s.D))
        qd = np.concatenate([wl.queries(i, p, p + 1) for i, p in dec]) if dec else np.zeros((0, s.Hq, s.D))
        kvd = [wl.kv(i, p, p + 1) for i, p in dec]
        kd = np.concatenate([a for a, _ in kvd]) if kvd else np.zeros((0, s.Hkv, s.D))
        vd = np.concatenate([b for _, b in kvd]) if kvd else np.zeros((0, s.Hkv, s.D))
        return tuple(_dev(x) for x in (q, k, v, qd, kd, vd))

    rng = np.random.default_rng(rng_seed)
    heads = [9 * k for k in range(s.Hkv)]           # one q head per KV group (64/8)
    samples = {i: [] for i in check_sessions}        # sid -> list of (pos, q row, gpu out [heads, D])
    done_rounds = 0
    while True:
        last = not runner.pending()
        out = runner.run_round(inputs)
        assert out is not None
        ext_plan, dec_plan = rounds[done_rounds]
        assert [(a, b, c) for a, b, c, _ in out["extend"]] == ext_plan
        assert out["decode"] == [(i, p + 1) for i, p in dec_plan]
        # the same round on the model: chunk appends, inserts at prefill
        # completion (the runner re-matches the inserted prefix), decode appends
        for sid, lo, hi, _ in out["extend"]:
            model_append(sid, hi - lo)
        for sid, lo, hi, _ in out["extend"]:
            if hi >= hist[sid]:
                h = int(hist[sid])
                model_tree.insert(list(toks[sid][:h]), model_slots[sid][:h], model_pool)
                model_tree.match(list(toks[sid][:h // s.page_size * s.page_size]))
        for sid, _ in out["decode"]:
            model_append(sid, 1)
        torch.cuda.synchronize()
        if out["extend"]:
            o = out["extend_out"]
            for sid, lo, hi, off in out["extend"]:
                if sid not in samples:
                    continue
                for i in sorted({0, hi - lo - 1, int(rng.integers(hi - lo))}):
                    samples[sid].append((lo + i, wl.queries(sid, lo + i, lo + i + 1)[0],
                                         o[off + i, heads].float().cpu().numpy()))
        if out["decode"]:
            o = out["decode_out"]
            for j, (sid, L) in enumerate(out["decode"]):
                if sid in samples:
                    samples[sid].append((L - 1, wl.queries(sid, L - 1, L)[0], o[j, heads].float().cpu().numpy()))
        done_rounds += 1
        if last:
            break
    assert done_rounds == len(rounds)
    # req_to_token rows of every session, bit-exact against the model's slots
    tab = cache.r2t.cpu().numpy()
    for sid, st in enumerate(rows):
        want = np.array(model_slots[sid], np.int32)
        assert len(st.slots) == len(want) == int(hist[sid]) + st_decoded(runner, sid)
        np.testing.assert_array_equal(tab[st.row, :len(want)], want)
        np.testing.assert_array_equal(st.slots, want)

    worst = 0.0
    n_rows = 0
    for sid, smp in samples.items():
        top = max(p for p, _, _ in smp) + 1
        K, V = wl.kv(sid, 0, top)
        pos = np.array([p for p, _, _ in smp])
        Q = np.stack([q for _, q, _ in smp])
        O, _, _, _ = oracle.attention([K], [V], np.zeros(len(pos)), pos, Q, s.Hq, s.Hkv, heads=heads)
        got = np.stack([g for _, _, g in smp])
        worst = max(worst, float(np.max(np.abs(got - O))))
        n_rows += len(pos)
    return worst, n_rows, len(rounds)


def test_multiturn_small_all_sessions_checked():
    wl = W.multiturn(seed=1, n_sessions=12, median=900, h_max=3000, num_slots=1 << 16)
    worst, n_rows, n_rounds = run_multiturn(wl, check_sessions=range(12))
    print(f"multiturn small: {n_rounds} rounds, {n_rows} sampled rows x 8 heads, max abs err {worst:.3e}",
          flush=True)
    assert worst <= BF16_TOL


def test_multiturn_full_size_sampled():
    wl = W.multiturn(seed=0)
    worst, n_rows, n_rounds = run_multiturn(wl, check_sessions=range(wl.n))
    print(f"multiturn full: {wl.n} sessions, hist median {int(np.median(wl.hist))} max {int(wl.hist.max())}, "
          f"hit {wl.cached.sum() / wl.hist.sum():.3f}, {n_rounds} rounds; req_to_token rows of all sessions "
          f"bit-exact; sampled {n_rows} rows x 8 heads of all sessions, max abs err {worst:.3e}", flush=True)
    assert worst <= BF16_TOL
