#!/usr/bin/env python3
"""Benchmark of the paged prefix-shared attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config extend|decode|fork|multiturn]
                    [--no-cpu-baseline]

Default workload ("extend"): 64 requests share a cached 2048-token prefix and
each adds 256 new causal tokens (32 query / 8 KV heads, head_dim 128, bf16,
2^20-slot pool, page size 1), then decodes one token.  One step is one pass
of the whole path over one batch:
  a1/a2  host: batched longest-prefix match + lock, slot allocation
  a3     GPU: req_to_token rows (prefix slots + new slots)
  a4     GPU: store the new tokens' K/V into the pool
  a5     GPU: extend attention (bf16 MFMA)
  a2     host: insert the requests into the radix tree (prefill complete)
  a7     GPU: cascade decode of one token per request (shared prefix read
         once for the group), with its K/V store and req_to_token append
  host:  unlock, free the decode slots, LRU-evict the requests' suffixes.
Host work of a step overlaps the GPU work of the previous one (pinned
staging buffers, asynchronous copies).  Inputs (Q/K/V) are resident in HBM
before the timed region.  Prints ONE JSON line.

Other --config values time the decode-batch, fork-sweep and multi-turn
workloads for reporting; their lines have the same shape.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="extend", choices=["extend", "decode", "fork", "multiturn"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    return ap.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "prefix_shared_paged_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel):
    """HBM bytes per launch measured with rocprofv3 --pmc (profiles/traffic.json),
    valid only for the kernel sources it was measured on."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


class Pinned:
    """Ring of pinned host staging buffers, reused only after their copies finished."""

    def __init__(self, torch, n_slots, sizes):
        self.torch = torch
        self.bufs = [{k: torch.empty(n, dtype=dt, pin_memory=True) for k, (n, dt) in sizes.items()}
                     for _ in range(n_slots)]
        self.events = [None] * n_slots
        self.i = 0

    def next(self):
        i = self.i
        self.i = (self.i + 1) % len(self.bufs)
        if self.events[i] is not None:
            self.events[i].synchronize()
        return i, self.bufs[i]

    def done(self, i):
        ev = self.torch.cuda.Event()
        ev.record()
        self.events[i] = ev


# ---------------------------------------------------------------------------
# default workload: extend over a shared cached prefix + one cascade decode token
# ---------------------------------------------------------------------------
def bench_extend(args):
    import torch
    import workloads as W
    import prefix_shared_paged_amd as sp
    from prefix_shared_paged_amd import accounting as acc
    from prefix_shared_paged_amd.paged_cache import PagedKVCache

    wl = W.extend(seed=0)
    s = wl.spec
    B, P, E = wl.B, int(wl.prefix_len[0]), 256
    Hq, Hkv, D = s.Hq, s.Hkv, s.D
    dev = "cuda"
    bf = torch.bfloat16
    cache = PagedKVCache(s.num_slots, 1, Hkv, D, bf, B + 1, P + E + 1, W.pool_order(s), dev)
    # the shared prefix: computed once earlier, now cached
    pre_tok = wl.prefix_tokens(0)
    [st] = cache.admit([pre_tok])
    cache.append([st], [P])
    Kp, Vp = wl.prefix_kv(0)
    cache.store(torch.from_numpy(Kp).to(dev).to(bf), torch.from_numpy(Vp).to(dev).to(bf), st.slots)
    cache.insert(st)
    cache.release(st)
    tree, pool = cache.tree, cache.pool

    # resident inputs (same values every step; the work is redone in full)
    q_ext = torch.from_numpy(np.concatenate([wl.queries(r, E) for r in range(B)])).to(dev).to(bf)
    kv = [wl.suffix_kv(r, E + 1) for r in range(B)]
    k_ext = torch.from_numpy(np.concatenate([k[:E] for k, _ in kv])).to(dev).to(bf)
    v_ext = torch.from_numpy(np.concatenate([v[:E] for _, v in kv])).to(dev).to(bf)
    k_dec = torch.from_numpy(np.stack([k[E] for k, _ in kv])).to(dev).to(bf)
    v_dec = torch.from_numpy(np.stack([v[E] for _, v in kv])).to(dev).to(bf)
    q_dec = torch.from_numpy(np.stack([wl.queries(r, 1, step=1)[0] for r in range(B)])).to(dev).to(bf)
    del kv
    o_ext = torch.empty_like(q_ext)
    o_dec = torch.empty_like(q_dec)
    rows = torch.arange(B, dtype=torch.int32, device=dev)
    prefix_lens = torch.full((B,), P, dtype=torch.int32, device=dev)
    q_off = torch.arange(0, (B + 1) * E, E, dtype=torch.int64, device=dev)
    seq_lens = torch.full((B,), P + E + 1, dtype=torch.int32, device=dev)
    gptr = torch.tensor([0, B], dtype=torch.int32, device=dev)
    gpl = torch.tensor([P], dtype=torch.int32, device=dev)
    ws = torch.empty(sp.cascade_workspace_size(B, 1, P + E + 1, B, P, Hq, Hkv, D), dtype=torch.uint8,
                     device=dev)
    d_prefix = torch.empty(B * P, dtype=torch.int32, device=dev)
    d_poff = torch.arange(0, (B + 1) * P, P, dtype=torch.int64, device=dev)
    d_new = torch.empty(B * (E + 1), dtype=torch.int32, device=dev)
    d_noff = torch.arange(0, (B + 1) * (E + 1), E + 1, dtype=torch.int64, device=dev)
    d_store = torch.empty(B * E, dtype=torch.int32, device=dev)
    pin = Pinned(torch, 3, {"prefix": (B * P, torch.int32), "new": (B * (E + 1), torch.int32),
                            "store": (B * E, torch.int32)})
    stream = torch.cuda.current_stream()
    ev_ext = []

    def tokens_of(step):
        toks = [np.concatenate([pre_tok, W.tokens(s, W.T_TOK_SUFFIX, E, W.SIBLING_BASE + r, r, step)])
                for r in range(B)]
        off = np.arange(0, (B + 1) * (P + E), P + E, dtype=np.int64)
        return np.concatenate(toks).astype(np.int32), off

    step_tokens = {}

    def step(i, timed):
        if i not in step_tokens:
            step_tokens[i] = tokens_of(i)
        flat, off = step_tokens[i]
        # a2: match + lock;  a1: allocate E + 1 slots per request
        mslots, lens, nodes = tree.match_batch(flat, off, lock=True)
        assert int(lens.min()) == P and int(lens.max()) == P
        last = mslots[off[:-1] + P - 1]
        new, noff = pool.alloc_batch(np.full(B, E + 1, np.int64), lens, last)
        new2 = new.reshape(B, E + 1)
        k, buf = pin.next()
        buf["prefix"].numpy().reshape(B, P)[:] = mslots.reshape(B, P + E)[:, :P]
        buf["new"].numpy()[:] = new
        buf["store"].numpy().reshape(B, E)[:] = new2[:, :E]
        d_prefix.copy_(buf["prefix"], non_blocking=True)
        d_new.copy_(buf["new"], non_blocking=True)
        d_store.copy_(buf["store"], non_blocking=True)
        pin.done(k)
        # a3: req_to_token rows (prefix || E + 1 new slots)
        sp.build_req_to_token(cache.r2t, rows, d_new, d_noff, prefix_slots=d_prefix, prefix_off=d_poff)
        # a4: store the new tokens' K/V
        sp.store_kv(k_ext, v_ext, d_store, cache.k_pool, cache.v_pool)
        # a5: extend attention
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        sp.extend_attn(q_ext, cache.k_pool, cache.v_pool, cache.r2t, rows, prefix_lens, q_off, E, o=o_ext)
        if timed:
            e1.record()
            ev_ext.append((e0, e1))
        # a2: prefill complete -> insert (prefix + E tokens) into the tree
        ins_slots = np.concatenate([mslots.reshape(B, P + E)[:, :P], new2[:, :E]], axis=1).reshape(-1)
        tree.insert_batch(flat, ins_slots, off, pool)
        # a7: one decode token per request, cascade over the shared prefix (stores its K/V first)
        sp.cascade_decode_attn(q_dec, cache.k_pool, cache.v_pool, cache.r2t, rows, seq_lens, gptr, gpl,
                               P + E + 1, B, P, k_new=k_dec, v_new=v_dec, o=o_dec, workspace=ws)
        # release: unlock, free decode slots, evict this step's suffixes (LRU leaves)
        tree.lock_batch(nodes, -1)
        pool.free(new2[:, E])
        freed = tree.evict(B * E, pool)
        assert freed == B * E

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    ext_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_ext]))

    # decode-only timings (flat vs cascade) on the same state, outside the step
    def time_call(fn, n=20):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    # leave one admitted batch in place for the decode-only timings
    flat, off = tokens_of(10 ** 6)
    mslots, lens, nodes = tree.match_batch(flat, off, lock=True)
    new, _ = pool.alloc_batch(np.full(B, E + 1, np.int64), lens, mslots[off[:-1] + P - 1])
    d_prefix.copy_(torch.from_numpy(mslots.reshape(B, P + E)[:, :P].reshape(-1).copy()))
    d_new.copy_(torch.from_numpy(new))
    sp.build_req_to_token(cache.r2t, rows, d_new, d_noff, prefix_slots=d_prefix, prefix_off=d_poff)
    dws = torch.empty(sp.decode_workspace_size(B, P + E + 1, Hq, Hkv, D), dtype=torch.uint8, device=dev)
    flat_ms = time_call(lambda: sp.decode_attn(q_dec, cache.k_pool, cache.v_pool, cache.r2t, rows, seq_lens,
                                               P + E + 1, o=o_dec, workspace=dws))
    casc_ms = time_call(lambda: sp.cascade_decode_attn(q_dec, cache.k_pool, cache.v_pool, cache.r2t, rows,
                                                       seq_lens, gptr, gpl, P + E + 1, B, P, o=o_dec,
                                                       workspace=ws))

    flops = acc.extend_flops([P] * B, [E] * B, Hq, D)
    tflops = flops / (ext_ms * 1e-3) / 1e12
    elt = 2
    L = [P + E + 1] * B
    flat_bytes = acc.decode_bytes_flat(L, Hq, Hkv, D, elt)
    casc_bytes = acc.decode_bytes_cascade(L, [0] * B, [P], Hq, Hkv, D, elt)
    tokens_per_step = B * E + B
    traffic = traffic_record("extend_bf16_kernel")
    line = {
        "metric": "decode attn tokens/s + HBM GB/s; extend attn TFLOP/s (frac of roofline)",
        "value": tokens_per_step / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "extend: 64 requests x 256 new causal tokens over a cached shared 2048-token "
                               "prefix, then 1 cascade-decode token each; 32/8 heads, head_dim 128, "
                               "2^20-slot pool, page 1",
                   "batch": B, "prefix": P, "new_tokens": E, "Hq": Hq, "Hkv": Hkv, "head_dim": D},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "extend_bf16_kernel", "flops_per_launch": flops, "avg_launch_ms": ext_ms},
        "extend_tflops": tflops,
        "decode": {"flat_ms": flat_ms, "cascade_ms": casc_ms,
                   "flat_hbm_gbps": flat_bytes / (flat_ms * 1e-3) / 1e9,
                   "cascade_hbm_gbps": casc_bytes / (casc_ms * 1e-3) / 1e9,
                   "cascade_tokens_per_s": B / (casc_ms * 1e-3),
                   "flat_algorithmic_bytes": flat_bytes, "cascade_algorithmic_bytes": casc_bytes},
    }
    return line, ("extend", wl, P, E)


def cpu_baseline_extend(wl, P, E, target_s):
    """Time the oracle (fp64 C, all host threads) on a bounded sample of the same
    workload: all 256 extend rows (32 heads each) of the first n requests, n
    chosen from a one-request calibration to take about target_s seconds."""
    import oracle
    import workloads as W
    s = wl.spec
    Kp, Vp = wl.prefix_kv(0)

    def run(n_req):
        Ks, Vs, rr, pos, Q = [], [], [], [], []
        for r in range(n_req):
            ks, vs = wl.suffix_kv(r, E + 1)
            Ks.append(np.concatenate([Kp, ks[:E]]))
            Vs.append(np.concatenate([Vp, vs[:E]]))
            rr += [r] * E
            pos += list(range(P, P + E))
            Q.append(wl.queries(r, E))
        Q = np.concatenate(Q)
        t0 = time.perf_counter()
        oracle.attention(Ks, Vs, rr, pos, Q, s.Hq, s.Hkv)
        return time.perf_counter() - t0

    t1 = run(1)
    n = int(max(1, min(wl.B, round(target_s / max(t1, 1e-3)))))
    t = run(n) if n > 1 else t1
    return {"value": n * E / t, "unit": "tokens/s", "cores": oracle.default_threads(), "kind": "oracle",
            "sample": f"extend rows of the first {n} of 64 requests ({n * E} query tokens x 32 heads over "
                      f"{P}+i keys), fp64 oracle, {t:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); multi-GPU runs are not part "
              "of this build", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X); none is visible", file=sys.stderr)
        sys.exit(1)
    if args.config == "extend":
        line, ctx = bench_extend(args)
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_extend(ctx[1], ctx[2], ctx[3], args.cpu_seconds)
        else:
            line["cpu_baseline"] = None
    else:
        from prefix_shared_paged_amd import benchmarks
        line = benchmarks.run(args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
