#!/usr/bin/env python3
"""Benchmark of the paged prefix-shared attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--config extend|tiny|decode|fork|verify|mla|hicache|multiturn]
                    [--kv bf16|fp8] [--no-cpu-baseline]

Default ("extend"): one JSON line carrying both halves of the metric from one
run.
  * The extend workload, timed step by step: 64 requests share a cached
    2048-token prefix and each adds 256 new causal tokens (32 query / 8 KV
    heads, head_dim 128, bf16, 2^20-slot pool, page size 1), then decodes
    one token.  One step is one pass of the whole path over one batch:
      a1/a2  host: batched longest-prefix match + lock, slot allocation
      a3     GPU: req_to_token rows (prefix slots + new slots)
      a4     GPU: store the new tokens' K/V into the pool
      a5     GPU: extend attention (bf16 MFMA)
      a2     host: insert the requests into the radix tree (prefill complete)
      a7     GPU: cascade decode of one token per request (shared prefix read
             once for the group), with its K/V store and req_to_token append
      host:  unlock, free the decode slots, LRU-evict the requests' suffixes.
    Host work of a step overlaps the GPU work of the previous one (pinned
    staging buffers, asynchronous copies).  `value` is the step's query
    tokens per second; `roofline` is the extend kernel (bf16 MFMA).
  * The decode batch (256 requests in 16 prefix groups, contexts up to 8192,
    2^21-slot pool): flat and cascade decode calls, each with its own HBM
    roofline ("decode_batch").
  * The parallel-sampling fork sweep (16 prompts of 4096 tokens x 8
    branches, suffixes 1..512, cascade decode per step): its aggregate HBM
    roofline ("fork_sweep").
Before every timed call a 512 MiB scratch buffer is read and written (twice
the 256 MB Infinity Cache, far beyond the L2s), outside the call's events:
it stands in for the model's other layers between two calls of this layer,
so no call finds the previous repetition's data in a cache.  Inputs (Q/K/V)
are resident in HBM before the timed region.

Other --config values print one line each: tiny (the fp32 4-request
extend + decode, hipEvent medians of >= 50 calls and the full oracle),
decode, fork, verify (small-q extend: q_len new tokens per request over long
cached contexts), mla (latent decode: one 576-dim latent row per token shared
by every query head), hicache (KV rows moved between a page-locked host tier
and the pool) and multiturn (chunked prefill interleaved with decode, page
16; extend and decode calls timed separately and summed over the rounds).
--kv fp8 runs the decode and fork workloads over an FP8 (e4m3fn) KV cache
with per-head factors (the same bf16 queries, bf16 MFMA arithmetic, one byte
per cached element).
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
PEAK_HOST_LINK_GBPS = 63.0     # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes, 128b/130b
PEAK_F32_VALU_TFLOPS = 157.3   # MI355X fp32 vector (256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (dual) x 2.4 GHz)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="extend",
                    choices=["extend", "tiny", "decode", "fork", "verify", "mla", "hicache", "multiturn"])
    ap.add_argument("--mla-heads", type=int, default=128, help="query heads of the mla workload")
    ap.add_argument("--q-len", type=int, default=4, help="new tokens per request of the verify workload")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"],
                    help="KV cache element type of the decode and fork workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (scales HBM counters)")
    ap.add_argument("--no-decode", action="store_true",
                    help="default config: leave out the decode-batch and fork-sweep parts")
    return ap.parse_args()


# the sources each traffic record depends on (a change to any of them makes
# the record stale)
DECODE_SOURCES = ["kernels_decode.hip", "kernels_decode_rows.hip", "decode_rows.h", "decode_util.h",
                  "store_util.h", "kernels_misc.hip", "api.hip", "common.h"]
KERNEL_SOURCES = {
    "extend_bf16_kernel": ["kernels_extend.hip", "common.h"],
    "cascade_decode_call": DECODE_SOURCES,
    "cascade_decode_call_fp8": DECODE_SOURCES,
    "flat_decode_call": DECODE_SOURCES,
    "flat_decode_call_fp8": DECODE_SOURCES,
}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "prefix_shared_paged_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
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
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


class Pinned:
    """Ring of page-locked staging blocks for the slot lists a step sends to
    the device.  Each ring slot is one block holding every array (int32), so a
    step's lists go in a single copy on the compute stream; a host block is
    refilled only after its copy has finished.  (A copy stream of its own was
    tried: the cross-stream event waits cost more per step than they hid.)"""

    def __init__(self, torch, n_slots, sizes, dev):
        self.torch = torch
        self.offs, total = {}, 0
        for k, (n, dt) in sizes.items():
            assert dt == torch.int32
            self.offs[k] = (total, n)
            total += n
        self.blocks = [torch.empty(total, dtype=torch.int32, pin_memory=True) for _ in range(n_slots)]
        self.bufs = [{k: b[o:o + n] for k, (o, n) in self.offs.items()} for b in self.blocks]
        self.dblocks = [torch.empty(total, dtype=torch.int32, device=dev) for _ in range(n_slots)]
        self.copied = [None] * n_slots
        self.i = 0

    def next(self):
        i = self.i
        self.i = (self.i + 1) % len(self.bufs)
        if self.copied[i] is not None:
            self.copied[i].synchronize()
        return i, self.bufs[i]

    def send(self, i):
        """Copy slot i to its device block; returns the device views of its arrays."""
        d = self.dblocks[i]
        d.copy_(self.blocks[i], non_blocking=True)
        ev = self.torch.cuda.Event()
        ev.record()
        self.copied[i] = ev
        return {k: d[o:o + n] for k, (o, n) in self.offs.items()}


class MallFlush:
    """Reads and writes a 512 MiB scratch buffer on the launch stream (twice
    the 256 MB Infinity Cache, far beyond the 4 MB L2 of each XCD), so the
    next call finds none of the previous repetition's data in a cache.  Runs
    before every timed call, outside its events; it stands in for the other
    layers of a model that run between two calls of one layer."""
    MIB = 512

    def __init__(self, torch, dev):
        self.torch = torch
        self.buf = torch.zeros(self.MIB << 18, dtype=torch.int32, device=dev)

    def __call__(self):
        self.buf.add_(1)

    def time_ms(self, n=10):
        t = time_events(self, n)
        return float(np.median(t))


def hbm_roofline(byts, ms, kernel, traffic=None, **extra):
    """Roofline object of an HBM-bound call: algorithmic bytes / time against
    8 TB/s; with a counter record (traffic, HBM bytes per launch) also the
    measured HBM rate."""
    gbps = byts / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
            "traffic": traffic, "kernel": kernel, "bytes_per_launch": byts, "avg_launch_ms": ms}
    if traffic:
        roof["hbm_counter_gbps"] = traffic / (ms * 1e-3) / 1e9
        roof["hbm_counter_frac"] = roof["hbm_counter_gbps"] / PEAK_HBM_GBPS
    roof.update(extra)
    return roof


# ---------------------------------------------------------------------------
# default workload: extend over a shared cached prefix + one cascade decode token
# ---------------------------------------------------------------------------
def bench_extend(args, flush):
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
    d_poff = torch.arange(0, (B + 1) * P, P, dtype=torch.int64, device=dev)
    d_noff = torch.arange(0, (B + 1) * (E + 1), E + 1, dtype=torch.int64, device=dev)
    pin = Pinned(torch, 3, {"prefix": (B * P, torch.int32), "new": (B * (E + 1), torch.int32),
                            "store": (B * E, torch.int32)}, dev)
    ev_ext = []

    def tokens_of(step):
        toks = [np.concatenate([pre_tok, W.tokens(s, W.T_TOK_SUFFIX, E, W.SIBLING_BASE + r, r, step)])
                for r in range(B)]
        off = np.arange(0, (B + 1) * (P + E), P + E, dtype=np.int64)
        return np.concatenate(toks).astype(np.int32), off

    # every step's request tokens (the workload's input) exist before timing starts
    step_tokens = [tokens_of(i) for i in range(args.warmup + args.steps)]

    def step(i, timed):
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
        dv = pin.send(k)
        # a3: req_to_token rows (prefix || E + 1 new slots)
        sp.build_req_to_token(cache.r2t, rows, dv["new"], d_noff, prefix_slots=dv["prefix"], prefix_off=d_poff)
        # a4: store the new tokens' K/V
        sp.store_kv(k_ext, v_ext, dv["store"], cache.k_pool, cache.v_pool)
        # a5: extend attention (caches flushed first, outside its events)
        flush()
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        sp.extend_attn(q_ext, cache.k_pool, cache.v_pool, cache.r2t, rows, prefix_lens, q_off, E, o=o_ext)
        if timed:
            e1.record()
            ev_ext.append((e0, e1))
        # a2: prefill complete -> insert (prefix + E tokens) into the tree; the
        # matched CSR already holds the prefix slots, the new ones go behind them
        mslots.reshape(B, P + E)[:, P:] = new2[:, :E]
        tree.insert_batch(flat, mslots, off, pool)
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
    ext_ms, ext_stalls = event_mean_ms(ev_ext)
    ext_med = float(np.median([a.elapsed_time(b) for a, b in ev_ext]))

    flops = acc.extend_flops([P] * B, [E] * B, Hq, D)
    tflops = flops / (ext_ms * 1e-3) / 1e12
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
                     "kernel": "extend_bf16_kernel", "flops_per_launch": flops, "avg_launch_ms": ext_ms,
                     "median_launch_ms": ext_med, "host_stalled_launches_excluded": ext_stalls},
        "extend_tflops": tflops,
        "mall_flush_ms": flush.time_ms(),
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



# ---------------------------------------------------------------------------
# shared helpers for the other workloads
# ---------------------------------------------------------------------------
def fill_random(t, scale=0.5, seed=0, chunk=1 << 26):
    """Fill a bf16 device tensor with N(0,1)*scale values (device RNG, in chunks)."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    flat = t.view(-1)
    for i in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - i)
        flat[i:i + n] = (torch.randn(n, generator=g, device=t.device) * scale).to(t.dtype)


def fill_fp8(cache, seed, scale=0.5, chunk=1 << 18):
    """Fill an FP8 cache's code pools by quantising N(0,1)*scale bf16 rows
    through the library's store (device RNG, in chunks of slots)."""
    import torch
    import prefix_shared_paged_amd as sp
    g = torch.Generator(device=cache.k_pool.device)
    g.manual_seed(seed)
    S, Hkv, D = cache.k_pool.shape
    for i in range(0, S, chunk):
        n = min(chunk, S - i)
        k = (torch.randn((n, Hkv, D), generator=g, device=cache.k_pool.device) * scale).to(torch.bfloat16)
        v = (torch.randn((n, Hkv, D), generator=g, device=cache.k_pool.device) * scale).to(torch.bfloat16)
        sl = torch.arange(i, i + n, dtype=torch.int32, device=cache.k_pool.device)
        sp.store_kv_fp8(k, v, sl, cache.k_pool, cache.v_pool, cache.k_scale, cache.v_scale)
    torch.cuda.synchronize()


def kv_args(cache):
    """Pool arguments of the decode calls (pools, plus the factors of an FP8 cache)."""
    return (cache.k_pool, cache.v_pool, cache.k_scale, cache.v_scale) if cache.fp8 else (cache.k_pool, cache.v_pool)


def cpu_baseline_rows(K_list, V_list, rows, Hq, Hkv, target_s, what, kv_scale=None):
    """Time the oracle on query rows (req, pos, q) of given logical sequences; the
    sample grows from a calibration run to take about target_s seconds.  With
    kv_scale (FP8 cache factors) the oracle quantises K/V first (untimed) and
    attends over the dequantised values."""
    import oracle
    import oracle.fp8 as F8
    rows = list(rows)
    if kv_scale is not None:
        K_list = [F8.decode(F8.quantize(K, kv_scale[0])).astype(np.float32) for K in K_list]
        V_list = [F8.decode(F8.quantize(V, kv_scale[1])).astype(np.float32) for V in V_list]

    def run(k):
        sub = rows[:k]
        t0 = time.perf_counter()
        oracle.attention(K_list, V_list, [r for r, _, _ in sub], [p for _, p, _ in sub],
                         np.stack([q for _, _, q in sub]), Hq, Hkv, kv_scale=kv_scale)
        return time.perf_counter() - t0

    k = max(1, min(len(rows), 8))
    t = run(k)
    k2 = int(min(len(rows), max(k, k * target_s / max(t, 1e-3))))
    if k2 > k:
        k, t = k2, run(k2)
    return {"value": k / t, "unit": "tokens/s", "cores": __import__("oracle").default_threads(),
            "kind": "oracle", "sample": f"{k} {what} query tokens (all {Hq} heads), fp64 oracle, {t:.1f} s"}


def setup_groups(cache, wl, store_prefix=False):
    """Insert each group's prefix into the tree (its K/V are whatever the pool holds)."""
    for g in range(wl.G):
        toks = wl.prefix_tokens(g)
        [st] = cache.admit([toks])
        cache.append([st], [len(toks)])
        cache.insert(st)
        cache.release(st)


def event_mean_ms(ev):
    """Mean HIP-event time of the timed calls (pairs recorded around each call
    on its stream).  When the host stalls between recording the first event
    and launching the call, the GPU idles and the pair measures the stall; a
    call timed at more than 4x the median is such a case: it is left out of
    the mean and counted (second result)."""
    t = np.array([a.elapsed_time(b) for a, b in ev], np.float64)
    keep = t <= 4.0 * float(np.median(t))
    return float(t[keep].mean()), int((~keep).sum())


def time_events(fn, n, warm=3):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def box_peaks():
    """The chip's sustained ceilings, measured in the same process with the
    library's probes (sgl_probe.h): the dense bf16 MFMA rate (2,048
    workgroups x 4 waves x 2,048 rounds of 8 independent 32x32x16 MFMAs) and
    the streaming copy bandwidth (1 GiB read and written once, bytes moved =
    read + written); medians of 5 event-timed launches after 3 untimed.  The
    probe's output is checked against its closed form, so the work was done."""
    import torch
    import prefix_shared_paged_amd as sp
    out = torch.empty(2048 * sp.PROBE_THREADS, dtype=torch.float32, device="cuda")
    iters = 2048
    flop = sp.probe_mfma_bf16(out, iters)
    t_mfma = float(np.median(time_events(lambda: sp.probe_mfma_bf16(out, iters), 5)))
    ok = bool((out == 8 * 16 * iters).all().item())
    del out
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    moved = sp.probe_copy(src, dst)
    t_copy = float(np.median(time_events(lambda: sp.probe_copy(src, dst), 5)))
    ok = ok and bool(torch.equal(src[:1 << 20], dst[:1 << 20]))
    del src, dst
    torch.cuda.empty_cache()
    tflops = flop / (t_mfma * 1e-3) / 1e12
    gbps = moved / (t_copy * 1e-3) / 1e9
    return {"mfma_bf16_tflops": tflops, "mfma_frac_of_peak": tflops / PEAK_BF16_TFLOPS,
            "copy_gbps": gbps, "copy_frac_of_peak": gbps / PEAK_HBM_GBPS, "probe_ms": [t_mfma, t_copy],
            "checked": ok}


def with_box(roof, box):
    """A roofline object with its fraction of the box's measured ceiling."""
    if not roof or not box:
        return roof
    meas = box["mfma_bf16_tflops"] if roof.get("unit") == "TFLOP/s" else box["copy_gbps"] if roof.get(
        "unit") == "GB/s" and roof.get("bound") == "hbm" else None
    if meas:
        roof["box_peak"] = meas
        roof["frac_of_box_peak"] = roof["achieved"] / meas
    return roof


def base_line(metric_value, ms, args, config, roofline, extra):
    line = {"metric": "decode attn tokens/s + HBM GB/s; extend attn TFLOP/s (frac of roofline)",
            "value": metric_value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": config,
            "roofline": roofline}
    line.update(extra)
    return line


# ---------------------------------------------------------------------------
# decode batch: 256 requests in 16 prefix groups, one token each (flat and cascade)
# ---------------------------------------------------------------------------
def measure_decode(args, flush, fp8=False):
    """The 256-request decode batch, flat and cascade: per-call HIP events
    (caches flushed before each call, outside its events) and each call's HBM
    roofline.  Returns (result dict, workload)."""
    import torch
    import workloads as W
    import prefix_shared_paged_amd as sp
    from prefix_shared_paged_amd import accounting as acc
    from prefix_shared_paged_amd.paged_cache import PagedKVCache

    wl = W.decode(seed=0)
    s = wl.spec
    B, G, Hq, Hkv, D = wl.B, wl.G, s.Hq, s.Hkv, s.D
    dev = "cuda"
    L = wl.ctx_len.astype(np.int64)
    P = wl.prefix_len[wl.grp].astype(np.int64)
    cache = PagedKVCache(s.num_slots, 1, Hkv, D, torch.bfloat16, B + G, int(L.max()) + 1, W.pool_order(s), dev,
                         kv_scale=W.fp8_scales(s) if fp8 else None)
    if fp8:
        fill_fp8(cache, seed=1)
    else:
        fill_random(cache.k_pool, seed=1)
        fill_random(cache.v_pool, seed=2)
    setup_groups(cache, wl)
    toks = [np.concatenate([wl.prefix_tokens(wl.grp[r]), wl.suffix_tokens(r)]) for r in range(B)]
    rows = cache.admit(toks)
    assert all(st.matched == P[r] for r, st in enumerate(rows))
    cache.append(rows, (L - P - 1).tolist())          # cached history of each suffix
    q = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    kn = torch.empty((B, Hkv, D), dtype=torch.bfloat16, device=dev)
    vn = torch.empty((B, Hkv, D), dtype=torch.bfloat16, device=dev)
    for t, sd in ((q, 3), (kn, 4), (vn, 5)):
        fill_random(t, seed=sd)
    o = torch.empty_like(q)
    req_rows = cache.rows_tensor(rows)
    seq = torch.from_numpy(L.astype(np.int32)).to(dev)
    col0 = torch.from_numpy((L - 1).astype(np.int32)).to(dev)
    gptr = torch.from_numpy(np.concatenate([[0], np.cumsum(np.bincount(wl.grp, minlength=G))]).astype(np.int32)).to(dev)
    gpl = torch.from_numpy(wl.prefix_len.astype(np.int32)).to(dev)
    ws_f = torch.empty(sp.decode_workspace_size(B, int(L.max()), Hq, Hkv, D), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(sp.cascade_workspace_size(B, G, int(L.max()), 16, int(wl.prefix_len.max()), Hq, Hkv, D),
                       dtype=torch.uint8, device=dev)
    d_noff = torch.arange(B + 1, dtype=torch.int64, device=dev)
    pin = Pinned(torch, 3, {"new": (B, torch.int32)}, dev)
    pool = cache.pool
    last = np.array([int(st.slots[-1]) for st in rows], np.int32)
    ev = []

    def step(cascade, timed):
        # a1: one slot per request for the current token;  a3: append it to req_to_token
        new, _ = pool.alloc_batch(np.ones(B, np.int64), L - 1, last)
        k, buf = pin.next()
        buf["new"].numpy()[:] = new
        d_new = pin.send(k)["new"]
        sp.build_req_to_token(cache.r2t, req_rows, d_new, d_noff, new_col0=col0)
        flush()
        if timed:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
        if cascade:   # a4 + a7
            (sp.cascade_decode_attn_fp8kv if fp8 else sp.cascade_decode_attn)(
                q, *kv_args(cache), cache.r2t, req_rows, seq, gptr, gpl, int(L.max()), 16,
                int(wl.prefix_len.max()), k_new=kn, v_new=vn, o=o, workspace=ws_c)
        else:         # a4 + a6
            (sp.decode_attn_fp8kv if fp8 else sp.decode_attn)(
                q, *kv_args(cache), cache.r2t, req_rows, seq, int(L.max()), k_new=kn, v_new=vn, o=o,
                workspace=ws_f)
        if timed:
            b.record()
            ev.append((a, b))
        pool.free(new)

    res = {}
    for mode in ("cascade", "flat"):
        ev.clear()
        for _ in range(args.warmup):
            step(mode == "cascade", False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(mode == "cascade", True)
        torch.cuda.synchronize()
        mean, stalls = event_mean_ms(ev)
        res[mode] = dict(wall_ms_per_step=(time.perf_counter() - t0) * 1e3 / args.steps, call_ms=mean,
                         median_ms=float(np.median([a.elapsed_time(b) for a, b in ev])), stalls=stalls)
    kelt = 1 if fp8 else 2
    sfx = "_fp8" if fp8 else ""
    flat_bytes = acc.decode_bytes_flat(L, Hq, Hkv, D, kelt, 2, stored=B)
    casc_bytes = acc.decode_bytes_cascade(L, wl.grp, wl.prefix_len, Hq, Hkv, D, kelt, 2, stored=B)
    out = {}
    for mode, byts in (("flat", flat_bytes), ("cascade", casc_bytes)):
        r = res[mode]
        kern = ("flat decode call (split kernel + merge)" if mode == "flat"
                else "cascade decode call (prefix + suffix split kernels + merge)")
        roof = hbm_roofline(byts, r["call_ms"], kern, traffic_record(f"{mode}_decode_call{sfx}"),
                            median_launch_ms=r["median_ms"], host_stalled_calls_excluded=r["stalls"])
        out[mode] = {"call_ms": r["call_ms"], "tokens_per_s": B / (r["call_ms"] * 1e-3),
                     "algorithmic_bytes": byts, "roofline": roof, "wall_ms_per_step": r["wall_ms_per_step"]}
    out["flat"]["note"] = ("flat decode counts each request's shared prefix once per request (the method's "
                           "algorithmic bytes); the chip serves repeated prefix rows from L2/MALL, so its HBM "
                           "traffic is hbm_counter_gbps, not achieved")
    out["config"] = {"workload": "decode: 256 requests in 16 prefix groups (prefix ~U[512,4096], context "
                                 "~U[max(1024,P+1),8192]), one token each (stored, then attended); 32/8 heads, "
                                 "head_dim 128, 2^21-slot pool, page 1"
                                 + (", FP8 e4m3fn KV cache with per-head factors" if fp8 else ""),
                     "batch": B, "groups": G, "kv_cache": "fp8_e4m3fn" if fp8 else "bf16"}
    return out, wl


def bench_decode(args, flush):
    import workloads as W
    fp8 = args.kv == "fp8"
    res, wl = measure_decode(args, flush, fp8)
    s = wl.spec
    B, Hq, Hkv = wl.B, s.Hq, s.Hkv
    c = res["cascade"]
    line = base_line(B / (c["call_ms"] * 1e-3), c["call_ms"], args, res["config"], c["roofline"], {
        "flat": res["flat"], "cascade": c, "mall_flush_ms": flush.time_ms()})
    if not args.no_cpu_baseline:
        # oracle sample: decode rows of the requests (as many as the target
        # time takes), drawn by the seeded generator
        L = wl.ctx_len
        Ks, Vs, rws = [], [], []
        for r in range(min(B, 96)):
            K, V = wl.logical_kv(r)
            Ks.append(K)
            Vs.append(V)
            rws.append((r, int(L[r]) - 1, wl.queries(r, 1)[0]))
        line["cpu_baseline"] = cpu_baseline_rows(Ks, Vs, rws, Hq, Hkv, args.cpu_seconds, "decode",
                                                 W.fp8_scales(s) if fp8 else None)
    return line


# ---------------------------------------------------------------------------
# fork: 16 prompts x 4096 tokens, 8 branches each; suffixes grow 1..512 (cascade)
# ---------------------------------------------------------------------------
def measure_fork(args, flush, fp8=False, n_sweeps=1):
    """The fork sweep: per step s = 1..512 one cascade decode call (caches
    flushed before it, outside its events); aggregate = sum of bytes / sum of
    call times over the sweep.  Returns (result dict, workload)."""
    import torch
    import workloads as W
    import prefix_shared_paged_amd as sp
    from prefix_shared_paged_amd import accounting as acc
    from prefix_shared_paged_amd.paged_cache import PagedKVCache

    wl = W.fork(seed=0)
    s = wl.spec
    B, G, Hq, Hkv, D = wl.B, wl.G, s.Hq, s.Hkv, s.D
    Pp, S = 4096, 512
    dev = "cuda"
    cache = PagedKVCache(s.num_slots, 1, Hkv, D, torch.bfloat16, B + G, Pp + S + 1, W.pool_order(s), dev,
                         kv_scale=W.fp8_scales(s) if fp8 else None)
    if fp8:
        fill_fp8(cache, seed=1)
    else:
        fill_random(cache.k_pool, seed=1)
        fill_random(cache.v_pool, seed=2)
    setup_groups(cache, wl)
    rows = cache.admit([np.concatenate([wl.prefix_tokens(wl.grp[r]), wl.suffix_tokens(r, 1)]) for r in range(B)])
    assert all(st.matched == Pp for st in rows)
    q = torch.empty((S, B, Hq, D), dtype=torch.bfloat16, device=dev)     # one query batch per step
    kn = torch.empty((S, B, Hkv, D), dtype=torch.bfloat16, device=dev)
    vn = torch.empty((S, B, Hkv, D), dtype=torch.bfloat16, device=dev)
    for t, sd in ((q, 3), (kn, 4), (vn, 5)):
        fill_random(t, seed=sd)
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    req_rows = cache.rows_tensor(rows)
    gptr = torch.arange(0, B + 1, 8, dtype=torch.int32, device=dev)
    gpl = torch.full((G,), Pp, dtype=torch.int32, device=dev)
    seqs = [torch.full((B,), Pp + k, dtype=torch.int32, device=dev) for k in range(1, S + 1)]
    col0s = [torch.full((B,), Pp + k - 1, dtype=torch.int32, device=dev) for k in range(1, S + 1)]
    ws = torch.empty(sp.cascade_workspace_size(B, G, Pp + S, 8, Pp, Hq, Hkv, D), dtype=torch.uint8, device=dev)
    d_new = torch.empty((S, B), dtype=torch.int32, device=dev)
    d_noff = torch.arange(B + 1, dtype=torch.int64, device=dev)
    pool = cache.pool
    pin = torch.empty((S, B), dtype=torch.int32, pin_memory=True)
    per_s = np.zeros(S)

    def sweep(timed):
        # a1 for the whole sweep up front (host), one upload; then 512 decode rounds
        cur = np.full(B, Pp, np.int64)
        last = np.array([int(st.slots[-1]) for st in rows], np.int32)
        slots = np.empty((S, B), np.int32)
        for k in range(S):
            new, _ = pool.alloc_batch(np.ones(B, np.int64), cur, last)
            slots[k] = new
            cur += 1
            last = new
        pin.numpy()[:] = slots
        d_new.copy_(pin, non_blocking=True)
        evs = []
        for k in range(S):
            sp.build_req_to_token(cache.r2t, req_rows, d_new[k], d_noff, new_col0=col0s[k])
            flush()
            if timed:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
            (sp.cascade_decode_attn_fp8kv if fp8 else sp.cascade_decode_attn)(
                q[k], *kv_args(cache), cache.r2t, req_rows, seqs[k], gptr, gpl, Pp + k + 1, 8, Pp,
                k_new=kn[k], v_new=vn[k], o=o, workspace=ws)
            if timed:
                b.record()
                evs.append((a, b))
        torch.cuda.synchronize()
        pool.free(slots.reshape(-1))
        return evs

    sweep(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_sweeps):
        evs = sweep(True)
        per_s += np.array([a.elapsed_time(b) for a, b in evs])
    wall = (time.perf_counter() - t0) * 1e3 / n_sweeps
    per_s /= n_sweeps
    kelt = 1 if fp8 else 2
    bytes_s = np.array([acc.decode_bytes_cascade([Pp + k] * B, np.repeat(np.arange(G), 8), [Pp] * G, Hq, Hkv, D,
                                                 kelt, 2, stored=B) for k in range(1, S + 1)], np.float64)
    tot_ms = float(per_s.sum())
    roof = hbm_roofline(float(bytes_s.sum()), tot_ms, "cascade decode call, summed over the sweep s = 1..512",
                        None, bytes_per_sweep=float(bytes_s.sum()), avg_call_ms=float(per_s.mean()))
    out = {"sweep_ms": tot_ms, "wall_ms_per_sweep": wall, "tokens_per_s": B * S / (tot_ms * 1e-3),
           "roofline": roof, "sweeps": n_sweeps,
           "per_s_gbps": {str(k): float(bytes_s[k - 1] / (per_s[k - 1] * 1e-3) / 1e9) for k in (1, 2, 64, 256, 512)},
           "per_s_ms": {str(k): float(per_s[k - 1]) for k in (1, 2, 64, 256, 512)},
           "config": {"workload": "fork: 16 prompts x 4096 tokens, 8 branches each (128 requests), suffix grows "
                                  "1..512 in lockstep, cascade decode per step (current token stored, then "
                                  "attended); 32/8 heads, head_dim 128, 2^18-slot pool"
                                  + (", FP8 e4m3fn KV cache with per-head factors" if fp8 else ""),
                      "prompts": G, "branches": 8, "prompt_len": Pp, "steps_per_sweep": S,
                      "kv_cache": "fp8_e4m3fn" if fp8 else "bf16"}}
    return out, wl


def bench_fork(args, flush):
    import workloads as W
    fp8 = args.kv == "fp8"
    n_sweeps = max(1, args.steps // 10)
    res, wl = measure_fork(args, flush, fp8, n_sweeps)
    s = wl.spec
    B, Hq, Hkv = wl.B, s.Hq, s.Hkv
    line = base_line(res["tokens_per_s"], res["sweep_ms"], args, res["config"], res["roofline"], {
        k: v for k, v in res.items() if k not in ("roofline", "config")})
    line["steps"] = n_sweeps
    line["mall_flush_ms"] = flush.time_ms()
    if not args.no_cpu_baseline:
        Ks, Vs, rws = [], [], []
        for r in range(0, B, 4):
            K, V = wl.logical_kv(r, 512)
            Ks.append(K)
            Vs.append(V)
            rws.append((len(Ks) - 1, 4096 + 512 - 1, wl.queries(r, 1)[0]))
        line["cpu_baseline"] = cpu_baseline_rows(Ks, Vs, rws, Hq, Hkv, args.cpu_seconds, "fork (s=512)",
                                                 W.fp8_scales(s) if fp8 else None)
    return line


# ---------------------------------------------------------------------------
# verify: 64 requests, own cached contexts ~U[2048, 8192], q_len new tokens each
# ---------------------------------------------------------------------------
def bench_verify(args, flush):
    import torch
    import workloads as W
    import prefix_shared_paged_amd as sp
    from prefix_shared_paged_amd import accounting as acc
    from prefix_shared_paged_amd.paged_cache import PagedKVCache

    E = args.q_len
    wl = W.verify(seed=0, q_len=E)
    s = wl.spec
    B, Hq, Hkv, D = wl.B, s.Hq, s.Hkv, s.D
    P = wl.prefix_len.astype(np.int64)
    dev = "cuda"
    cache = PagedKVCache(s.num_slots, 1, Hkv, D, torch.bfloat16, 2 * B, int(P.max()) + E + 1, W.pool_order(s), dev)
    fill_random(cache.k_pool, seed=1)
    fill_random(cache.v_pool, seed=2)
    setup_groups(cache, wl)
    rows = cache.admit([wl.prefix_tokens(r) for r in range(B)])
    assert all(st.matched == P[r] for r, st in enumerate(rows))
    n = B * E
    q = torch.empty((n, Hq, D), dtype=torch.bfloat16, device=dev)
    kn = torch.empty((n, Hkv, D), dtype=torch.bfloat16, device=dev)
    vn = torch.empty((n, Hkv, D), dtype=torch.bfloat16, device=dev)
    for t, sd in ((q, 3), (kn, 4), (vn, 5)):
        fill_random(t, seed=sd)
    o = torch.empty_like(q)
    req_rows = cache.rows_tensor(rows)
    pl = torch.from_numpy(P.astype(np.int32)).to(dev)
    q_off = torch.from_numpy(np.arange(B + 1, dtype=np.int64) * E).to(dev)
    col0 = torch.from_numpy(P.astype(np.int32)).to(dev)
    ws_n = sp.extend_workspace_size(B, n, E, cache.r2t.shape[1], Hq, Hkv, D)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev) if ws_n else None
    pin = Pinned(torch, 3, {"new": (n, torch.int32)}, dev)
    pool = cache.pool
    last = np.array([int(st.slots[-1]) for st in rows], np.int32)
    ev = []

    def step(timed):
        # a1: q_len draft slots per request; a3: append them to req_to_token;
        # a4 + a5: store the drafts' K/V and attend (small-q extend); the
        # drafts are then rejected (slots freed) so every step sees the same shapes
        new, _ = pool.alloc_batch(np.full(B, E, np.int64), P, last)
        k, buf = pin.next()
        buf["new"].numpy()[:] = new
        d_new = pin.send(k)["new"]
        sp.build_req_to_token(cache.r2t, req_rows, d_new, q_off, new_col0=col0)
        flush()
        if timed:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
        sp.extend_attn(q, cache.k_pool, cache.v_pool, cache.r2t, req_rows, pl, q_off, E, k_new=kn, v_new=vn,
                       o=o, workspace=ws)
        if timed:
            b.record()
            ev.append((a, b))
        pool.free(new)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    call, stalls = event_mean_ms(ev)
    byts = acc.decode_bytes_flat(P + E, Hq, Hkv, D, 2) + (E - 1) * 2 * B * Hq * D * 2
    gbps = byts / (call * 1e-3) / 1e9
    config = {"workload": f"verify (small-q extend): {B} requests, own cached contexts ~U[2048,8192], {E} new "
                          "tokens each (stored, then attended causally); 32/8 heads, head_dim 128, 2^20-slot pool, "
                          "page 1", "batch": B, "q_len": E,
              "path": ("split-K" if E * (Hq // Hkv) <= 16 else "prefill kernel, key splits") if ws_n
              else "prefill kernel"}
    roof = {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
            "traffic": None, "kernel": "extend call (split kernel + merge, or the prefill kernel)",
            "bytes_per_launch": byts, "avg_launch_ms": call}
    line = base_line(n / (call * 1e-3), call, args, config, roof, {
        "call_ms": call, "wall_ms_per_step": ms, "host_stalled_calls_excluded": stalls,
        "tokens_per_s_call_only": n / (call * 1e-3)})
    if not args.no_cpu_baseline:
        Ks, Vs, rws = [], [], []
        for r in range(min(B, 8)):
            K, V = wl.logical_kv(r)
            Ks.append(K)
            Vs.append(V)
            for i in range(E):
                rws.append((r, int(P[r]) + i, wl.queries(r, E)[i]))
        line["cpu_baseline"] = cpu_baseline_rows(Ks, Vs, rws, Hq, Hkv, args.cpu_seconds, "verify")
    return line


# ---------------------------------------------------------------------------
# mla: latent decode, 128 requests in 16 groups of 8, one 576-dim latent per token
# ---------------------------------------------------------------------------
def bench_mla(args, flush):
    import torch
    import workloads as W
    import prefix_shared_paged_amd as sp

    wl = W.mla(seed=0, Hq=args.mla_heads)
    s = wl.spec
    B, G, Hq, Dqk, Dv = wl.B, wl.G, s.Hq, 576, 512
    M = B // G
    dev = "cuda"
    L = wl.ctx_len.astype(np.int64)
    Pg = wl.prefix_len.astype(np.int64)
    # request r: its group's prefix slots, then its own; the pool is random
    # latents (values do not change the work)
    pool = torch.empty((s.num_slots, Dqk), dtype=torch.bfloat16, device=dev)
    fill_random(pool, seed=1)
    perm = W.pool_order(s)
    stride = int(L.max()) + 1
    r2t_h = np.full((B, stride), -1, np.int32)
    pos = 0
    for g in range(G):
        pre = perm[pos:pos + Pg[g]]
        pos += Pg[g]
        for r in range(g * M, (g + 1) * M):
            n = int(L[r] - Pg[g])
            r2t_h[r, :Pg[g]] = pre
            r2t_h[r, Pg[g]:L[r]] = perm[pos:pos + n]
            pos += n
    r2t = torch.from_numpy(r2t_h).to(dev)
    q = torch.empty((B, Hq, Dqk), dtype=torch.bfloat16, device=dev)
    kvn = torch.empty((B, Dqk), dtype=torch.bfloat16, device=dev)
    fill_random(q, seed=3)
    fill_random(kvn, seed=4)
    o = torch.empty((B, Hq, Dv), dtype=torch.bfloat16, device=dev)
    rows = torch.arange(B, dtype=torch.int32, device=dev)
    seq = torch.from_numpy(L.astype(np.int32)).to(dev)
    gptr = torch.from_numpy((np.arange(G + 1) * M).astype(np.int32)).to(dev)
    gpl = torch.from_numpy(Pg.astype(np.int32)).to(dev)
    ws_f = torch.empty(sp.mla_decode_workspace_size(B, int(L.max()), Hq), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(sp.mla_cascade_workspace_size(B, G, int(L.max()), M, int(Pg.max()), Hq), dtype=torch.uint8,
                       device=dev)
    flat = lambda: sp.mla_decode_attn(q, pool, r2t, rows, seq, int(L.max()), kv_new=kvn, o=o, workspace=ws_f)
    casc = lambda: sp.mla_cascade_decode_attn(q, pool, r2t, rows, seq, gptr, gpl, int(L.max()), M, int(Pg.max()),
                                              kv_new=kvn, o=o, workspace=ws_c)
    res = {}
    for name, fn in (("cascade", casc), ("flat", flat)):
        for _ in range(args.warmup):
            flush()
            fn()
        torch.cuda.synchronize()
        evs = []
        t0 = time.perf_counter()
        for _ in range(args.steps):
            flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        res[name] = ((time.perf_counter() - t0) * 1e3 / args.steps, event_mean_ms(evs)[0])
    row_b = Dqk * 2 + 4                                   # latent + its req_to_token entry
    qo = B * Hq * (Dqk + Dv) * 2
    flat_bytes = int(L.sum()) * row_b + qo
    casc_bytes = (int(Pg.sum()) + int((L - Pg[wl.grp]).sum())) * row_b + qo
    flops = float(L.sum()) * Hq * (Dqk + Dv) * 2
    ms_c, call_c = res["cascade"]
    ms_f, call_f = res["flat"]
    gbps_c = casc_bytes / (call_c * 1e-3) / 1e9
    gbps_f = flat_bytes / (call_f * 1e-3) / 1e9
    config = {"workload": f"mla latent decode: {B} requests in {G} prefix groups of {M} (prefix ~U[512,4096], context "
                          f"~U[max(1024,P+1),8192]), one token each, cascade decode; {Hq} query heads over one "
                          "576-dim latent per token (values: its first 512), 2^21-slot pool, page 1",
              "batch": B, "groups": G, "Hq": Hq, "Dqk": Dqk, "Dv": Dv}
    roof = {"bound": "hbm", "achieved": gbps_c, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps_c / PEAK_HBM_GBPS,
            "traffic": None, "kernel": "mla cascade decode call (prefix + suffix split kernels + merge)",
            "bytes_per_launch": casc_bytes, "avg_launch_ms": call_c}
    line = base_line(B / (call_c * 1e-3), call_c, args, config, roof, {"wall_ms_per_step": ms_c,
        "flat": {"call_ms": call_f, "hbm_gbps": gbps_f, "frac": gbps_f / PEAK_HBM_GBPS,
                 "tflops": flops / (call_f * 1e-3) / 1e12, "algorithmic_bytes": flat_bytes},
        "cascade": {"call_ms": call_c, "hbm_gbps": gbps_c, "algorithmic_bytes": casc_bytes,
                    "tflops": flops / (call_c * 1e-3) / 1e12, "mfma_frac": flops / (call_c * 1e-3) / 1e12 / 2500.0},
        "flops_per_call": flops})
    if not args.no_cpu_baseline:
        import oracle
        q_h = q[:4].float().cpu().numpy()
        kvn_h = kvn[:4].float().cpu().numpy()
        t0 = time.perf_counter()
        for r in range(4):
            lat = pool[torch.from_numpy(r2t_h[r, :L[r] - 1].astype(np.int64)).to(dev)].float().cpu().numpy()
            lat = np.concatenate([lat, kvn_h[r][None]])[:, None, :]
            oracle.attention([lat], [np.ascontiguousarray(lat[:, :, :Dv])], [0], [int(L[r]) - 1], q_h[r][None], Hq, 1,
                             scale=1.0 / np.sqrt(192.0))
        t = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": 4 / t, "unit": "tokens/s", "cores": __import__("oracle").default_threads(),
                                "kind": "oracle", "sample": f"4 decode tokens (all {Hq} heads), fp64 oracle, "
                                                            f"{t:.1f} s including the latent gathers"}
    return line


# ---------------------------------------------------------------------------
# hicache: one layer's K/V rows of 65,536 tokens between a pinned host tier and the pool
# ---------------------------------------------------------------------------
def bench_hicache(args, flush):
    import torch
    import prefix_shared_paged_amd as sp

    Hkv, D, num_slots, n_host, n = 8, 128, 1 << 20, 1 << 18, 65536
    dev = "cuda"
    rng = np.random.default_rng(0)
    pools = [torch.empty((num_slots, Hkv, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    for i, p in enumerate(pools):
        fill_random(p, seed=i + 1)
    hosts = [torch.full((n_host, Hkv, D), 0.25 * (i + 1), dtype=torch.bfloat16, pin_memory=True) for i in range(2)]
    # 32 prefixes of 2048 tokens whose rows are scattered over the host tier
    # and the pool (page size 1)
    slots = torch.from_numpy(rng.permutation(num_slots)[:n].astype(np.int32)).to(dev)
    hrows = torch.from_numpy(rng.permutation(n_host)[:n].astype(np.int64)).to(dev)
    row_bytes = Hkv * D * 2
    moved = 2 * n * row_bytes + n * (4 + 8)               # K and V rows + the two index arrays
    pre = lambda: sp.hicache_prefetch(hosts[0], hosts[1], hrows, slots, pools[0], pools[1])
    wb = lambda: sp.hicache_write_back(pools[0], pools[1], slots, hrows, hosts[0], hosts[1])
    # the host link's practical ceiling: one DMA copy of the same bytes, contiguous
    dma_src = torch.empty(2 * n * row_bytes, dtype=torch.uint8, pin_memory=True)
    dma_dst = torch.empty(2 * n * row_bytes, dtype=torch.uint8, device=dev)
    dma = lambda: dma_dst.copy_(dma_src, non_blocking=True)
    res = {}
    for name, fn in (("prefetch", pre), ("write_back", wb), ("dma_h2d", dma)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs = []
        for _ in range(args.steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        res[name] = ((time.perf_counter() - t0) * 1e3 / args.steps, event_mean_ms(evs)[0])
    ms, call = res["prefetch"]
    gbps = moved / (call * 1e-3) / 1e9
    wb_gbps = moved / (res["write_back"][1] * 1e-3) / 1e9
    dma_gbps = 2 * n * row_bytes / (res["dma_h2d"][1] * 1e-3) / 1e9
    config = {"workload": "hicache prefetch: K and V rows of 65,536 tokens (32 prefixes of 2048) of one layer "
                          "(8 KV heads x 128, bf16: 4 KiB per token) gathered from a 2^18-row page-locked host tier "
                          "into a 2^20-slot pool, rows scattered on both sides (page 1)",
              "tokens": n, "Hkv": Hkv, "D": D}
    roof = {"bound": "host-link", "achieved": gbps, "peak": PEAK_HOST_LINK_GBPS, "unit": "GB/s",
            "frac": gbps / PEAK_HOST_LINK_GBPS, "traffic": None, "kernel": "move_rows_kernel<0> (prefetch)",
            "bytes_per_launch": moved, "avg_launch_ms": call}
    line = base_line(n / (ms * 1e-3), ms, args, config, roof, {
        "write_back": {"call_ms": res["write_back"][1], "gbps": wb_gbps, "frac": wb_gbps / PEAK_HOST_LINK_GBPS},
        "dma_h2d_contiguous": {"call_ms": res["dma_h2d"][1], "gbps": dma_gbps}})
    if not args.no_cpu_baseline:
        from oracle import hicache
        k = 4096
        host_np = hosts[0][:n_host].view(torch.int16).numpy()
        pool_np = np.zeros((8192, Hkv, D), np.int16)
        hr = hrows[:k].cpu().numpy()
        t0 = time.perf_counter()
        reps = 0
        while True:
            hicache.load(pool_np, host_np, hr, np.arange(k))
            hicache.load(pool_np, host_np, hr, np.arange(k))   # the V tier
            reps += 1
            if time.perf_counter() - t0 > min(args.cpu_seconds, 5.0):
                break
        t = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": reps * k / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                "sample": f"{reps} x {k} tokens (K and V rows) gathered by the oracle's row loop "
                                          f"from the pinned host tier into an 8192-row array, {t:.1f} s"}
    return line


# ---------------------------------------------------------------------------
# multi-turn: 128 sessions, ~70% cached history, chunked prefill (512) + decode, page 16
# ---------------------------------------------------------------------------
def bench_multiturn(args, flush):
    import torch
    import workloads as W
    from prefix_shared_paged_amd import accounting as acc
    from prefix_shared_paged_amd.chunked import ChunkedRunner, plan_rounds
    from prefix_shared_paged_amd.paged_cache import PagedKVCache

    wl = W.multiturn(seed=0)
    s = wl.spec
    n, Hq, Hkv, D = wl.n, s.Hq, s.Hkv, s.D
    dev = "cuda"
    rounds = plan_rounds(wl.hist, wl.cached, wl.chunk)
    max_dec = len(rounds)
    toks = [W.tokens(s, W.T_TOK_PREFIX, int(wl.hist[i]) + max_dec, i + 1, i) for i in range(n)]
    stride = int(wl.hist.max()) + max_dec + 16
    # round inputs, resident in HBM before timing
    inp = []
    for ext, dec in rounds:
        ne = sum(hi - lo for _, lo, hi in ext)
        tq = torch.empty((ne, Hq, D), dtype=torch.bfloat16, device=dev)
        tk = torch.empty((ne, Hkv, D), dtype=torch.bfloat16, device=dev)
        tv = torch.empty((ne, Hkv, D), dtype=torch.bfloat16, device=dev)
        dq = torch.empty((len(dec), Hq, D), dtype=torch.bfloat16, device=dev)
        dk = torch.empty((len(dec), Hkv, D), dtype=torch.bfloat16, device=dev)
        dv = torch.empty((len(dec), Hkv, D), dtype=torch.bfloat16, device=dev)
        for j, t in enumerate((tq, tk, tv, dq, dk, dv)):
            if t.numel():
                fill_random(t, seed=100 + j)
        inp.append((tq, tk, tv, dq, dk, dv))
    ext_flops = [sum(acc.extend_flops([lo], [hi - lo], Hq, D) for _, lo, hi in e) for e, _ in rounds]
    dec_bytes = [acc.decode_bytes_flat([p + 1 for _, p in d], Hq, Hkv, D, 2, stored=len(d)) if d else 0
                 for _, d in rounds]

    class Timing:
        """HIP events right around each library call (after a cache flush)."""

        def __init__(self):
            self.ev = {"extend": [], "decode": []}
            self.open = None

        def before(self, kind):
            flush()
            a = torch.cuda.Event(enable_timing=True)
            a.record()
            self.open = a

        def after(self, kind):
            b = torch.cuda.Event(enable_timing=True)
            b.record()
            self.ev[kind].append((self.open, b))

    def run_once(timed):
        cache = PagedKVCache(s.num_slots, s.page_size, Hkv, D, torch.bfloat16, 2 * n, stride, W.pool_order(s), dev)
        if run_once.pools is None:
            fill_random(cache.k_pool, seed=1)
            fill_random(cache.v_pool, seed=2)
            run_once.pools = (cache.k_pool, cache.v_pool)
        else:
            cache.k_pool, cache.v_pool = run_once.pools
        setup = cache.admit([t[:int(c)] for t, c in zip(toks, wl.cached)])
        cache.append(setup, [int(c) for c in wl.cached])
        for st in setup:
            cache.insert(st)
            cache.release(st)
        runner = ChunkedRunner(cache, wl.chunk)
        runner.admit(list(range(n)), toks, wl.hist)
        torch.cuda.synchronize()
        it = iter(inp)
        timing = Timing()
        t0 = time.perf_counter()
        while True:
            last = not runner.pending()
            runner.run_round(lambda ext, dec: next(it), timing=timing)
            if last:
                break
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3, timing

    run_once.pools = None
    run_once(False)
    tot_ms, ext_ms, dec_ms = [], [], []
    for _ in range(max(1, args.steps // 10)):
        ms, tm = run_once(True)
        tot_ms.append(ms)
        ext_ms.append([a.elapsed_time(b) for a, b in tm.ev["extend"]])
        dec_ms.append([a.elapsed_time(b) for a, b in tm.ev["decode"]])
    ms = float(np.mean(tot_ms))
    e_ms = np.mean(np.array(ext_ms), axis=0)          # per extend call, averaged over runs
    d_ms = np.mean(np.array(dec_ms), axis=0)
    n_tokens = sum(hi - lo for e, _ in rounds for _, lo, hi in e) + sum(len(d) for _, d in rounds)
    flops = float(sum(f for f, (e, _) in zip(ext_flops, rounds) if e))
    dbytes = float(sum(b for b, (_, d) in zip(dec_bytes, rounds) if d))
    ext_tflops = flops / (e_ms.sum() * 1e-3) / 1e12
    config = {"workload": "multiturn: 128 sessions, history lognormal(median 3000, sigma 1) clamped to "
                          "[32, 32768], ~70% cached, chunked prefill 512 interleaved with decode, page 16; "
                          "64/8 heads, head_dim 128, 2^20-slot pool", "sessions": n, "rounds": len(rounds)}
    roof = {"bound": "mfma", "achieved": ext_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ext_tflops / PEAK_BF16_TFLOPS, "traffic": None,
            "kernel": "extend calls (chunked prefill), summed over the rounds",
            "flops_per_run": flops, "extend_ms_per_run": float(e_ms.sum()), "extend_calls": int(len(e_ms))}
    line = base_line(n_tokens / (ms * 1e-3), ms, args, config, roof, {
        "decode": {"roofline": hbm_roofline(dbytes, float(d_ms.sum()),
                                            "decode calls (split kernel + merge), summed over the rounds",
                                            None, decode_calls=int(len(d_ms))),
                   "tokens_per_s": sum(len(d) for _, d in rounds) / (d_ms.sum() * 1e-3)},
        "extend_ms_per_call": e_ms.tolist(), "decode_ms_per_call": d_ms.tolist(),
        "tokens_per_run": n_tokens, "mall_flush_ms": flush.time_ms(),
        "note": "ms_per_step is one whole run (all rounds: host bookkeeping, copies, cache flushes and both "
                "calls); the rooflines sum only the calls' own events"})
    line["steps"] = len(tot_ms)
    if not args.no_cpu_baseline:
        # oracle sample: the last 128 prefill rows of the 24 sessions around
        # the median history
        Ks, Vs, rws = [], [], []
        for i in np.argsort(wl.hist)[len(wl.hist) // 2 - 12: len(wl.hist) // 2 + 12]:
            K, V = wl.kv(int(i), 0, int(wl.hist[i]))
            Ks.append(K)
            Vs.append(V)
            for p in range(int(wl.hist[i]) - 128, int(wl.hist[i])):
                rws.append((len(Ks) - 1, p, wl.queries(int(i), p, p + 1)[0]))
        line["cpu_baseline"] = cpu_baseline_rows(Ks, Vs, rws, Hq, Hkv, args.cpu_seconds, "multiturn prefill")
    return line


# ---------------------------------------------------------------------------
# tiny: 4 fp32 requests over a shared 64-token prefix, 16 new tokens + 1 decode
# ---------------------------------------------------------------------------
def bench_tiny(args, flush):
    """hipEvent medians of >= 50 extend calls and >= 50 decode calls (caches
    flushed before each), and the full oracle on the host."""
    import torch
    import oracle
    import workloads as W
    import prefix_shared_paged_amd as sp
    from prefix_shared_paged_amd import accounting as acc
    from prefix_shared_paged_amd.paged_cache import PagedKVCache

    wl = W.tiny(seed=0)
    s = wl.spec
    B, P, E = wl.B, 64, 16
    Hq, Hkv, D = s.Hq, s.Hkv, s.D
    dev = "cuda"
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    cache = PagedKVCache(s.num_slots, 1, Hkv, D, torch.float32, B + 1, P + E + 2, W.pool_order(s), dev)
    [st] = cache.admit([wl.prefix_tokens(0)])
    cache.append([st], [P])
    Kp, Vp = wl.prefix_kv(0)
    cache.store(f32(Kp), f32(Vp), st.slots)
    cache.insert(st)
    cache.release(st)
    rows = cache.admit([np.concatenate([wl.prefix_tokens(0), wl.suffix_tokens(r, E)]) for r in range(B)])
    assert all(r.matched == P for r in rows)
    cache.append(rows, [E + 1] * B)
    kv = [wl.suffix_kv(r, E + 1) for r in range(B)]
    for r, st in enumerate(rows):
        cache.store(f32(kv[r][0]), f32(kv[r][1]), st.slots[P:])
    q_ext = f32(np.concatenate([wl.queries(r, E) for r in range(B)]))
    q_dec = f32(np.stack([wl.queries(r, 1, step=1)[0] for r in range(B)]))
    req_rows = cache.rows_tensor(rows)
    plen = torch.full((B,), P, dtype=torch.int32, device=dev)
    q_off = torch.arange(0, (B + 1) * E, E, dtype=torch.int64, device=dev)
    seq = torch.full((B,), P + E + 1, dtype=torch.int32, device=dev)
    o_ext, o_dec = torch.empty_like(q_ext), torch.empty_like(q_dec)
    ws = torch.empty(sp.decode_workspace_size(B, P + E + 1, Hq, Hkv, D), dtype=torch.uint8, device=dev)
    n = max(50, args.steps)

    def timed(fn):
        for _ in range(args.warmup):
            flush()
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(n):
            flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))

    t0 = time.perf_counter()
    ext = timed(lambda: sp.extend_attn(q_ext, cache.k_pool, cache.v_pool, cache.r2t, req_rows, plen, q_off, E,
                                       o=o_ext))
    dec = timed(lambda: sp.decode_attn(q_dec, cache.k_pool, cache.v_pool, cache.r2t, req_rows, seq, P + E + 1,
                                       o=o_dec, workspace=ws))
    wall = (time.perf_counter() - t0) * 1e3
    flops_e = acc.extend_flops([P] * B, [E] * B, Hq, D)
    flops_d = acc.decode_flops([P + E + 1] * B, Hq, D)
    byts_d = acc.decode_bytes_flat([P + E + 1] * B, Hq, Hkv, D, 4)
    step_ms = ext + dec
    tflops = (flops_e + flops_d) / (step_ms * 1e-3) / 1e12
    config = {"workload": "tiny fp32: 4 requests sharing a 64-token prefix, 16 new tokens each (one extend "
                          "call), then one decode token each (one decode call, L = 81); 8/8 heads, head_dim 64, "
                          "1024-slot shuffled pool, page 1", "batch": B, "prefix": P, "new_tokens": E}
    roof = {"bound": "alu", "achieved": tflops, "peak": PEAK_F32_VALU_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / PEAK_F32_VALU_TFLOPS, "traffic": None,
            "kernel": "extend_f32 + decode split_f32 + merge (latency-bound: the fraction is not meaningful)",
            "flops_per_step": flops_e + flops_d, "avg_launch_ms": step_ms}
    line = base_line((B * E + B) / (step_ms * 1e-3), step_ms, args, config, roof, {
        "extend": {"median_us": ext * 1e3, "flops": flops_e, "tokens_per_s": B * E / (ext * 1e-3)},
        "decode": {"median_us": dec * 1e3, "kv_bytes": byts_d, "gbps": byts_d / (dec * 1e-3) / 1e9,
                   "tokens_per_s": B / (dec * 1e-3)},
        "reps": n, "timing": "hipEvent median per call, caches flushed before each", "wall_ms_all_reps": wall})
    line["dtype"] = "f32"
    line["steps"] = n
    if not args.no_cpu_baseline:
        Ks = [np.concatenate([Kp, kv[r][0]]) for r in range(B)]
        Vs = [np.concatenate([Vp, kv[r][1]]) for r in range(B)]
        rr = [r for r in range(B) for _ in range(E)] + list(range(B))
        pos = [P + i for _ in range(B) for i in range(E)] + [P + E] * B
        Q = np.concatenate([q_ext.cpu().numpy(), q_dec.cpu().numpy()])
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.attention(Ks, Vs, rr, pos, Q, Hq, Hkv)
            reps += 1
            if time.perf_counter() - t0 > min(args.cpu_seconds, 5.0):
                break
        t = (time.perf_counter() - t0) / reps
        line["cpu_baseline"] = {"value": (B * E + B) / t, "unit": "tokens/s", "cores": oracle.default_threads(),
                                "kind": "oracle", "sample": f"the full workload (64 extend rows + 4 decode rows, "
                                                            f"all 8 heads), fp64 oracle, {t * 1e3:.2f} ms per run, "
                                                            f"{reps} runs"}
    return line


def log(msg):
    """Progress on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); multi-GPU runs are not "
              "supported", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X); none is visible", file=sys.stderr)
        sys.exit(1)
    flush = MallFlush(torch, "cuda")
    if args.config == "extend":
        line, ctx = bench_extend(args, flush)
        log(f"extend steps done: {line['ms_per_step']:.3f} ms/step, extend kernel "
            f"{line['roofline']['avg_launch_ms']:.3f} ms")
        if not args.no_decode:
            torch.cuda.empty_cache()
            dec, _ = measure_decode(args, flush)
            line["decode_batch"] = dec
            log(f"decode batch done: flat {dec['flat']['call_ms']:.3f} ms, cascade {dec['cascade']['call_ms']:.3f} ms")
            torch.cuda.empty_cache()
            fork, _ = measure_fork(args, flush)
            line["fork_sweep"] = fork
            log(f"fork sweep done: {fork['sweep_ms']:.1f} ms per sweep")
            torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_extend(ctx[1], ctx[2], ctx[3], args.cpu_seconds)
        else:
            line["cpu_baseline"] = None
    else:
        line = {"tiny": bench_tiny, "decode": bench_decode, "fork": bench_fork, "verify": bench_verify,
                "mla": bench_mla, "hicache": bench_hicache,
                "multiturn": bench_multiturn}[args.config](args, flush)
    torch.cuda.empty_cache()
    box = box_peaks()
    line["box"] = box
    with_box(line.get("roofline"), box)
    log(f"box probes done: {box['mfma_bf16_tflops']:.0f} TFLOP/s bf16 MFMA, {box['copy_gbps']:.0f} GB/s copy")
    print(json.dumps(line, default=lambda x: x.item() if hasattr(x, "item") else str(x)), flush=True)


if __name__ == "__main__":
    main()
