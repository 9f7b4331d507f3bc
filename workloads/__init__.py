"""Seeded synthetic inputs for the paged prefix-shared attention workloads.

This module only DRAWS inputs: token ids, group structure, lengths, the
initial order of the slot pool's free list, and Q/K/V values.  It holds none
of the method's arithmetic (no attention, no matching, no allocation), so the
oracle and the HIP path can both consume it without sharing code.

Every random array is drawn from numpy's PCG64 seeded by a tuple
(seed, stream tag, entity ids...), so any piece (one request's keys, one
group's prefix, one decode step's queries) can be regenerated on its own
without materialising the whole workload.

Values: the shapes and distributions are those of the five workloads:
  tiny      fp32, 4 requests sharing a 64-token prefix + 16 new tokens each,
            8/8 heads, head_dim 64, N(0,1), 1024 slots, page size 1
  extend    bf16, 64 requests sharing a cached 2048-token prefix + 256 new
            tokens each, 32/8 heads, head_dim 128, N(0,1)*0.5, 2^20 slots
  decode    bf16, 256 requests in 16 groups of 16, group prefix ~U[512,4096],
            context ~U[max(1024, P+1), 8192], 32/8/128, 2^21 slots
  fork      bf16, 16 prompts x 4096 tokens, 8 branches each, suffix 1..512,
            32/8/128, 2^18 slots
  verify    bf16, 64 requests, own cached contexts ~U[2048, 8192], q_len new
            tokens each (2-16: the verify step of speculative decoding),
            32/8/128, 2^20 slots
  mla       bf16, 128 requests in 16 prefix groups of 8, prefix ~U[512,4096],
            context ~U[max(1024,P+1),8192], one 576-dim latent row per token
            (values: its first 512 dims), 128 (or 16) query heads, 2^21 slots
  multiturn bf16, 128 sessions, history ~ lognormal(median 3000, sigma 1)
            clamped to [32, 32768], cached 16*floor(0.7 H / 16), chunks of
            512, page size 16, 64/8/128, 2^20 slots
bf16 values are drawn in float32 and rounded to the nearest bf16 (ties to
even); both paths consume the rounded values.
"""
from dataclasses import dataclass, field

import numpy as np

VOCAB = 128000
SIBLING_BASE = 120000   # first token after a shared prefix: SIBLING_BASE + sibling index

# stream tags
T_TOK_PREFIX, T_TOK_SUFFIX, T_KV_PREFIX, T_KV_SUFFIX, T_Q, T_LEN, T_POOL, T_KV_NEW, T_FP8 = range(9)


def rng(seed, *ids):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed)] + [int(i) for i in ids])))


def round_to_bf16(x):
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    u = np.array(x, np.float32, copy=True).view(np.uint32)   # finite inputs only
    lsb = (u >> 16) & 1
    u += 0x7FFF
    u += lsb
    u &= 0xFFFF0000
    return u.view(np.float32)


def bf16_bits(x):
    """float32 array holding bf16 values -> uint16 bit patterns."""
    x = np.ascontiguousarray(x, np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass
class Spec:
    name: str
    dtype: str            # "f32" or "bf16"
    Hq: int
    Hkv: int
    D: int
    page_size: int
    num_slots: int
    value_scale: float    # values ~ N(0,1) * value_scale
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def scale(self):
        return 1.0 / np.sqrt(self.D)


def values(spec, shape, *ids):
    """Q/K/V values for one entity: N(0,1)*scale, rounded to bf16 for bf16 specs."""
    x = rng(spec.seed, *ids).standard_normal(shape, dtype=np.float32)
    if spec.value_scale != 1.0:
        x = x * np.float32(spec.value_scale)
    if spec.dtype == "bf16":
        x = round_to_bf16(x)
    return x


def fp8_scales(spec):
    """Per-KV-head factors (k_scale, v_scale), float32 [Hkv] each, of an FP8
    KV cache over this workload's values: value_scale * U(4, 6) / 448, i.e.
    the largest code stands for 4 to 6 standard deviations (values beyond it
    clamp).  Drawn, not computed from the data."""
    r = rng(spec.seed, T_FP8)
    k = (spec.value_scale * r.uniform(4.0, 6.0, spec.Hkv) / 448.0).astype(np.float32)
    v = (spec.value_scale * r.uniform(4.0, 6.0, spec.Hkv) / 448.0).astype(np.float32)
    return k, v


def pool_order(spec):
    """Initial free-list order of the slot pool: a seeded permutation of page ids."""
    n_pages = spec.num_slots // spec.page_size
    return rng(spec.seed, T_POOL).permutation(n_pages).astype(np.int32)


def tokens(spec, tag, n, first, *ids):
    """n synthetic token ids; token 0 is forced to `first` (None = random)."""
    t = rng(spec.seed, tag, *ids).integers(1, SIBLING_BASE, size=n, dtype=np.int64).astype(np.int32)
    if n > 0 and first is not None:
        t[0] = first
    return t


# ---------------------------------------------------------------------------
# Group-structured workloads: groups of requests that share a prefix.
# Request r belongs to group grp[r] and is sibling sib[r] in it; its logical
# sequence is  prefix(grp) || suffix(r).
# ---------------------------------------------------------------------------
@dataclass
class GroupWorkload:
    spec: Spec
    prefix_len: np.ndarray    # [G]
    grp: np.ndarray           # [B]
    sib: np.ndarray           # [B]
    ctx_len: np.ndarray       # [B] full logical length L_r at the evaluated step

    @property
    def B(self):
        return len(self.grp)

    @property
    def G(self):
        return len(self.prefix_len)

    def group_members(self, g):
        return np.nonzero(self.grp == g)[0]

    def prefix_tokens(self, g):
        return tokens(self.spec, T_TOK_PREFIX, int(self.prefix_len[g]), g + 1, g)

    def suffix_tokens(self, r, n=None):
        n = int(self.ctx_len[r] - self.prefix_len[self.grp[r]]) if n is None else n
        return tokens(self.spec, T_TOK_SUFFIX, n, SIBLING_BASE + int(self.sib[r]), r)

    def prefix_kv(self, g):
        P = int(self.prefix_len[g])
        s = self.spec
        return (values(s, (P, s.Hkv, s.D), T_KV_PREFIX, g, 0),
                values(s, (P, s.Hkv, s.D), T_KV_PREFIX, g, 1))

    def suffix_kv(self, r, n=None):
        n = int(self.ctx_len[r] - self.prefix_len[self.grp[r]]) if n is None else n
        s = self.spec
        return (values(s, (n, s.Hkv, s.D), T_KV_SUFFIX, r, 0),
                values(s, (n, s.Hkv, s.D), T_KV_SUFFIX, r, 1))

    def logical_kv(self, r, n_suffix=None):
        kp, vp = self.prefix_kv(self.grp[r])
        ks, vs = self.suffix_kv(r, n_suffix)
        return np.concatenate([kp, ks]), np.concatenate([vp, vs])

    def queries(self, r, n, step=0):
        # spec.extra["q_scale"] (a power of two, so bf16 values stay exact)
        # widens the queries alone: sharper softmax over the same keys
        s = self.spec
        q = values(s, (n, s.Hq, s.D), T_Q, r, step)
        qs = s.extra.get("q_scale", 1.0)
        return q * np.float32(qs) if qs != 1.0 else q


def tiny(seed=0):
    """4 requests sharing a 64-token prefix, 16 new tokens each, then 1 decode token."""
    spec = Spec("tiny", "f32", 8, 8, 64, 1, 1024, 1.0, seed)
    B = 4
    return GroupWorkload(spec, np.array([64]), np.zeros(B, np.int64), np.arange(B),
                         np.full(B, 64 + 16 + 1, np.int64))


def extend(seed=0, B=64, prefix=2048, new=256, Hq=32, Hkv=8, D=128, num_slots=1 << 20):
    """B requests sharing a cached prefix, each adding `new` causal tokens."""
    spec = Spec("extend", "bf16", Hq, Hkv, D, 1, num_slots, 0.5, seed)
    return GroupWorkload(spec, np.array([prefix]), np.zeros(B, np.int64), np.arange(B),
                         np.full(B, prefix + new, np.int64))


def decode(seed=0, G=16, per_group=16, p_lo=512, p_hi=4096, l_lo=1024, l_hi=8192,
           Hq=32, Hkv=8, D=128, num_slots=1 << 21):
    """Decode batch of G*per_group requests in G prefix groups."""
    spec = Spec("decode", "bf16", Hq, Hkv, D, 1, num_slots, 0.5, seed)
    r = rng(seed, T_LEN)
    P = r.integers(p_lo, p_hi + 1, size=G)
    grp = np.repeat(np.arange(G), per_group)
    sib = np.tile(np.arange(per_group), G)
    L = np.array([r.integers(max(l_lo, P[g] + 1), l_hi + 1) for g in grp], np.int64)
    return GroupWorkload(spec, P.astype(np.int64), grp, sib, L)


def fork(seed=0, G=16, branches=8, prompt=4096, max_suffix=512, Hq=32, Hkv=8, D=128,
         num_slots=1 << 18):
    """G prompts, each forked into `branches` branches; ctx_len holds the longest step."""
    spec = Spec("fork", "bf16", Hq, Hkv, D, 1, num_slots, 0.5, seed,
                extra={"max_suffix": max_suffix})
    grp = np.repeat(np.arange(G), branches)
    sib = np.tile(np.arange(branches), G)
    return GroupWorkload(spec, np.full(G, prompt, np.int64), grp, sib,
                         np.full(G * branches, prompt + max_suffix, np.int64))


def verify(seed=0, B=64, q_len=4, p_lo=2048, p_hi=8192, Hq=32, Hkv=8, D=128, num_slots=1 << 20):
    """Small-q extend (the verify step of speculative decoding): B requests,
    each with its own cached context of P ~ U[p_lo, p_hi] tokens (one request
    per group) and q_len new tokens."""
    spec = Spec("verify", "bf16", Hq, Hkv, D, 1, num_slots, 0.5, seed, extra={"q_len": q_len})
    P = rng(seed, T_LEN).integers(p_lo, p_hi + 1, size=B).astype(np.int64)
    return GroupWorkload(spec, P, np.arange(B, dtype=np.int64), np.zeros(B, np.int64), P + q_len)


def mla(seed=0, G=16, per_group=8, p_lo=512, p_hi=4096, l_lo=1024, l_hi=8192, Hq=128, num_slots=1 << 21):
    """Latent (MLA-style) decode batch: G*per_group requests in G prefix groups,
    one latent row of 576 dims per token (D holds 576; values are its first 512),
    Hq query heads over one KV head."""
    spec = Spec("mla", "bf16", Hq, 1, 576, 1, num_slots, 0.5, seed, extra={"Dv": 512})
    r = rng(seed, T_LEN)
    P = r.integers(p_lo, p_hi + 1, size=G)
    grp = np.repeat(np.arange(G), per_group)
    sib = np.tile(np.arange(per_group), G)
    L = np.array([r.integers(max(l_lo, P[g] + 1), l_hi + 1) for g in grp], np.int64)
    return GroupWorkload(spec, P.astype(np.int64), grp, sib, L)


# ---------------------------------------------------------------------------
# Multi-turn sessions (no cross-session sharing).
# ---------------------------------------------------------------------------
@dataclass
class SessionWorkload:
    spec: Spec
    hist: np.ndarray      # H_s: full history length to prefill
    cached: np.ndarray    # c_s: already cached (16-aligned, ~70%)
    chunk: int
    decode_tokens: int    # decode steps run after a session's prefill completes

    @property
    def n(self):
        return len(self.hist)

    def tokens(self, s):
        return tokens(self.spec, T_TOK_PREFIX, int(self.hist[s]) + self.decode_tokens, s + 1, s)

    def kv(self, s, lo, hi):
        """K/V of positions [lo, hi) of session s, drawn in 512-token blocks."""
        spec = self.spec
        blk = 512
        ks, vs = [], []
        for b in range(lo // blk, -(-hi // blk)):
            k = values(spec, (blk, spec.Hkv, spec.D), T_KV_SUFFIX, s, b, 0)
            v = values(spec, (blk, spec.Hkv, spec.D), T_KV_SUFFIX, s, b, 1)
            a0 = max(lo, b * blk) - b * blk
            a1 = min(hi, (b + 1) * blk) - b * blk
            ks.append(k[a0:a1])
            vs.append(v[a0:a1])
        if not ks:
            z = np.zeros((0, spec.Hkv, spec.D), np.float32)
            return z, z.copy()
        return np.concatenate(ks), np.concatenate(vs)

    def queries(self, s, lo, hi):
        """Queries of positions [lo, hi) of session s (one draw per position)."""
        spec = self.spec
        out = np.empty((hi - lo, spec.Hq, spec.D), np.float32)
        for i, t in enumerate(range(lo, hi)):
            out[i] = values(spec, (spec.Hq, spec.D), T_Q, s, t)
        return out


def multiturn(seed=0, n_sessions=128, median=3000, sigma=1.0, h_min=32, h_max=32768,
              hit=0.7, chunk=512, decode_tokens=1, Hq=64, Hkv=8, D=128, num_slots=1 << 20):
    spec = Spec("multiturn", "bf16", Hq, Hkv, D, 16, num_slots, 0.5, seed)
    r = rng(seed, T_LEN)
    H = np.clip(np.round(np.exp(np.log(median) + sigma * r.standard_normal(n_sessions))),
                h_min, h_max).astype(np.int64)
    c = (16 * np.floor(hit * H / 16)).astype(np.int64)
    return SessionWorkload(spec, H, c, chunk, decode_tokens)
