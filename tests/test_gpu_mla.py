"""GPU parity of the latent (MLA-style) decode, through the C ABI.

The latent pool, queries and the current tokens' latents are drawn on the
device from a seeded generator; request r's logical latent sequence is its
rows of the pool (prefix rows shared by its group) plus its current token.
Expected: the fp64 oracle with K = latent (576 dims), V = the latent's first
512 dims, one KV head; max |o - r| <= 2e-2 (bf16 inputs), LSE within 1e-3.
The current token's latent must land in the pool bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from prefix_shared_paged_amd import mla_cascade_decode_attn, mla_decode_attn

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
LSE_TOL = 1e-3
DQK, DV = 576, 512
SCALE = 1.0 / math.sqrt(192.0)


def _print(*a):
    print(*a, flush=True)


def _dev_i(x, dtype=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(x)).to(dtype).to("cuda")


def _case(seed, Hq, members, prefixes, L, num_slots=1 << 17, q_scale=0.5):
    """Groups of requests sharing prefix slots; returns the device tensors and
    the host bookkeeping needed by the oracle."""
    B = sum(members)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    pool = (torch.randn((num_slots, DQK), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    q = (torch.randn((B, Hq, DQK), generator=gen, device="cuda") * q_scale).to(torch.bfloat16)
    kv_new = (torch.randn((B, DQK), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    perm = np.random.default_rng(seed).permutation(num_slots).astype(np.int32)
    stride = int(max(L)) + 1
    r2t = np.full((B, stride), -1, np.int32)
    pos, r = 0, 0
    grp = []
    for g, (m, P) in enumerate(zip(members, prefixes)):
        pre = perm[pos:pos + P]
        pos += P
        for _ in range(m):
            n = int(L[r]) - P
            r2t[r, :P] = pre
            r2t[r, P:L[r]] = perm[pos:pos + n]
            pos += n
            grp.append(g)
            r += 1
    assert pos <= num_slots
    gptr = np.concatenate([[0], np.cumsum(members)]).astype(np.int32)
    return dict(pool=pool, q=q, kv_new=kv_new, r2t=r2t, L=np.asarray(L, np.int64), gptr=gptr,
                P=np.asarray(prefixes, np.int64), grp=np.asarray(grp), B=B, Hq=Hq)


def _run(c, cascade):
    B, Hq = c["B"], c["Hq"]
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    pool = c["pool"].clone()
    args = (c["q"], pool, _dev_i(c["r2t"]), _dev_i(np.arange(B)), _dev_i(c["L"]))
    if cascade:
        o = mla_cascade_decode_attn(*args, _dev_i(c["gptr"]), _dev_i(c["P"]), int(c["L"].max()),
                                    int(np.diff(c["gptr"]).max()), int(c["P"].max()), kv_new=c["kv_new"],
                                    scale=SCALE, lse=lse)
    else:
        o = mla_decode_attn(*args, int(c["L"].max()), kv_new=c["kv_new"], scale=SCALE, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), pool


def _oracle(c, reqs):
    new_h = c["kv_new"].float().cpu().numpy()
    q_h = c["q"].float().cpu().numpy()
    Os, LSEs = [], []
    for r in reqs:
        L = int(c["L"][r])
        rows = c["pool"][torch.from_numpy(c["r2t"][r, :L - 1].astype(np.int64)).cuda()].float().cpu().numpy()
        lat = np.concatenate([rows, new_h[r][None]])[:, None, :]
        O, _, _, LSE = oracle.attention([lat], [np.ascontiguousarray(lat[:, :, :DV])], [0], [L - 1],
                                        q_h[r][None], c["Hq"], 1, scale=SCALE)
        Os.append(O[0])
        LSEs.append(LSE[0])
    return np.stack(Os), np.stack(LSEs)


def _check(c, reqs, tag):
    O, LSE = _oracle(c, reqs)
    for cascade in (False, True):
        o, lse, pool = _run(c, cascade)
        err = float(np.max(np.abs(o[reqs].astype(np.float64) - O)))
        lerr = float(np.max(np.abs(lse[reqs] - LSE)))
        _print(f"mla {tag} {'cascade' if cascade else 'flat'}: max abs err {err:.3e}, lse err {lerr:.2e}")
        assert err <= BF16_TOL and lerr <= LSE_TOL
        # the current token's latent was stored bit for bit
        slots = torch.from_numpy(c["r2t"][np.arange(c["B"]), c["L"] - 1].astype(np.int64)).cuda()
        assert torch.equal(pool[slots], c["kv_new"])


@pytest.mark.parametrize("Hq", [16, 32, 48, 64, 96, 128])
def test_mla_small(Hq):
    # 48 and 96 heads leave the last workgroup of a request with row blocks
    # past the last head (both kernel shapes)
    # groups of 1, 3, 5 and 16 requests; prefixes of 0, 1, 300 and 1024 keys;
    # contexts on and next to the 16-key tiles and 512-key splits
    members = [1, 3, 5, 16]
    prefixes = [0, 1, 300, 1024]
    rng = np.random.default_rng(Hq)
    L = []
    for m, P in zip(members, prefixes):
        L += [int(x) for x in rng.integers(P + 1, 1400, m)]
    L[1] = 2            # prefix 1 + current token
    L[4] = 301          # suffix = the current token only
    L[9] = 1025
    L[10] = 1536
    L[11] = 1537
    c = _case(3 + Hq, Hq, members, prefixes, L)
    _check(c, list(range(c["B"])), f"small Hq={Hq}")


@pytest.mark.parametrize("Hq", [16, 64, 128])
def test_mla_decode_shape_sampled(Hq):
    # the benchmark's shape: 128 requests in 16 groups of 8, prefixes
    # ~U[512, 4096], contexts ~U[max(1024, P+1), 8192]; 128 heads (all of
    # them, 1024-key splits, two workgroups of four 16-row blocks per split),
    # 64 heads (2048-key splits, one workgroup per split) and 16 heads (one
    # tensor-parallel share of 128); sampled requests, all heads
    rng = np.random.default_rng(9)
    members = [8] * 16
    prefixes = [int(x) for x in rng.integers(512, 4097, 16)]
    L = [int(rng.integers(max(1024, P + 1), 8193)) for P in prefixes for _ in range(8)]
    c = _case({16: 21, 64: 22, 128: 23}[Hq], Hq, members, prefixes, L, num_slots=1 << 20)
    reqs = sorted(set(rng.choice(c["B"], 24, replace=False).tolist() + [0, c["B"] - 1]
                      + [int(np.argmax(L))]))
    _check(c, reqs, f"decode shape Hq={Hq}")


def test_mla_cascade_workspace_sized_for_larger_bounds():
    # groups of 4 requests x 16 heads (64 query rows: the prefix stage runs);
    # the workspace is sized for longer prefixes and contexts than the call
    # has, and the call fits its prefix splits to it
    from prefix_shared_paged_amd import mla_cascade_workspace_size
    rng = np.random.default_rng(77)
    members = [4] * 8
    prefixes = [int(x) for x in rng.integers(1024, 2113, 8)]
    L = [int(rng.integers(P + 1, P + 600)) for P in prefixes for _ in range(4)]
    c = _case(77, 16, members, prefixes, L, num_slots=1 << 18)
    B = c["B"]
    ws = torch.empty(mla_cascade_workspace_size(B, 8, 8192, 4, 4032, 16), dtype=torch.uint8, device="cuda")
    pool = c["pool"].clone()
    lse = torch.empty((B, 16), dtype=torch.float32, device="cuda")
    o = mla_cascade_decode_attn(c["q"], pool, _dev_i(c["r2t"]), _dev_i(np.arange(B)), _dev_i(c["L"]),
                                _dev_i(c["gptr"]), _dev_i(c["P"]), int(c["L"].max()), 4, int(c["P"].max()),
                                kv_new=c["kv_new"], scale=SCALE, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    O, LSE = _oracle(c, list(range(B)))
    err = float(np.max(np.abs(o.float().cpu().numpy().astype(np.float64) - O)))
    lerr = float(np.max(np.abs(lse.cpu().numpy() - LSE)))
    _print(f"mla cascade, workspace for larger bounds: max abs err {err:.3e}, lse err {lerr:.2e}")
    assert err <= BF16_TOL and lerr <= LSE_TOL


@pytest.mark.parametrize("Hq,members", [(16, [1, 2, 4, 3]), (32, [1, 2, 2]), (64, [1, 1])])
def test_mla_cascade_prefix_stage(Hq, members):
    # groups whose members x heads fit one prefix-stage workgroup (<= 64 rows),
    # so the cascade runs its prefix stage (other groups take the flat splits)
    rng = np.random.default_rng(Hq + len(members))
    prefixes = [0, 515, 1024, 47][:len(members)]
    L = []
    for m, P in zip(members, prefixes):
        L += [int(x) for x in rng.integers(P + 1, P + 1400, m)]
    L[0] = 1
    c = _case(31 + Hq, Hq, members, prefixes, L)
    _check(c, list(range(c["B"])), f"prefix stage Hq={Hq} members={members}")


@pytest.mark.parametrize("Hq", [16, 128])
def test_mla_peaky(Hq):
    # queries 4x wider than the latents (N(0,1) x 2): the softmax concentrates
    # on few keys, so a key missed or counted twice shows in the output
    members = [1, 3, 5, 16]
    prefixes = [0, 1, 300, 1024]
    rng = np.random.default_rng(40 + Hq)
    L = []
    for m, P in zip(members, prefixes):
        L += [int(x) for x in rng.integers(P + 1, 2600, m)]
    c = _case(41 + Hq, Hq, members, prefixes, L, q_scale=2.0)
    _check(c, list(range(c["B"])), f"peaky Hq={Hq}")
