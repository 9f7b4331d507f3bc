"""Validation mode of the device calls (GPU; the checks run on the host).

With validation switched on (sgl_set_validate(1)), a device call copies its
index metadata to the host first and returns SGL_ERR_INVALID -- enqueuing
nothing -- on an out-of-range slot, row or length, a length beyond the row
stride, or a cascade group whose requests do not share the group's prefix
slots.  Each case below checks the status and that nothing ran: the output
keeps its sentinel values and the pool rows the call would have stored into
keep theirs.  Every malformed argument here is caught on the host; none of
these calls reaches a kernel.
"""
import numpy as np
import pytest
import torch

import prefix_shared_paged_amd as sp

pytestmark = pytest.mark.gpu

S, HQ, HKV, D, B, STRIDE = 4096, 32, 8, 128, 4, 256


@pytest.fixture
def validating():
    prev = sp.set_validate(1)
    yield
    sp.set_validate(prev)


def _case(seed=0):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    rnd = lambda *shape: (torch.randn(shape, generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    c = dict(kp=rnd(S, HKV, D), vp=rnd(S, HKV, D), q=rnd(B, HQ, D), kn=rnd(B, HKV, D), vn=rnd(B, HKV, D))
    r2t = torch.randperm(S, generator=gen, device="cuda")[:B * STRIDE].to(torch.int32).view(B, STRIDE)
    r2t[:, :64] = r2t[0, :64].clone()          # one group sharing a 64-token prefix
    c["r2t"] = r2t.contiguous()
    c["rows"] = torch.arange(B, dtype=torch.int32, device="cuda")
    c["seq"] = torch.tensor([200, 180, 256, 100], dtype=torch.int32, device="cuda")
    c["gptr"] = torch.tensor([0, B], dtype=torch.int32, device="cuda")
    c["gpl"] = torch.tensor([64], dtype=torch.int32, device="cuda")
    return c


def _decode(c, cascade, max_seq=256, o=None):
    o = torch.full((B, HQ, D), 7.0, dtype=torch.bfloat16, device="cuda") if o is None else o
    if cascade:
        sp.cascade_decode_attn(c["q"], c["kp"], c["vp"], c["r2t"], c["rows"], c["seq"], c["gptr"], c["gpl"],
                               max_seq, B, 64, k_new=c["kn"], v_new=c["vn"], o=o)
    else:
        sp.decode_attn(c["q"], c["kp"], c["vp"], c["r2t"], c["rows"], c["seq"], max_seq, k_new=c["kn"],
                       v_new=c["vn"], o=o)
    return o


def _expect_invalid(fn, c, o_shape=(B, HQ, D)):
    """fn(o) must fail with SGL_ERR_INVALID and leave o and both pools as they were."""
    o = torch.full(o_shape, 7.0, dtype=torch.bfloat16, device="cuda")
    k0, v0 = c["kp"].clone(), c["vp"].clone()
    with pytest.raises(sp.SglError) as e:
        fn(o)
    torch.cuda.synchronize()
    assert e.value.status == sp.SGL_ERR_INVALID, sp.status_string(e.value.status)
    assert bool((o == 7.0).all()), "the failed call wrote its output"
    assert torch.equal(c["kp"], k0) and torch.equal(c["vp"], v0), "the failed call stored K/V"


def test_set_validate_switches_in_process():
    prev = sp.set_validate(1)
    try:
        assert sp.set_validate(0) == 1
        assert sp.set_validate(-1) == 0
        assert sp.set_validate(1) == -1
    finally:
        sp.set_validate(prev)


@pytest.mark.parametrize("cascade", [False, True])
def test_valid_call_is_unchanged_by_validation(validating, cascade):
    c = _case(1)
    o1 = _decode(c, cascade)
    sp.set_validate(0)
    o2 = _decode(c, cascade)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("cascade", [False, True])
def test_decode_out_of_range_slot(validating, cascade):
    c = _case(2)
    c["r2t"][1, 50] = S                       # one past the pool
    _expect_invalid(lambda o: _decode(c, cascade, o=o), c)
    c["r2t"][1, 50] = -3
    _expect_invalid(lambda o: _decode(c, cascade, o=o), c)


@pytest.mark.parametrize("cascade", [False, True])
def test_decode_bad_row(validating, cascade):
    c = _case(3)
    c["rows"][2] = B                          # the table has rows 0..B-1
    _expect_invalid(lambda o: _decode(c, cascade, o=o), c)


@pytest.mark.parametrize("cascade", [False, True])
def test_decode_seq_len_beyond_row_stride(validating, cascade):
    c = _case(4)
    c["seq"][0] = STRIDE + 1
    _expect_invalid(lambda o: _decode(c, cascade, max_seq=STRIDE + 1, o=o), c)
    c["seq"][0] = 200
    c["seq"][3] = 0                           # a decode context holds at least the current token
    _expect_invalid(lambda o: _decode(c, cascade, o=o), c)


def test_decode_seq_len_beyond_max_bound(validating):
    c = _case(5)
    _expect_invalid(lambda o: _decode(c, False, max_seq=255, o=o), c)   # seq[2] = 256


def test_cascade_group_prefix_mismatch(validating):
    c = _case(6)
    other = int(c["r2t"][0, 200])             # a valid slot, not the prefix's
    c["r2t"][2, 10] = other
    _expect_invalid(lambda o: _decode(c, True, o=o), c)
    # the same table is fine for flat decode, and for a cascade whose group
    # prefix ends before the differing column
    _decode(c, False)
    c["gpl"][0] = 10
    _decode(c, True)
    torch.cuda.synchronize()


def test_cascade_group_arrays(validating):
    c = _case(7)
    c["gpl"][0] = 101                         # longer than request 3's context (100)
    _expect_invalid(lambda o: _decode(c, True, o=o), c)
    c["gpl"][0] = 64
    c["gptr"][1] = B - 1                      # the groups must cover the batch
    _expect_invalid(lambda o: _decode(c, True, o=o), c)


def test_cascade_prefix_reaching_the_current_token(validating):
    # a call that stores the current tokens needs every group prefix to end
    # before its requests' current positions; with no token to store the
    # prefix may cover a whole context
    c = _case(9)
    c["r2t"][:, :100] = c["r2t"][0, :100].clone()
    c["gpl"][0] = 100                         # request 3's whole context (100), its current token included
    _expect_invalid(lambda o: _decode(c, True, o=o), c)
    o = torch.full((B, HQ, D), 7.0, dtype=torch.bfloat16, device="cuda")
    sp.cascade_decode_attn(c["q"], c["kp"], c["vp"], c["r2t"], c["rows"], c["seq"], c["gptr"], c["gpl"],
                           256, B, 100, o=o)
    torch.cuda.synchronize()
    assert not bool((o == 7.0).any())
    # a current token whose slot is one of the group's prefix slots
    c["gpl"][0] = 64
    c["r2t"][1, 179] = c["r2t"][0, 5]         # request 1's current position (seq 180)
    _expect_invalid(lambda o: _decode(c, True, o=o), c)


def test_extend_invalid_metadata(validating):
    c = _case(8)
    E = 8
    q = c["q"][:, :, :].repeat(E, 1, 1)[:B * E].contiguous()       # [B*E, HQ, D]
    kn = c["kn"].repeat(E, 1, 1)[:B * E].contiguous()
    vn = c["vn"].repeat(E, 1, 1)[:B * E].contiguous()
    plen = torch.tensor([100, 64, 200, 10], dtype=torch.int32, device="cuda")
    q_off = torch.arange(0, (B + 1) * E, E, dtype=torch.int64, device="cuda")

    def ext(o, plen=plen, q_off=q_off, rows=c["rows"]):
        sp.extend_attn(q, c["kp"], c["vp"], c["r2t"], rows, plen, q_off, E, k_new=kn, v_new=vn, o=o)

    shape = (B * E, HQ, D)
    o = torch.full(shape, 7.0, dtype=torch.bfloat16, device="cuda")
    ext(o)                                                       # valid
    torch.cuda.synchronize()
    assert not bool((o == 7.0).any())
    bad = c["r2t"].clone()
    c["r2t"][2, 203] = S + 5                                     # a new token's slot out of range
    _expect_invalid(ext, c, shape)
    c["r2t"].copy_(bad)
    _expect_invalid(lambda o: ext(o, plen=torch.tensor([100, 64, STRIDE - E + 1, 10], dtype=torch.int32,
                                                       device="cuda")), c, shape)     # past the row
    _expect_invalid(lambda o: ext(o, q_off=torch.tensor([0, 8, 16, 24, 31], dtype=torch.int64,
                                                        device="cuda")), c, shape)    # q_off[B] != n_tokens
    _expect_invalid(lambda o: ext(o, rows=torch.tensor([0, 1, 2, -1], dtype=torch.int32, device="cuda")),
                    c, shape)


# ---------------------------------------------------------------------------
# device-side index check (sgl_count_bad_slots): stream-ordered, no host copy
# ---------------------------------------------------------------------------
def _count_bad(r2t, rows, seq, max_seq, num_slots):
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    sp.count_bad_slots(r2t, rows, seq, max_seq, num_slots, cnt)
    torch.cuda.synchronize()
    return int(cnt.item()) & 0xFFFFFFFF


def _count_bad_host(r2t, rows, seq, max_seq, num_slots):
    t, rs, ls = r2t.cpu().numpy(), rows.cpu().numpy(), seq.cpu().numpy()
    n = 0
    for r, L in zip(rs, ls):
        if r < 0 or r >= t.shape[0] or L < 0 or L > min(t.shape[1], max_seq):
            n += 1
            continue
        ids = t[r, :L]
        n += int(np.count_nonzero((ids < 0) | (ids >= num_slots)))
    return n


def test_count_bad_slots_clean_table_counts_zero():
    c = _case()
    assert _count_bad(c["r2t"], c["rows"], c["seq"], 256, S) == 0
    # the same table against a smaller pool: every id >= 1000 in the rows counts
    want = _count_bad_host(c["r2t"], c["rows"], c["seq"], 256, 1000)
    assert want > 0 and _count_bad(c["r2t"], c["rows"], c["seq"], 256, 1000) == want


def test_count_bad_slots_marked_ids_rows_and_lengths():
    c = _case(3)
    r2t = c["r2t"].clone()
    r2t[0, 5] = -1                 # inside row 0's 200 keys
    r2t[1, 179] = S                # the last key of row 1
    r2t[1, 180] = -7               # past row 1's length: not read, not counted
    r2t[2, 0] = 1 << 30
    rows = torch.tensor([0, 1, 2, 3, 9, 1], dtype=torch.int32, device="cuda")       # row 9 is outside the table
    seq = torch.tensor([200, 180, 256, 100, 10, 300], dtype=torch.int32, device="cuda")   # 300 > stride
    want = _count_bad_host(r2t, rows, seq, 256, S)
    assert want == 5
    assert _count_bad(r2t, rows, seq, 256, S) == want
    # a length above max_seq_len counts as well, and adds to what the counter holds
    cnt = torch.full((1,), 4, dtype=torch.int32, device="cuda")
    sp.count_bad_slots(r2t, rows[:4], seq[:4], 199, S, cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 4 + _count_bad_host(r2t, rows[:4], seq[:4], 199, S)


def test_count_bad_slots_long_rows_span_several_chunks():
    # rows of 9,000 keys (three 4,096-key chunks), bad ids near each chunk edge
    n_rows, stride, slots = 3, 9000, 1 << 16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    r2t = torch.randint(0, slots, (n_rows, stride), generator=gen, device="cuda", dtype=torch.int32)
    for col in (0, 4095, 4096, 8191, 8192, 8999):
        r2t[1, col] = slots + col
    r2t[2, 4096] = -3
    rows = torch.arange(n_rows, dtype=torch.int32, device="cuda")
    seq = torch.tensor([9000, 9000, 4096], dtype=torch.int32, device="cuda")   # row 2 stops before its bad id
    assert _count_bad(r2t, rows, seq, 9000, slots) == 6
