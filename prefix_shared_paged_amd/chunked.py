"""Chunked prefill interleaved with decode over a paged prefix cache.

Long prompts are split into chunks so prefill work mixes with decode work in
every round ("SGLang：从前端 DSL 到 SRT 服务运行时" (oripoin.cn): chunked
prefill keeps long prompts from stalling decode; "Lecture 16 · 案例研究：SGLang"
(semidirectx.com) section 3 models a fixed prompt-token budget per round).
One round:
  1. every session with prompt tokens left runs its next chunk of at most
     `chunk` tokens, all in ONE batched extend call (a chunk attends to the
     session's cached prefix, its earlier chunks and itself, causally); a
     session whose prompt is done is inserted into the radix tree (prefill
     completion);
  2. every session whose prompt finished in an earlier round decodes one
     token, all in ONE batched decode call.
Slots come from the paged pool (whole pages; a session first fills the rest
of its own last page).  The values of a round (Q/K/V of the positions it
processes) come from a caller callback, so the same driver serves the tests
(seeded host values) and the benchmark (tensors already resident in HBM).
"""
import numpy as np

from . import decode_attn, decode_workspace_size, extend_attn, extend_workspace_size


class Session:
    __slots__ = ("sid", "tokens", "hist", "row", "pos", "decoded", "done_round")

    def __init__(self, sid, tokens, hist, row):
        self.sid = sid
        self.tokens = tokens      # prompt (hist tokens) followed by decode tokens
        self.hist = hist          # prompt length H
        self.row = row            # PagedKVCache row
        self.pos = row.matched    # next position to prefill
        self.decoded = 0
        self.done_round = -1      # round in which its prefill completed


def plan_rounds(hist, cached, chunk):
    """Host-only dry run: per round, the extend list [(sid, lo, hi)] and the
    decode list [(sid, position)] the runner will execute (ends with one
    decode-only round after the last prefill chunk)."""
    pos = list(cached)
    done = [-1] * len(hist)
    dec = [0] * len(hist)
    rounds = []
    r = 0
    while True:
        pending = [i for i in range(len(hist)) if pos[i] < hist[i]]
        ext = [(i, pos[i], min(hist[i], pos[i] + chunk)) for i in pending]
        dl = [(i, hist[i] + dec[i]) for i in range(len(hist)) if pos[i] >= hist[i] and done[i] < r]
        if not ext and not dl:
            break
        rounds.append((ext, dl))
        for i, lo, hi in ext:
            pos[i] = hi
            if hi >= hist[i]:
                done[i] = r
        for i, _ in dl:
            dec[i] += 1
        r += 1
        if not pending:
            break
    return rounds


class ChunkedRunner:
    def __init__(self, cache, chunk=512):
        import torch
        self.torch = torch
        self.cache = cache
        self.chunk = chunk
        self.sessions = []
        self.round_no = 0
        self._ws = {}

    def admit(self, sids, token_lists, hists):
        rows = self.cache.admit(token_lists)
        for sid, toks, h, st in zip(sids, token_lists, hists, rows):
            self.sessions.append(Session(sid, np.asarray(toks, np.int32), int(h), st))
        return rows

    def pending(self):
        return any(s.pos < s.hist for s in self.sessions)

    def _workspace(self, kind, nbytes):
        """A reusable workspace per call kind, grown when a round needs more."""
        ws = self._ws.get(kind)
        if ws is None or ws.numel() < nbytes:
            ws = self._ws[kind] = self.torch.empty(max(nbytes, 1), dtype=self.torch.uint8, device=self.cache.device)
        return ws

    def run_round(self, inputs, lse=False, timing=None):
        """Run one round.  inputs(ext, dec) gets ext = [(sid, lo, hi)] and
        dec = [(sid, position)] and returns device tensors
        (q_ext [n, Hq, D], k_ext, v_ext [n, Hkv, D], q_dec [m, Hq, D], k_dec, v_dec),
        rows in list order.  timing (optional) has before(kind) and
        after(kind), called right around the library's extend and decode
        calls (kind "extend" / "decode"): every host step of the round and
        every host-to-device copy of a call's arguments comes before
        before(kind).  Returns what ran, with the outputs."""
        torch = self.torch
        c = self.cache
        dev = c.device
        ext = [(s, s.pos, min(s.hist, s.pos + self.chunk)) for s in self.sessions if s.pos < s.hist]
        dec = [s for s in self.sessions if s.pos >= s.hist and s.done_round < self.round_no]
        if not ext and not dec:
            return None
        L = [s.hist + s.decoded + 1 for s in dec]
        q, k, v, qd, kd, vd = inputs([(s.sid, lo, hi) for s, lo, hi in ext],
                                     [(s.sid, l - 1) for s, l in zip(dec, L)])
        out = {"round": self.round_no, "extend": [], "decode": []}
        if ext:
            rows = [s.row for s, _, _ in ext]
            n = [hi - lo for _, lo, hi in ext]
            c.append(rows, n)
            offs = np.zeros(len(ext) + 1, np.int64)
            offs[1:] = np.cumsum(n)
            lse_t = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=dev) if lse else None
            rows_t = c.rows_tensor(rows)
            plen_t = torch.tensor([lo for _, lo, _ in ext], dtype=torch.int32, device=dev)
            off_t = torch.from_numpy(offs).to(dev)
            o = torch.empty_like(q)
            ws = self._workspace("extend", extend_workspace_size(len(ext), q.shape[0], max(n), c.r2t.shape[1],
                                                                 q.shape[1], c.Hkv, q.shape[2]))
            if timing is not None:
                timing.before("extend")
            extend_attn(q, c.k_pool, c.v_pool, c.r2t, rows_t, plen_t, off_t, max(n), k_new=k, v_new=v,
                        lse=lse_t, o=o, workspace=ws)
            if timing is not None:
                timing.after("extend")
            out["extend"] = [(s.sid, lo, hi, int(offs[i])) for i, (s, lo, hi) in enumerate(ext)]
            out["extend_out"] = o
            out["extend_lse"] = lse_t
            for s, lo, hi in ext:
                s.pos = hi
                if s.pos >= s.hist:
                    s.done_round = self.round_no
                    c.insert(s.row, s.hist)          # prefill complete
        if dec:
            rows = [s.row for s in dec]
            c.append(rows, [1] * len(dec))
            B, Hq, D = qd.shape
            ws = self._workspace("decode", decode_workspace_size(B, max(L), Hq, c.Hkv, D))
            rows_t = c.rows_tensor(rows)
            len_t = torch.tensor(L, dtype=torch.int32, device=dev)
            o = torch.empty_like(qd)
            if timing is not None:
                timing.before("decode")
            decode_attn(qd, c.k_pool, c.v_pool, c.r2t, rows_t, len_t, max(L), k_new=kd, v_new=vd, o=o,
                        workspace=ws)
            if timing is not None:
                timing.after("decode")
            out["decode"] = [(s.sid, l) for s, l in zip(dec, L)]
            out["decode_out"] = o
            for s in dec:
                s.decoded += 1
        self.round_no += 1
        return out
