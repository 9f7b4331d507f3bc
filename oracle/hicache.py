"""Host-tier KV rows (HiCache): oracle side, plain numpy.

TEST INFRASTRUCTURE ONLY: like the rest of oracle/, only tests/,
__graft_entry__.smoke() and the cpu_baseline leg of bench.py may import this.

SGLang's HiCache keeps KV that no longer fits the GPU pool in a larger host
tier and brings a matched prefix back into GPU slots before it is attended
("SGLang：从前端 DSL 到 SRT 服务运行时" (oripoin.cn), section "从 2024 年论文到
今天的缓存栈", the HiCache bullet: GPU memory is the first tier, host memory
the second, and a prefix matched in a lower tier is prefetched back).  The pages fix no format; reading
taken: a host tier of rows with the pool's own row layout ([rows, Hkv, D]),
and the two moves are row gathers:
  load:  pool[slots[i]]      <- host[host_rows[i]]   (host tier -> GPU pool)
  store: host[host_rows[i]]  <- pool[slots[i]]       (GPU pool -> host tier)
Both copy bytes unchanged.  Destinations are distinct (a slot is filled
once per load, a host row written once per store); sources may repeat.
"""
import numpy as np


def load(pool, host, host_rows, slots):
    """Return a copy of pool with row slots[i] replaced by host row host_rows[i]."""
    out = np.array(pool, copy=True)
    for i in range(len(slots)):
        out[int(slots[i])] = host[int(host_rows[i])]
    return out


def store(host, pool, slots, host_rows):
    """Return a copy of host with row host_rows[i] replaced by pool row slots[i]."""
    out = np.array(host, copy=True)
    for i in range(len(slots)):
        out[int(host_rows[i])] = pool[int(slots[i])]
    return out
