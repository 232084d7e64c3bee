"""CPU oracle for the adapter pool's residency policy (page allocation and
eviction).

TEST INFRASTRUCTURE.  Only the tests may import or call this module; it
shares no code with the library.

The S-LoRA page ("S-LoRA：一个GPU运行数千大模型成为可能", section 批处理, last
paragraph: every adapter is kept in host memory and only the adapters of the
running batch are loaded to the GPU; section 内存管理 and Unified Paging:
adapters of different ranks share one pool of pages, one page per rank row,
non-contiguous) fixes what the pool must hold, not how victims are chosen.
The plainest policy that the rest supports is written out here, step by step:

  * Admitting a batch: the needed adapters are its valid ids (0 <= a < N,
    rank > 0), each once, in ascending id order.  The protected set is the
    needed adapters plus those of the previous admitted batch (its kernels may
    still run while this batch's pages are copied in).  If the protected set's
    ranks add up to more than the pool's pages, the batch is refused and
    nothing changes.
  * Every needed adapter is stamped with this batch's index (its last use).
  * Each needed adapter that is not resident, in ascending id order, gets
    rank pages: while fewer pages are free, the resident adapter outside the
    protected set with the smallest (last use, id) is evicted and its pages
    freed; then the lowest-numbered free pages are taken, rank row j on the
    j-th of them.  Its rows are copied in maximal runs of consecutive pages.
  * The tables a batch runs with list each resident adapter's rank, the
    prefix sums of those ranks, and the pages in adapter order; an adapter
    that is not resident has rank 0 there.
"""
from __future__ import annotations

import numpy as np


class PageTable:
    def __init__(self, rank, n_pages: int):
        self.rank = [int(r) for r in rank]
        self.n_pages = int(n_pages)
        self.resident = {}            # adapter -> list of pages, rank row order
        self.last_use = {}
        self.free = set(range(self.n_pages))
        self.batch = 0                # index of the next admitted batch
        self.prev = set()             # adapters of the previous admitted batch

    def admit(self, ids):
        """Returns {"copies": [(adapter, first rank row, first page, rows)],
        "evicted": [adapters in eviction order]} or {"error": "capacity"}."""
        N = len(self.rank)
        need = sorted(set(int(a) for a in np.asarray(ids).reshape(-1).tolist()
                          if 0 <= int(a) < N and self.rank[int(a)] > 0))
        protected = set(need) | self.prev
        if sum(self.rank[a] for a in protected) > self.n_pages:
            return {"error": "capacity"}
        for a in need:
            self.last_use[a] = self.batch
        copies, evicted = [], []
        for a in need:
            if a in self.resident:
                continue
            r = self.rank[a]
            while len(self.free) < r:
                cands = [(self.last_use[v], v) for v in self.resident if v not in protected]
                victim = min(cands)[1]
                self.free |= set(self.resident.pop(victim))
                evicted.append(victim)
            pages = sorted(self.free)[:r]
            self.free -= set(pages)
            self.resident[a] = pages
            j = 0
            while j < r:
                k = j
                while k + 1 < r and pages[k + 1] == pages[k] + 1:
                    k += 1
                copies.append((a, j, pages[j], k - j + 1))
                j = k + 1
        self.prev = set(need)
        self.batch += 1
        return {"copies": copies, "evicted": evicted}

    def tables(self):
        """(rank, page_start, page_ids) of the current residency, int32."""
        N = len(self.rank)
        rk = [self.rank[a] if a in self.resident else 0 for a in range(N)]
        ps = [0]
        for r in rk:
            ps.append(ps[-1] + r)
        pid = [p for a in range(N) if a in self.resident for p in self.resident[a]]
        i32 = lambda v: np.asarray(v, dtype=np.int32)
        return i32(rk), i32(ps), i32(pid)


def trace(rank, n_pages, batches):
    """Admit each batch in turn; per batch the admit result and the tables."""
    pt = PageTable(rank, n_pages)
    out = []
    for ids in batches:
        res = pt.admit(ids)
        rk, ps, pid = pt.tables()
        out.append(dict(res, rank=rk, page_start=ps, page_ids=pid))
    return out
