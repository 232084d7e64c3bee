"""Pins for the residency oracle (oracle/residency.py): a hand-worked trace,
and invariants over random traces that any correct run of the policy keeps."""
import json
import os

import numpy as np
import pytest

from oracle import residency as R

GOLD = os.path.join(os.path.dirname(__file__), "golden", "residency_trace.json")


def test_golden_trace():
    g = json.load(open(GOLD))
    got = R.trace(g["rank"], g["n_pages"], g["batches"])
    for i, (a, e) in enumerate(zip(got, g["expected"])):
        if "error" in e:
            assert a.get("error") == e["error"], i
        else:
            assert [list(c) for c in a["copies"]] == e["copies"], i
            assert a["evicted"] == e["evicted"], i
        for k in ("rank", "page_start", "page_ids"):
            assert a[k].tolist() == e[k], (i, k)


@pytest.mark.parametrize("seed", range(6))
def test_random_traces_keep_the_invariants(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(3, 40))
    rank = rng.integers(0, 9, size=N)
    n_pages = int(rng.integers(8, 60))
    pt = R.PageTable(rank, n_pages)
    prev_res = {}
    for b in range(60):
        ids = rng.integers(-2, N + 2, size=int(rng.integers(0, 12)))
        before = {a: list(p) for a, p in pt.resident.items()}
        prev_batch = set(pt.prev)
        res = pt.admit(ids)
        need = set(int(a) for a in ids if 0 <= a < N and rank[a] > 0)
        if "error" in res:
            assert sum(rank[a] for a in need | prev_batch) > n_pages
            assert {a: list(p) for a, p in pt.resident.items()} == before
            continue
        # every needed adapter is resident with exactly its rank of pages
        for a in need:
            assert len(pt.resident[a]) == rank[a]
        # the previous batch's adapters were not evicted, kept their pages
        for a in prev_batch:
            if a in before:
                assert pt.resident.get(a) == before[a]
        # no page is used twice; used + free = all pages
        used = [p for ps in pt.resident.values() for p in ps]
        assert len(used) == len(set(used))
        assert set(used) | pt.free == set(range(n_pages)) and not (set(used) & pt.free)
        # adapters already resident keep their pages; copies cover exactly the new ones
        new = set(pt.resident) - set(before)
        for a in set(pt.resident) & set(before):
            assert pt.resident[a] == before[a]
        rows = {}
        for a, j0, p0, cnt in res["copies"]:
            assert a in new
            for q in range(cnt):
                assert pt.resident[a][j0 + q] == p0 + q
                rows.setdefault(a, set()).add(j0 + q)
        for a in new:
            assert rows.get(a, set()) == set(range(rank[a]))
        # evicted adapters are gone and were outside the protected set
        for a in res["evicted"]:
            assert a not in pt.resident and a not in need and a not in prev_batch
        rk, ps, pid = pt.tables()
        assert ps[-1] == len(pid) and np.all(np.diff(ps) == rk)


# ---------------------------------------------------------------- the library's page table

def _lib_trace(rank, n_pages, batches):
    from lora_adapter_amd import binding as B
    pt = B.PageTable(rank, n_pages)
    out = []
    for ids in batches:
        res = pt.admit(ids)
        rk, ps, pid = pt.tables()
        out.append(dict(res, rank=rk, page_start=ps, page_ids=pid))
    pt.close()
    return out


def _same(a, b):
    assert a.get("error") == b.get("error")
    if "error" not in a:
        assert [tuple(c) for c in a["copies"]] == [tuple(c) for c in b["copies"]]
        assert list(a["evicted"]) == list(b["evicted"])
    for k in ("rank", "page_start", "page_ids"):
        assert np.array_equal(a[k], b[k]), k


def test_library_page_table_matches_the_golden_trace():
    g = json.load(open(GOLD))
    for a, e in zip(_lib_trace(g["rank"], g["n_pages"], g["batches"]), g["expected"]):
        e = dict(e)
        for k in ("rank", "page_start", "page_ids"):
            e[k] = np.asarray(e[k], np.int32)
        _same(a, e)


@pytest.mark.parametrize("seed", range(8))
def test_library_page_table_matches_the_oracle(seed):
    """The host policy in the library, through the C ABI, against the oracle
    on random traces: copies, evictions and tables bit for bit."""
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(3, 200))
    rank = rng.integers(0, 17, size=N)
    n_pages = int(rng.integers(16, 400))
    batches = [rng.integers(-2, N + 2, size=int(rng.integers(0, 24))) for _ in range(80)]
    for a, b in zip(_lib_trace(rank, n_pages, batches), R.trace(rank, n_pages, batches)):
        _same(a, b)
