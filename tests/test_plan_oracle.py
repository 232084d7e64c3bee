"""Pins for the oracle's plan: an independent construction with numpy's
lexsort, the plan's invariants, the error words, and random cases."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import lora_oracle as O
from lora_adapter_amd import workloads as wl


def _lexsort_plan(ids, gates, rank, page_start, page_ids, n_pages):
    """Same contract, built from vectorised numpy: lexsort on the key columns."""
    ids = np.asarray(ids, dtype=np.int64)
    T, K = ids.shape
    flat = ids.reshape(-1)
    g = np.asarray(gates, dtype=np.float32).reshape(-1)
    N = len(rank)
    valid_id = (flat >= 0) & (flat < N)
    r = np.where(valid_id, np.asarray(rank)[np.clip(flat, 0, N - 1)], 0)
    rank_ok = (r >= 0) & (r <= O.MAX_RANK)
    cand = valid_id & rank_ok & (r > 0) & (g != 0)
    used = np.unique(flat[cand])
    bad = set()
    for a in used:
        s0, s1 = int(page_start[a]), int(page_start[a + 1])
        okp = s0 >= 0 and s1 - s0 == rank[a] and s1 <= len(page_ids)
        if okp and rank[a] > 0:
            okp = bool(np.all((page_ids[s0:s1] >= 0) & (page_ids[s0:s1] < n_pages)))
        if not okp:
            bad.add(int(a))
    act = cand & ~np.isin(flat, list(bad))
    idx = np.nonzero(act)[0]
    a = flat[idx]
    rr = np.asarray(rank)[a]
    bucket = np.where(rr <= 1, 0, np.ceil(np.log2(np.maximum(rr, 1))).astype(np.int64))
    bucket = np.where(rr > 128, 8, bucket)
    order = np.lexsort((idx, a, bucket))
    pair_tk = idx[order]
    sa = a[order]
    sb = bucket[order]
    starts = np.nonzero(np.concatenate([[True], sa[1:] != sa[:-1]]))[0] if len(sa) else np.zeros(0, int)
    seg_adapter = sa[starts]
    seg_off = np.append(starts, len(sa))
    seg_row_off = np.concatenate([[0], np.cumsum(np.asarray(rank)[seg_adapter])])
    segb = sb[starts]
    bso = [int(np.searchsorted(segb, b, side="left")) for b in range(10)]
    u_off = np.concatenate([[0], np.cumsum(np.asarray(rank)[sa])])
    slot_pos = np.full(T * K, -1)
    slot_pos[pair_tk] = np.arange(len(pair_tk))
    err = 0
    if np.any((flat < -1) | (flat >= N)):
        err |= O.ERR_BAD_ID
    if np.any(valid_id & ~rank_ok):
        err |= O.ERR_BAD_RANK
    if bad:
        err |= O.ERR_BAD_POOL
    return dict(pair_tk=pair_tk, pair_adapter=sa, seg_adapter=seg_adapter, seg_off=seg_off, seg_row_off=seg_row_off,
                bucket_seg_off=np.asarray(bso), u_off=u_off, slot_pos=slot_pos, err=err)


def _check_same(p, q):
    for k in ("pair_tk", "pair_adapter", "seg_adapter", "seg_off", "seg_row_off", "bucket_seg_off",
              "u_off", "slot_pos"):
        np.testing.assert_array_equal(p[k], np.asarray(q[k], dtype=np.int64), err_msg=k)
    assert p["header"][O.H_ERR] == q["err"]


def _check_invariants(p, ids, gates, rank):
    ids = np.asarray(ids)
    T, K = ids.shape
    h = p["header"]
    P, S = int(h[O.H_P]), int(h[O.H_S])
    assert len(p["pair_tk"]) == P and len(p["seg_adapter"]) == S
    assert len(set(p["pair_tk"].tolist())) == P
    assert np.all(np.diff(p["seg_off"]) > 0) if S else True
    for s in range(S):
        a = p["seg_adapter"][s]
        members = p["pair_tk"][p["seg_off"][s]:p["seg_off"][s + 1]]
        assert np.all(ids.reshape(-1)[members] == a)
        assert np.all(np.diff(members) > 0)          # stable within a segment
    buckets = [O.rank_bucket(int(rank[a])) for a in p["seg_adapter"]]
    assert buckets == sorted(buckets)
    assert len(set(p["seg_adapter"].tolist())) == S  # one segment per adapter
    assert p["u_off"][-1] == h[O.H_RPAIRS] and p["seg_row_off"][-1] == h[O.H_RUSED]
    for pos, tk in enumerate(p["pair_tk"]):
        assert p["slot_pos"][tk] == pos
    assert np.sum(p["slot_pos"] >= 0) == P


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_plan_matches_lexsort_on_workloads(cfg):
    w = wl.small(cfg)
    p = O.plan_workload(w)
    q = _lexsort_plan(w.ids, w.gates, w.rank, w.page_start, w.page_ids, w.n_pages)
    _check_same(p, q)
    _check_invariants(p, w.ids, w.gates, w.rank)


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_plan_full_size_routing(cfg):
    # full-size routing and ranks without drawing the big tensors
    rng = wl.streams(cfg)
    if cfg == 2:
        N, T = 64, 64
        rank = np.full(N, 16, np.int32)
        ids = rng["ids"].integers(0, N, size=(T, 1)).astype(np.int32)
        gates = np.ones((T, 1), np.float32)
    elif cfg == 3:
        N, T = 1024, 256
        rank = rng["ranks"].choice(np.array([8, 16, 32, 64, 128]), size=N).astype(np.int32)
        ids = wl.zipf_ids(rng["ids"], T, N).reshape(T, 1)
        gates = np.ones((T, 1), np.float32)
    else:
        N, T = 2048, 512
        rank = np.clip(rng["ranks"].geometric(0.25, size=N), 2, 16).astype(np.int32)
        ids, gates = wl.top2_softmax(rng["gates"], T, N)
    ps = np.concatenate([[0], np.cumsum(rank)]).astype(np.int32)
    pid = np.random.default_rng(0).permutation(int(rank.sum()) + 3)[:int(rank.sum())].astype(np.int32)
    p = O.plan(ids, gates, rank, ps, pid, int(rank.sum()) + 3)
    q = _lexsort_plan(ids, gates, rank, ps, pid, int(rank.sum()) + 3)
    _check_same(p, q)
    _check_invariants(p, ids, gates, rank)


def test_plan_error_words():
    rank = np.array([2, 0, 3, 2000, 1], np.int32)
    ps = np.array([0, 2, 2, 5, 5, 6], np.int32)        # adapter 3 claims 0 pages for rank 2000
    pid = np.array([0, 1, 2, 3, 4, 99], np.int32)      # adapter 4's page is out of range
    n_pages = 8
    ids = np.array([[0], [1], [2], [3], [4], [-1], [-2], [5]], np.int32)
    gates = np.ones((8, 1), np.float32)
    p = O.plan(ids, gates, rank, ps, pid, n_pages)
    assert p["header"][O.H_ERR] == O.ERR_BAD_ID | O.ERR_BAD_RANK | O.ERR_BAD_POOL
    # only adapters 0 and 2 survive: tokens 0 and 2
    assert sorted(p["pair_tk"].tolist()) == [0, 2]
    q = _lexsort_plan(ids, gates, rank, ps, pid, n_pages)
    _check_same(p, q)


def test_plan_empty_and_all_inactive():
    rank = np.array([4], np.int32)
    ps = np.array([0, 4], np.int32)
    pid = np.arange(4, dtype=np.int32)
    p = O.plan(np.zeros((0, 2), np.int32), np.zeros((0, 2), np.float32), rank, ps, pid, 4)
    assert p["header"][O.H_P] == 0 and p["header"][O.H_S] == 0
    assert p["bucket_seg_off"].tolist() == [0] * 10
    p = O.plan(np.full((5, 1), -1, np.int32), np.ones((5, 1), np.float32), rank, ps, pid, 4)
    assert p["header"][O.H_P] == 0 and p["slot_pos"].tolist() == [-1] * 5


@st.composite
def _plan_case(draw):
    N = draw(st.integers(1, 9))
    rank = np.asarray(draw(st.lists(st.sampled_from([0, 1, 2, 3, 4, 5, 8, 9, 16, 17, 33, 64, 65, 128, 129, 130]),
                                    min_size=N, max_size=N)), np.int32)
    T = draw(st.integers(0, 40))
    K = draw(st.integers(1, 3))
    ids = np.asarray(draw(st.lists(st.integers(-1, N - 1), min_size=T * K, max_size=T * K)),
                     np.int32).reshape(T, K)
    gates = np.asarray(draw(st.lists(st.sampled_from([0.0, -0.0, 1.0, 0.5, -2.0]),
                                     min_size=T * K, max_size=T * K)), np.float32).reshape(T, K)
    return ids, gates, rank


@settings(max_examples=150, deadline=None)
@given(_plan_case())
def test_plan_random(case):
    ids, gates, rank = case
    ps = np.concatenate([[0], np.cumsum(rank)]).astype(np.int32)
    n_pages = int(rank.sum()) + 2
    pid = np.random.default_rng(1).permutation(n_pages)[:int(rank.sum())].astype(np.int32)
    p = O.plan(ids, gates, rank, ps, pid, n_pages)
    q = _lexsort_plan(ids, gates, rank, ps, pid, n_pages)
    _check_same(p, q)
    _check_invariants(p, ids, gates, rank)
