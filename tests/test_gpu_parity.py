"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on
the same seeded inputs.

Bars: the plan is integer and compared bit for bit; floating outputs satisfy
max|gpu - oracle| / max|oracle| <= 1e-5 (fp32 inputs) or 1e-2 (bf16 inputs,
fp32 accumulation).  Bit-identities the method fixes are checked on the GPU
alone: rows whose slots are all inactive equal a base-only run bit for bit,
moving adapters to other pages changes nothing, and repeated runs agree.
"""
import functools

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from lora_adapter_amd import binding as B
from lora_adapter_amd import device as D
from lora_adapter_amd import workloads as wl
from oracle import lora_oracle as O

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()   # fails loudly if the HIP library is missing


@functools.lru_cache(None)
def small(i):
    return wl.small(i)


@functools.lru_cache(None)
def full(i):
    return wl.config(i)


def rel_err(gpu, ref):
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-300))


def run(w, **kw):
    L = D.DeviceLayer(w, **kw)
    L.run_plan()
    L.run_apply()
    torch.cuda.synchronize()
    return L


def assert_plan_equal(gpu, ref):
    np.testing.assert_array_equal(gpu["header"][:8], ref["header"][:8])
    for k in ("pair_tk", "seg_adapter", "seg_off", "seg_row_off", "bucket_seg_off", "u_off", "slot_pos",
              "pair_adapter"):
        np.testing.assert_array_equal(gpu[k], ref[k], err_msg=k)


# ---------------------------------------------------------------- plan

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_plan_small(cfg):
    w = small(cfg)
    L = D.DeviceLayer(w)
    L.run_plan()
    torch.cuda.synchronize()
    assert_plan_equal(L.read_plan(), O.plan_workload(w))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_plan_full(cfg):
    w = full(cfg)
    L = D.DeviceLayer(w)
    L.run_plan()
    torch.cuda.synchronize()
    assert_plan_equal(L.read_plan(), O.plan_workload(w))


def _tiny_pool_workload(N, T, K, rank, ids, gates, d=64, seed=0):
    return wl.build("tiny", seed, "bf16", T, K, d, d, np.asarray(rank, np.int32), ids, gates,
                    x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02)


def test_plan_errors_match_oracle():
    rank = np.array([2, 0, 3, 2000, 1], np.int32)
    ids = np.array([[0], [1], [2], [3], [4], [-1], [-2], [5]], np.int32)
    gates = np.ones((8, 1), np.float32)
    w = _tiny_pool_workload(5, 8, 1, [2, 0, 3, 0, 1], ids, gates)
    w.rank = rank                                   # adapter 3 claims rank 2000
    w.page_ids = w.page_ids.copy()
    w.page_ids[-1] = 10 ** 6                       # adapter 4's page out of range
    L = D.DeviceLayer(w, max_rank=4)
    L.run_plan()
    torch.cuda.synchronize()
    ref = O.plan(w.ids, w.gates, w.rank, w.page_start, w.page_ids, w.n_pages)
    got = L.read_plan()
    assert got["header"][B.PH_ERR] == B.DEVERR_BAD_ID | B.DEVERR_BAD_RANK | B.DEVERR_BAD_POOL
    assert_plan_equal(got, ref)


def test_plan_bad_page_ids_large_table():
    """A page table too large to copy to LDS (its ids are checked row by row
    after the segment order) with out-of-range page ids in two used
    adapters: both are dropped and BAD_POOL is set, as in the oracle.  The
    same batch through lora_forward (plan built inside the decode GEMM launch,
    per-slot shrink) gives the same plan and the oracle's Y."""
    rng = np.random.default_rng(21)
    N, T, K = 300, 96, 1
    rank = np.full(N, 128, np.int32)                # 38400 page ids
    ids = rng.integers(0, N, size=(T, K)).astype(np.int32)
    gates = np.ones((T, K), np.float32)
    w = wl.build("bigtable", 21, "bf16", T, K, 256, 256, rank, ids, gates,
                 x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02)
    used = np.unique(ids)
    w.page_ids = w.page_ids.copy()
    w.page_ids[w.page_start[used[0]] + 5] = -3
    w.page_ids[w.page_start[used[1]] + 127] = w.n_pages
    ref = O.plan(w.ids, w.gates, w.rank, w.page_start, w.page_ids, w.n_pages)
    L = D.DeviceLayer(w, max_rank=128)
    L.run_plan()
    torch.cuda.synchronize()
    got = L.read_plan()
    assert got["header"][B.PH_ERR] == B.DEVERR_BAD_POOL
    assert_plan_equal(got, ref)
    L.plan.zero_()
    B.lora_forward(L.ids, L.gates, L.T, L.K, L.X, L.W_t, L.Y, L.keep_mask, L.keep_scale, L.pool,
                   L.plan, L.ws)
    torch.cuda.synchronize()
    got = L.read_plan()
    assert got["header"][B.PH_ERR] == B.DEVERR_BAD_POOL
    assert_plan_equal(got, ref)
    err = rel_err(D.as_f64(L.Y_host()), O.apply_workload(w))
    assert err <= TOL["bf16"], err


def test_plan_large_pool_uses_global_counters():
    rng = np.random.default_rng(11)
    N, T, K = 10000, 3000, 2                       # N above the LDS counter limit
    rank = rng.integers(0, 5, size=N).astype(np.int32)
    ids = rng.integers(-1, N, size=(T, K)).astype(np.int32)
    gates = rng.choice(np.array([0.0, 1.0, -0.5], np.float32), size=(T, K))
    w = _tiny_pool_workload(N, T, K, rank, ids, gates)
    L = D.DeviceLayer(w)
    L.run_plan()
    torch.cuda.synchronize()
    assert_plan_equal(L.read_plan(), O.plan_workload(w))


def test_plan_empty_batch():
    w = _tiny_pool_workload(3, 0, 2, [1, 2, 3], np.zeros((0, 2), np.int32), np.zeros((0, 2), np.float32))
    L = D.DeviceLayer(w)
    L.run_plan()
    L.run_apply()
    torch.cuda.synchronize()
    got = L.read_plan()
    assert got["header"][B.PH_PAIRS] == 0 and got["header"][B.PH_SEGS] == 0
    assert got["bucket_seg_off"].tolist() == [0] * 10


# ---------------------------------------------------------------- apply

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_apply_small(cfg):
    w = small(cfg)
    L = run(w)
    assert L.read_plan()["header"][B.PH_ERR] == 0
    err = rel_err(D.as_f64(L.Y_host()), O.apply_workload(w))
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("d_out", [8192, 8320])
def test_apply_fused_epilogue_path(d_out):
    # enough output tiles that the expand runs inside the GEMM epilogue; the
    # last partial round of tiles runs as half tiles, and with d_out = 8320
    # some second halves lie wholly past the last column
    w = wl.config(4, T=2100, d_in=512, d_out=d_out, seed=77)
    L = run(w)
    err = rel_err(D.as_f64(L.Y_host()), O.apply_workload(w))
    assert err <= TOL["bf16"], err


SHORT_K_CASES = {
    # 256x256 fused tiles with 1, 2 and 3 K tiles of 64 (prologue, loop and
    # the copies clamped past the end)
    "fused_k64": lambda: wl.config(4, T=2100, d_in=64, d_out=8192, seed=71),
    "fused_k128": lambda: wl.config(4, T=2100, d_in=128, d_out=8192, seed=72),
    "fused_k192": lambda: wl.config(4, T=2100, d_in=192, d_out=8192, seed=73),
    # stream-K 256x128 pieces of one to a few K tiles
    "streamk_k2048": lambda: wl.config(3, T=300, d_in=2048, d_out=2048, n_adapters=64, seed=74),
    # decode tile whose last K chunk holds one 64-wide group
    "decode_k576": lambda: wl.config(2, T=64, d_in=576, d_out=640, seed=75),
}


@pytest.mark.parametrize("case", sorted(SHORT_K_CASES))
def test_apply_short_k(case):
    w = SHORT_K_CASES[case]()
    L = run(w)
    assert L.read_plan()["header"][B.PH_ERR] == 0
    err = rel_err(D.as_f64(L.Y_host()), O.apply_workload(w))
    assert err <= TOL[w.dtype], err


def test_apply_mixed_ranks_above_bucket_edges():
    rng = np.random.default_rng(5)
    N, T, K = 9, 130, 2
    rank = np.array([1, 2, 3, 7, 16, 17, 64, 129, 200], np.int32)
    ids = rng.integers(-1, N, size=(T, K)).astype(np.int32)
    gates = rng.standard_normal((T, K)).astype(np.float32)
    gates[rng.random((T, K)) < 0.1] = 0
    w = wl.build("mixed", 9, "bf16", T, K, 256, 384, rank, ids, gates,
                 x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02,
                 scale=rng.uniform(0.5, 2, N).astype(np.float32))
    L = run(w)
    assert_plan_equal(L.read_plan(), O.plan_workload(w))
    err = rel_err(D.as_f64(L.Y_host()), O.apply_workload(w))
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_apply_full(cfg):
    w = full(cfg)
    L = run(w)
    assert L.read_plan()["header"][B.PH_ERR] == 0
    err = rel_err(D.as_f64(L.Y_host()), O.apply_workload(w))
    assert err <= TOL[w.dtype], err


def test_apply_full_prefill_sampled_rows():
    w = full(4)
    L = run(w)
    lens = np.cumsum(w.meta["segment_lengths"])
    rng = np.random.default_rng(0)
    rows = sorted(set(rng.choice(w.T, 48, replace=False).tolist()
                      + [0, w.T - 1] + [int(x) for x in lens[:-1]] + [int(x) - 1 for x in lens[:-1]]))
    ref = O.apply_workload(w, rows=rows)
    got = D.as_f64(L.Y_host())[rows]
    err = rel_err(got, ref)
    assert err <= TOL["bf16"], err


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("cfg", ["small2", "dec3"])
def test_forward_all_inactive_equals_base_only(cfg):
    """lora_forward on a batch whose slots are all inactive (decode path:
    the GEMM tiles, then per-slot shrink parts that end at once): Y equals
    the base-only product bit for bit and the plan is empty."""
    w = small(2) if cfg == "small2" else FORWARD_CASES[cfg]()
    L = run(w)
    Yb = _base_only(L)
    L.ids.fill_(-1)
    L.Y.zero_()
    L.ws.zero_()
    B.lora_forward(L.ids, L.gates, L.T, L.K, L.X, L.W_t, L.Y, L.keep_mask, L.keep_scale,
                   L.pool, L.plan, L.ws)
    torch.cuda.synchronize()
    hdr = L.read_plan()["header"]
    assert hdr[B.PH_PAIRS] == 0 and hdr[B.PH_ERR] == 0
    assert np.array_equal(L.Y_host(), Yb)


def _base_only(L):
    ids_saved = L.ids.clone()
    L.ids.fill_(-1)
    Yb = torch.empty_like(L.Y)
    L.run_plan()
    L.run_apply(Y=Yb)
    torch.cuda.synchronize()
    L.ids.copy_(ids_saved)
    L.run_plan()
    torch.cuda.synchronize()
    return D.to_host(Yb)


@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_inactive_rows_equal_base_only_bit_for_bit(cfg):
    w = small(cfg)
    w2 = wl.config(cfg, T=w.T, d_in=w.d_in, d_out=w.d_out, n_adapters=w.n_adapters if cfg != 1 else None,
                   seed=w.meta["seed"])
    w2.gates = w2.gates.copy(); w2.ids = w2.ids.copy()
    w2.gates[::3] = 0.0
    w2.ids[1::5] = -1
    L = run(w2)
    Y = L.Y_host()
    Yb = _base_only(L)
    inactive = [t for t in range(w2.T)
                if all(w2.ids[t, k] < 0 or w2.gates[t, k] == 0 or w2.rank[w2.ids[t, k]] == 0
                       for k in range(w2.K))]
    assert len(inactive) > 0
    assert np.array_equal(Y[inactive], Yb[inactive])
    active = [t for t in range(w2.T) if t not in inactive]
    assert not np.array_equal(Y[active], Yb[active])


def test_moving_pages_changes_nothing():
    w = small(3)
    L1 = run(w)
    # same factors at other pages: permute the pool's rows and remap page ids
    rng = np.random.default_rng(4)
    perm = rng.permutation(w.n_pages)
    inv = np.argsort(perm)
    w2 = wl.Workload(**{**w.__dict__})
    w2.a_pages = w.a_pages[perm]
    w2.b_pages = w.b_pages[perm]
    w2.page_ids = inv[w.page_ids].astype(np.int32)
    L2 = run(w2)
    assert np.array_equal(L1.Y_host(), L2.Y_host())


@pytest.mark.parametrize("cfg", [2, 4])
def test_repeated_runs_are_bitwise_identical(cfg):
    w = small(cfg)
    L = run(w)
    Y1 = L.Y_host().copy()
    for _ in range(3):
        L.run_plan()
        L.run_apply()
    torch.cuda.synchronize()
    assert np.array_equal(Y1, L.Y_host())


@pytest.mark.parametrize("cfg", ["small2", "small3", "small5", "full2"])
def test_split_and_fused_entry_points_agree(cfg):
    """lora_apply runs the decode shrink inside the decode GEMM launch; the
    separate entry points (lora_shrink, lora_base_gemm, lora_expand_epilogue)
    run the same arithmetic in three launches: U and Y agree bit for bit."""
    w = small(int(cfg[-1])) if cfg.startswith("small") else full(int(cfg[-1]))
    L = run(w)
    U1, Y1 = L.U().copy(), L.Y_host().copy()
    L.ws.zero_()
    L.Y.zero_()
    L.run_shrink()
    B.lora_base_gemm(L.X, L.W_t, L.Y, L.T, L.K, L.pool, L.plan, L.ws)
    B.lora_expand_epilogue(L.X, L.W_t, L.Y, L.T, L.K, L.pool, L.plan, L.ws)
    torch.cuda.synchronize()
    assert np.array_equal(U1, L.U())
    assert np.array_equal(Y1, L.Y_host())


def _mixed_decode():
    """Decode-sized batch (T <= 128, two slots) with empty slots, zero gates,
    ranks across bucket edges and above the MFMA range, per-adapter scales."""
    rng = np.random.default_rng(15)
    N, T, K = 9, 100, 2
    rank = np.array([1, 2, 3, 7, 16, 17, 64, 129, 200], np.int32)
    ids = rng.integers(-1, N, size=(T, K)).astype(np.int32)
    gates = rng.standard_normal((T, K)).astype(np.float32)
    gates[rng.random((T, K)) < 0.1] = 0
    return wl.build("mixed-decode", 15, "bf16", T, K, 4608, 384, rank, ids, gates,
                    x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02,
                    scale=rng.uniform(0.5, 2, N).astype(np.float32))


FORWARD_CASES = {
    # decode shapes with a keep mask, d_in above one 4096-element block, and
    # ranks up to 128 over many adapters
    "dec4": lambda: wl.config(4, T=96, d_in=4608, d_out=704, seed=204),
    "dec3": lambda: wl.config(3, T=128, d_in=512, d_out=640, n_adapters=300, seed=203),
    "decmix": _mixed_decode,
}


@pytest.mark.parametrize("cfg", ["small1", "small2", "small3", "small4", "small5", "full2", "full3",
                                 "full5", "dec4", "dec3", "decmix"])
def test_forward_matches_plan_then_apply(cfg):
    """lora_forward in two launches (decode: GEMM + per-slot shrink, then
    epilogue + plan; stream-K: GEMM + plan, then shrink and epilogue): the
    plan, U and Y equal those of lora_plan then lora_apply bit for bit.  The same call captured in a graph is replayed three times, with
    eager work and synchronisation in between, and every replay gives the
    same Y."""
    if cfg in FORWARD_CASES:
        w = FORWARD_CASES[cfg]()
    else:
        w = small(int(cfg[-1])) if cfg.startswith("small") else full(int(cfg[-1]))
    L = run(w)
    P1, U1, Y1 = L.read_plan(), L.U().copy(), L.Y_host().copy()
    if cfg in FORWARD_CASES:
        assert_plan_equal(P1, O.plan_workload(w))
        err = rel_err(D.as_f64(Y1), O.apply_workload(w))
        assert err <= TOL[w.dtype], err

    def fwd():
        B.lora_forward(L.ids, L.gates, L.T, L.K, L.X, L.W_t, L.Y, L.keep_mask, L.keep_scale,
                       L.pool, L.plan, L.ws)

    L.ws.zero_()
    L.Y.zero_()
    L.plan.zero_()
    fwd()
    torch.cuda.synchronize()
    assert_plan_equal(L.read_plan(), P1)
    assert np.array_equal(U1, L.U())
    assert np.array_equal(Y1, L.Y_host())
    # the decode path's plan has no decode-shrink wave records: a shrink over
    # it finds each wave's start by search and gives the same U
    L.ws.zero_()
    L.run_shrink()
    torch.cuda.synchronize()
    assert np.array_equal(U1, L.U())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    torch.cuda.synchronize()
    for _ in range(3):
        L.Y.zero_()
        L.ws.zero_()
        L.plan.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_plan_equal(L.read_plan(), P1)
        assert np.array_equal(Y1, L.Y_host())


def test_u_capacity_error_skips_lora_and_flags():
    w = small(2)
    L = D.DeviceLayer(w, max_rank=1)          # U room for one rank row per slot only
    L.run_plan()
    L.run_apply()
    torch.cuda.synchronize()
    h = L.read_plan()["header"]
    assert h[B.PH_ERR] & B.DEVERR_CAPACITY
    base = D.as_f64(L.Y_host())
    ref = D.as_f64(w.X) @ D.as_f64(w.W_t).T
    assert rel_err(base, ref) <= TOL["bf16"]


# ---------------------------------------------------------------- merge

def _ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("which", ["small1", "small5", "full5"])
def test_merge_unmerge_and_switch(which):
    w = {"small1": lambda: small(1), "small5": lambda: small(5), "full5": lambda: full(5)}[which]()
    ids = w.merge_ids if w.merge_ids is not None else np.arange(min(4, w.n_adapters), dtype=np.int32)
    co = np.ones(len(ids), np.float32)
    L = D.DeviceLayer(w)
    W = L.W_t.clone()
    L.run_merge(W, ids, co)
    torch.cuda.synchronize()
    Wm = D.to_host(W)
    ref = O.merge_workload(w, ids=ids, coeffs=co)
    assert rel_err(D.as_f64(Wm), ref) <= TOL[w.dtype]
    # unmerge restores W to within one rounding of each step
    L.run_merge(W, ids, -co)
    torch.cuda.synchronize()
    W0, W2 = D.as_f64(w.W_t), D.as_f64(D.to_host(W))
    if w.dtype == "bf16":
        bound = _ulp_bf16(np.maximum(np.abs(W0), np.abs(D.as_f64(Wm)))) * 1.01
    else:
        bound = np.spacing(np.maximum(np.abs(W0), np.abs(D.as_f64(Wm))).astype(np.float32)).astype(np.float64) * 2.02
    assert np.all(np.abs(W2 - W0) <= bound + 1e-30)
    # fused switch from the merged state: -old, +new in one call
    new = np.array([(int(i) + 1) % w.n_adapters for i in ids[:2]], np.int32)
    sw_ids = np.concatenate([ids, new]).astype(np.int32)
    sw_co = np.concatenate([-co, np.ones(2, np.float32)])
    W3 = torch.from_numpy(np.ascontiguousarray(Wm).view(np.int16) if Wm.dtype == np.uint16 else Wm)
    W3 = W3.to("cuda")
    if Wm.dtype == np.uint16:
        W3 = W3.view(torch.bfloat16)
    L.run_merge(W3, sw_ids, sw_co)
    torch.cuda.synchronize()
    ref3 = O.merge_workload(w, W_t=Wm, ids=sw_ids, coeffs=sw_co)
    assert rel_err(D.as_f64(D.to_host(W3)), ref3) <= TOL[w.dtype]


def _merge_abs_delta(w, ids, co):
    """sum_i |c_i s_i| . (|A_i| |B_i|)^T in float64: the scale of the float32
    rounding the merged delta may carry."""
    out = np.zeros((w.d_out, w.d_in))
    for a, c in zip(ids.tolist(), co.tolist()):
        if not (0 <= a < w.n_adapters) or int(w.rank[a]) == 0:
            continue
        A, Bf = O.factors(a, w.rank, w.page_start, w.page_ids, w.a_pages, w.b_pages)
        out += abs(float(c) * float(w.scale[a])) * (np.abs(A) @ np.abs(Bf)).T
    return out


@pytest.mark.parametrize("which", ["small2", "small3", "small5", "full5"])
def test_merge_elementwise_bound(which):
    """Every merged element is the exact W + delta rounded once to bf16, up to
    the float32 summation of the delta: |gpu - ref| <= ulp(ref)/2 (one
    rounding) + 1e-5 sum|c s A B| (float32 products and sums)."""
    w = {"small2": lambda: small(2), "small3": lambda: small(3), "small5": lambda: small(5),
         "full5": lambda: full(5)}[which]()
    if w.merge_ids is not None:
        ids = np.asarray(w.merge_ids, np.int32)
    else:
        rng = np.random.default_rng(11)
        ids = rng.integers(0, w.n_adapters, size=6).astype(np.int32)
    co = np.where(np.arange(len(ids)) % 2 == 0, 1.0, -0.75).astype(np.float32)
    L = D.DeviceLayer(w)
    W = L.W_t.clone()
    L.run_merge(W, ids, co)
    torch.cuda.synchronize()
    got = D.as_f64(D.to_host(W))
    ref = O.merge_workload(w, ids=ids, coeffs=co)
    bound = 0.5 * _ulp_bf16(np.abs(ref) * 1.01) + 1e-5 * _merge_abs_delta(w, ids, co) + 1e-30
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:4])


@pytest.mark.parametrize("which", [3, 2])
def test_merge_long_list_with_duplicates(which):
    """300 entries (two groups of list reads), repeated ids and signed
    coefficients, more listed rank rows than one LDS list holds (workload 3:
    d_out 1344, the float32-FMA kernel; workload 2: 512 x 768, the MFMA
    kernel's chunked path)."""
    w = small(which)
    rng = np.random.default_rng(3)
    ids = rng.integers(0, w.n_adapters, size=300).astype(np.int32)
    ids[::7] = ids[0]                                  # many repeats of one adapter
    co = rng.uniform(-1.0, 1.0, size=300).astype(np.float32)
    assert int(w.rank[ids[:256]].sum()) > 1024
    L = D.DeviceLayer(w)
    W = L.W_t.clone()
    L.run_merge(W, ids, co)
    torch.cuda.synchronize()
    ref = O.merge_workload(w, ids=ids, coeffs=co)
    assert rel_err(D.as_f64(D.to_host(W)), ref) <= TOL[w.dtype]


def test_merged_weight_base_matches_apply():
    w = small(2)
    a = int(w.ids[0, 0])
    g = np.float32(0.75)
    w1 = wl.Workload(**{**w.__dict__})
    w1.ids = np.full((w.T, 1), a, np.int32)
    w1.gates = np.full((w.T, 1), g, np.float32)
    L = run(w1)
    Y_apply = D.as_f64(L.Y_host())
    W = L.W_t.clone()
    L.run_merge(W, [a], [g])
    Yb = torch.empty_like(L.Y)
    L.ids.fill_(-1)
    L.run_plan()
    L.run_apply(Y=Yb, W_t=W)
    torch.cuda.synchronize()
    assert rel_err(D.as_f64(D.to_host(Yb)), Y_apply) <= TOL["bf16"]


# ---------------------------------------------------------------- grads

def _check_grads(w, L):
    dA, dB, gws = L.grad_buffers()
    L.run_grad(dA, dB, gws)
    torch.cuda.synchronize()
    g = O.grad_workload(w)
    rA, rB = O.grad_pages(g, w.rank, w.page_start, w.page_ids, w.n_pages, w.d_in, w.d_out)
    gA, gB = dA.cpu().numpy().astype(np.float64), dB.cpu().numpy().astype(np.float64)
    used = ~np.isnan(rA[:, 0])
    assert np.all(np.isnan(gA[~used])) and np.all(np.isnan(gB[~used]))   # other pages untouched
    assert rel_err(gA[used], rA[used]) <= TOL[w.dtype]
    assert rel_err(gB[used], rB[used]) <= TOL[w.dtype]


def test_grads_small():
    w = small(4)
    _check_grads(w, run(w))


def test_grads_multi_adapter_top2():
    w = small(5)
    w = wl.Workload(**{**w.__dict__})
    w.dY = wl._normal(np.random.default_rng(3), (w.T, w.d_out), 1.0, "bf16")
    _check_grads(w, run(w))


def test_grads_mfma_mixed_ranks_top2():
    """A batch large enough for the MFMA outer products (T*K >= 2048): two
    slots per token, empty slots and zero gates, ranks below and above the
    16-row blocks, a keep mask."""
    rng = np.random.default_rng(23)
    N, T, K = 12, 1100, 2
    rank = np.array([3, 16, 17, 40, 64, 5, 8, 1, 33, 16, 2, 24], np.int32)
    ids = rng.integers(-1, N, size=(T, K)).astype(np.int32)
    gates = rng.standard_normal((T, K)).astype(np.float32)
    gates[rng.random((T, K)) < 0.1] = 0
    w = wl.build("grad-mfma", 23, "bf16", T, K, 512, 768, rank, ids, gates,
                 x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02, keep_p=0.9, with_dY=True,
                 scale=rng.uniform(0.5, 2, N).astype(np.float32))
    _check_grads(w, run(w))


def test_grads_full_prefill():
    w = full(4)
    _check_grads(w, run(w))
