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


FUSED_RUN_CASES = {
    # contiguous segments of ranks 8 and 16 whose U runs start 16-byte
    # aligned: 32-row blocks inside a segment load U in 16-byte pieces
    "aligned_r8_r16": ((8, 16, 8, 16), (512, 544, 480, 564)),
    # a rank-5 segment of odd length first, so the rank-8 and rank-16 runs
    # after it start misaligned (element-wise loads), a rank-12 segment (no
    # run form) and segment edges inside blocks
    "misaligned_r5_r12": ((5, 8, 12, 16, 16), (333, 421, 389, 517, 440)),
}


@pytest.mark.parametrize("case", sorted(FUSED_RUN_CASES))
def test_apply_fused_u_runs(case):
    """The fused epilogue's U loads: a block of consecutive pairs of one
    rank-8 or rank-16 adapter whose U starts 16-byte aligned is loaded in
    16-byte pieces and shuffled to its lanes; other blocks element by
    element.  Every row of Y against the oracle."""
    ranks, lens = FUSED_RUN_CASES[case]
    rank = np.asarray(ranks, np.int32)
    T = int(sum(lens))
    ids = np.repeat(np.arange(len(rank), dtype=np.int32), lens).reshape(T, 1)
    gates = np.ones((T, 1), np.float32)
    w = wl.build("fused-u-runs-" + case, 97, "bf16", T, 1, 256, 8192, rank, ids, gates,
                 x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02)
    # 9 x 32 tiles of 256 x 256: the fused-epilogue form
    assert T == 2100 and ((T + 255) // 256) * (8192 // 256) >= 256
    L = run(w)
    assert L.read_plan()["header"][B.PH_ERR] == 0
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


@pytest.mark.parametrize("masked", [False, True])
def test_apply_rank_bucket_edges(masked):
    """Ranks at and around every rank-bucket edge of the plan (1, 2 | 3, 4 |
    5, 8 | 9, 16 | 17, 33), two slots per token, with and without a keep mask:
    plan, Y and every pair's U against the oracle."""
    rng = np.random.default_rng(91 + masked)
    rank = np.array([1, 2, 3, 4, 5, 8, 9, 16, 17, 33], np.int32)
    N, T, K = len(rank), 300, 2
    ids = rng.integers(-1, N, size=(T, K)).astype(np.int32)
    gates = rng.uniform(0.2, 1.5, size=(T, K)).astype(np.float32)
    w = wl.build("bucket-edges", 91, "bf16", T, K, 1024, 704, rank, ids, gates,
                 x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02,
                 keep_p=0.9 if masked else None)
    L = run(w)
    assert_plan_equal(L.read_plan(), O.plan_workload(w))
    assert rel_err(D.as_f64(L.Y_host()), O.apply_workload(w)) <= TOL["bf16"]
    # U against the oracle's x~.A.c for every pair
    P = L.read_plan()
    U = L.U()
    for p in range(int(P["header"][B.PH_PAIRS])):
        tk = int(P["pair_tk"][p]); t, k = divmod(tk, K)
        a = int(w.ids[t, k])
        A, _ = O.factors(a, w.rank, w.page_start, w.page_ids, w.a_pages, w.b_pages)
        x = D.as_f64(w.X[t])
        if masked:
            x = x * w.keep_mask[t] * float(np.float32(w.keep_scale))
        ref = float(w.gates[t, k]) * float(w.scale[a]) * (x @ A)
        got = U[P["u_off"][p]:P["u_off"][p + 1]].astype(np.float64)
        assert np.max(np.abs(got - ref)) <= 1e-5 * max(1.0, np.max(np.abs(ref))), (p, a)


def test_apply_fused_rowwise_expand():
    """The fused 256 x 256 epilogue's row-by-row expand (K = 2, ranks above 16),
    every row against the oracle."""
    w = _fused_rowwise()
    L = run(w)
    assert rel_err(D.as_f64(L.Y_host()), O.apply_workload(w)) <= TOL["bf16"]


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


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_apply_full(cfg):
    # every row against the oracle (the prefill batch's oracle takes seconds)
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


def _topk(T, K, N, d_in, d_out, seed, ranks=(2, 5, 8, 16, 17, 33)):
    """Top-K routing (softmax over the K chosen of N(0,1) logits) over N
    adapters with ranks drawn from `ranks`."""
    rng = np.random.default_rng(seed)
    rank = rng.choice(np.asarray(ranks, np.int32), size=N).astype(np.int32)
    ids, gates = wl.topk_softmax(rng, T, N, K)
    return wl.build(f"top{K}-{T}x{d_in}x{d_out}", seed, "bf16", T, K, d_in, d_out, rank, ids, gates,
                    x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02)


def _decode_k4():
    return _topk(100, 4, 40, 1024, 768, 404)


def _fused_rowwise():
    """256 x 256 fused-epilogue shape whose blocks take the row-by-row expand
    (two slots per token, ranks around the MFMA-expand limit of 16)."""
    rng = np.random.default_rng(77)
    T, K, N = 2100, 2, 4
    rank = np.array([3, 17, 64, 129], np.int32)
    ids = rng.integers(0, N, size=(T, K)).astype(np.int32)
    gates = rng.uniform(0.25, 1.0, size=(T, K)).astype(np.float32)
    return wl.build("fused-rowwise", 77, "bf16", T, K, 256, 8192, rank, ids, gates,
                    x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02)


FORWARD_CASES = {
    # top-4 and top-8 routing: decode (per-slot shrink), split-K and stream-K
    "dec_k4": _decode_k4,
    "dec_k8": lambda: _topk(64, 8, 30, 512, 640, 408),
    "sk_k8": lambda: _topk(512, 8, 64, 2048, 2048, 418),
    "split_k4": lambda: _topk(300, 4, 48, 1024, 1536, 414),
    # decode shapes with a keep mask, d_in above one 4096-element block, and
    # ranks up to 128 over many adapters
    "dec4": lambda: wl.config(4, T=96, d_in=4608, d_out=704, seed=204),
    "dec3": lambda: wl.config(3, T=128, d_in=512, d_out=640, n_adapters=300, seed=203),
    "decmix": _mixed_decode,
}


@pytest.mark.parametrize("cfg", ["small1", "small2", "small3", "small4", "small5", "full2", "full3",
                                 "full5", "dec4", "dec3", "decmix", "dec_k4", "dec_k8", "sk_k8",
                                 "split_k4"])
def test_forward_matches_plan_then_apply(cfg):
    """lora_forward in two launches (decode: the plan in workgroup 0 beside
    the GEMM and the per-slot shrink, then the epilogue, which also moves U
    to the plan's layout; stream-K: the plan beside the GEMM, then shrink and
    epilogue): the plan, U and Y equal those of lora_plan then lora_apply bit
    for bit.  The same call captured in a graph is replayed three times, with
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


def test_u_capacity_error_through_forward_decode():
    """lora_forward on a decode shape (per-slot shrink in the GEMM launch)
    follows lora_apply's rule when U does not fit the workspace: the LoRA term
    is skipped, so Y is the base product, and the error bit is set."""
    w = small(2)
    L = D.DeviceLayer(w, max_rank=1)
    B.lora_forward(L.ids, L.gates, L.T, L.K, L.X, L.W_t, L.Y, L.keep_mask, L.keep_scale, L.pool,
                   L.plan, L.ws)
    torch.cuda.synchronize()
    h = B.lora_plan_header(L.plan)
    assert h[B.PH_ERR] & B.DEVERR_CAPACITY
    Yf = L.Y_host().copy()
    L2 = D.DeviceLayer(w, max_rank=1)
    L2.run_plan()
    L2.run_apply()
    torch.cuda.synchronize()
    assert np.array_equal(Yf, L2.Y_host())
    ref = D.as_f64(w.X) @ D.as_f64(w.W_t).T
    assert rel_err(D.as_f64(Yf), ref) <= TOL["bf16"]


@pytest.mark.parametrize("cfg", [2, 5])
def test_plan_header_reader_matches_oracle(cfg):
    w = small(cfg)
    L = D.DeviceLayer(w)
    L.run_plan()
    h = B.lora_plan_header(L.plan)          # waits for the plan on the stream
    ref = O.plan_workload(w)["header"]
    assert h[:8] == [int(v) for v in ref[:8]]


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
    coefficients, more listed rank rows than one LDS list holds (the small
    heterogeneous-rank recipe: d_out 1344, the float32-FMA kernel; the small
    decode recipe: 512 x 768, the MFMA kernel's chunked path)."""
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


@pytest.mark.parametrize("d_in,N,seed", [(512, 600, 31), (320, 300, 32), (768, 40, 33)])
def test_grads_mfma_many_segments(d_in, N, seed):
    """The MFMA outer products with hundreds of segments (more than 256, so
    the workgroup's segment search takes two rounds), several segments per
    256-pair chunk, ranks from 1 to 40 (segments that skip a 16-row block),
    empty slots and a keep mask; d_in = 320 sends dA to the vector form."""
    rng = np.random.default_rng(seed)
    T, K = 2048, 1
    rank = rng.integers(1, 41, size=N).astype(np.int32)
    ids = rng.integers(-1, N, size=(T, K)).astype(np.int32)
    gates = rng.standard_normal((T, K)).astype(np.float32)
    w = wl.build(f"grad-mfma-segs-{seed}", seed, "bf16", T, K, d_in, 512, rank, ids, gates,
                 x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02, keep_p=0.9, with_dY=True,
                 scale=rng.uniform(0.5, 2, N).astype(np.float32))
    print(f"case {w.name}: segments {len(np.unique(ids[ids >= 0]))}", flush=True)
    _check_grads(w, run(w))


def test_grads_full_prefill():
    w = full(4)
    _check_grads(w, run(w))


# ---------------------------------------------------------------- input gradient dX

def _with_dY(w, seed=11):
    """The workload with a seeded N(0,1) dY when its recipe has none."""
    if w.dY is None:
        v = np.random.default_rng(seed).standard_normal((w.T, w.d_out)).astype(np.float32)
        w.dY = v if w.dtype == "f32" else wl.f32_to_bf16_bits(v)
    return w


def _grad_x_run(w):
    L = D.DeviceLayer(w)
    L.run_plan()
    L.run_apply()
    dA, dB, gws = L.grad_buffers()
    L.run_grad(dA, dB, gws)
    Wn = L.weight_transposed()
    dX, xws = L.grad_x_buffers()
    L.run_grad_x(Wn, gws, dX, xws)
    torch.cuda.synchronize()
    return L, D.to_host(dX)


def test_transpose_is_exact():
    for dt, (r, c) in (("bf16", (704, 512)), ("f32", (256, 192)), ("bf16", (100, 37))):
        v = np.random.default_rng(r).standard_normal((r, c)).astype(np.float32)
        a = v if dt == "f32" else wl.f32_to_bf16_bits(v)
        src = D.to_device(a, "cuda")
        dst = torch.empty((c, r), dtype=src.dtype, device="cuda")
        B.lora_transpose(src, dst, r, c, B.LORA_F32 if dt == "f32" else B.LORA_BF16)
        torch.cuda.synchronize()
        assert np.array_equal(D.to_host(dst), a.T)


@pytest.mark.parametrize("cfg", ["small1", "small2", "small3", "small4", "small5", "dec_k4"])
def test_grad_x_small(cfg):
    """dX = dY.W^T + the masked LoRA term, against the oracle (every GEMM
    form: fp32 tiles, decode split-K, split/stream-K 256 x 128, and top-2 and
    four-slot routing)."""
    if cfg == "dec_k4":
        w = _decode_k4()
    else:
        w = wl.small(int(cfg[-1]))
    w = _with_dY(w)
    L, got = _grad_x_run(w)
    ref = O.grad_x_workload(w)
    assert rel_err(D.as_f64(got), ref) <= TOL[w.dtype]


def test_grad_x_prefill_fused_shape():
    """A batch large enough for the 256 x 256 tile GEMM (written as partials
    here), with the keep mask, every row against the oracle."""
    w = wl.config(4, T=2100, d_in=1024, d_out=1536, seed=444)
    L, got = _grad_x_run(w)
    ref = O.grad_x_workload(w)
    assert rel_err(D.as_f64(got), ref) <= TOL["bf16"]


def _with_mask(w, keep_p=0.9, seed=12):
    """The workload with a seeded Bernoulli(keep_p) keep mask on X when its
    recipe has none (the forward, the gradients and dX all see it)."""
    if w.keep_mask is None:
        rng = np.random.default_rng(seed)
        w.keep_mask = (rng.random((w.T, w.d_in)) < keep_p).astype(np.uint8)
        w.keep_scale = float(np.float32(1.0 / keep_p))
    return w


# 17 x 16 output tiles of 256 x 256 (ragged in both): the dX GEMM takes the
# LoRA term and the keep mask in its own epilogue, the last 16 tiles as
# 256 x 128 halves
_FUSED_X = dict(T=4300, d_in=3904, d_out=512)


@pytest.mark.parametrize("cfg,mask", [(4, True), (5, True), (3, True), (3, False), (5, False)])
def test_grad_x_fused_tiles(cfg, mask):
    """dX with the LoRA term in the 256 x 256 tile GEMM's epilogue, every row
    against the oracle: rank-16 segments (MFMA blocks), top-2 routing (the
    row path), mixed ranks up to 128 (both paths in one batch), with and
    without the keep mask."""
    extra = {} if cfg == 4 else {"n_adapters": 40}
    w = _with_dY(wl.config(cfg, seed=460 + cfg, **_FUSED_X, **extra))
    if mask:
        w = _with_mask(w)
    else:
        w.keep_mask = None
        w.keep_scale = 1.0
    assert B.lora_grad_x_workspace_bytes(w.T, w.d_in, w.d_out, B.LORA_BF16) < 1024
    L, got = _grad_x_run(w)
    ref = O.grad_x_workload(w)
    assert rel_err(D.as_f64(got), ref) <= TOL["bf16"]


def test_grad_x_fused_inactive_rows_equal_base_bit_for_bit():
    """In the fused epilogue a row with no active slot, inside a block whose
    other rows carry a masked LoRA term, is dY.W^T rounded once."""
    w = wl.config(4, seed=470, **_FUSED_X)
    w.ids[::3] = -1
    L, got = _grad_x_run(w)
    w0 = wl.config(4, seed=470, **_FUSED_X)
    w0.ids[:] = -1
    L0, base = _grad_x_run(w0)
    assert np.array_equal(got[::3], base[::3])
    assert rel_err(D.as_f64(got), O.grad_x_workload(w)) <= TOL["bf16"]


def test_grad_x_full_prefill_sampled_rows():
    w = full(4)
    L, got = _grad_x_run(w)
    rows = np.unique(np.concatenate([np.arange(0, w.T, 97), [0, w.T - 1],
                                     np.cumsum(w.meta["segment_lengths"])[:-1]]))
    ref = O.grad_x_workload(wl.subset(w, rows))
    assert rel_err(D.as_f64(got[rows]), ref) <= TOL["bf16"]


def test_grad_x_full_prefill_every_row():
    """The input gradient of the full fine-tune prefill batch (8192 x 11008
    -> 4096, keep mask, one fused launch) on every row against the oracle."""
    w = full(4)
    L, got = _grad_x_run(w)
    assert rel_err(D.as_f64(got), O.grad_x_workload(w)) <= TOL["bf16"]


def test_grad_x_inactive_rows_equal_base_bit_for_bit():
    w = _with_dY(wl.small(5))
    L, got = _grad_x_run(w)
    ids0 = w.ids.copy()
    w2 = _with_dY(wl.small(5))
    w2.ids = ids0.copy()
    w2.ids[::3] = -1                      # every third token: no active slot
    L2, got2 = _grad_x_run(w2)
    w3 = _with_dY(wl.small(5))
    w3.ids = np.full_like(ids0, -1)
    L3, base = _grad_x_run(w3)
    for t in range(0, w.T, 3):
        assert np.array_equal(got2[t], base[t])
    ref = O.grad_x_workload(w2)
    assert rel_err(D.as_f64(got2), ref) <= TOL["bf16"]


# ---------------------------------------------------------------- merge across layers

def _layer_set(shapes, N=24, seed=900):
    """Layers of different shapes, each with its own pool of N adapters
    (ranks and factors drawn per layer), sharing adapter ids."""
    return [wl.config(5, T=8, d_in=di, d_out=do, n_adapters=N, seed=seed + i)
            for i, (di, do) in enumerate(shapes)]


@pytest.mark.parametrize("case", ["mixed_shapes", "many_layers", "fallback_widths"])
def test_merge_layers_matches_per_layer(case):
    if case == "mixed_shapes":
        shapes = [(1024, 1024), (1024, 2816), (2816, 1024), (512, 640), (1280, 1280)]
    elif case == "many_layers":
        shapes = [(256 + 128 * (i % 3), 384) for i in range(19)]     # two launches
    else:
        shapes = [(576, 704), (512, 512)]                            # 576: not a multiple of 128
    ws = _layer_set(shapes)
    Ls = [D.DeviceLayer(w) for w in ws]
    rng = np.random.default_rng(31)
    ids = rng.choice(24, size=8, replace=False).astype(np.int32)
    co = rng.choice(np.array([1.0, -1.0, 0.5, -2.0], np.float32), size=8)
    mi = D.to_device(ids, "cuda")
    cf = D.to_device(co, "cuda")
    Wm = [L.W_t.clone() for L in Ls]
    print(f"merge layers case {case}: {len(Ls)} layers", flush=True)
    B.lora_merge_delta_layers(Wm, [L.pool for L in Ls], mi, cf, 8)
    Wr = [L.W_t.clone() for L in Ls]
    for W, L in zip(Wr, Ls):
        B.lora_merge_delta(W, L.pool, mi, cf, 8)
    torch.cuda.synchronize()
    refs = O.merge_layers([dict(W_t=w.W_t, rank=w.rank, scale=w.scale, page_start=w.page_start,
                                page_ids=w.page_ids, a_pages=w.a_pages, b_pages=w.b_pages)
                           for w in ws], ids, co)
    for l, (a, b, ref) in enumerate(zip(Wm, Wr, refs)):
        ga, gb = D.to_host(a), D.to_host(b)
        assert np.array_equal(ga, gb), f"layer {l} differs from lora_merge_delta"
        assert rel_err(D.as_f64(ga), ref) <= TOL["bf16"], l


def test_merge_layers_rejects_shared_weight_and_mixed_dtype():
    ws = _layer_set([(512, 512), (512, 512)])
    Ls = [D.DeviceLayer(w) for w in ws]
    mi = D.to_device(np.array([0, 1], np.int32), "cuda")
    cf = D.to_device(np.array([1.0, 1.0], np.float32), "cuda")
    W = Ls[0].W_t.clone()
    with pytest.raises(B.LoraError) as ei:
        B.lora_merge_delta_layers([W, W], [Ls[0].pool, Ls[1].pool], mi, cf, 2)
    assert ei.value.status == B.LORA_ERR_INVALID_ARG
    f = D.DeviceLayer(wl.small(1))
    with pytest.raises(B.LoraError) as ei:
        B.lora_merge_delta_layers([W, f.W_t], [Ls[0].pool, f.pool], mi, cf, 2)
    assert ei.value.status == B.LORA_ERR_INVALID_ARG


# ---------------------------------------------------------------- pool residency

def test_residency_batches_match_a_fully_resident_pool():
    """Adapters streamed from a pinned host store into a pool that holds
    85 % of their rank rows: each batch's copies run on a side stream while
    the previous batch computes; every batch's Y equals lora_forward over the
    fully resident pool bit for bit, the tables equal the policy oracle's, and
    every resident adapter's pages hold its rows."""
    from oracle import residency as RO
    w = wl.config(3, T=96, d_in=512, d_out=1344, n_adapters=60, seed=303)
    L = D.DeviceLayer(w)
    # host store: adapter a's rows in rank-row order
    rows = np.concatenate([w.page_ids[w.page_start[a]:w.page_start[a + 1]]
                           for a in range(w.n_adapters)]).astype(np.int64)
    store_row = w.page_start[:-1].astype(np.int64)
    sa = D.to_device(w.a_pages[rows], "cpu").pin_memory()
    sb = D.to_device(w.b_pages[rows], "cpu").pin_memory()
    n_pages = int(0.85 * int(w.rank.sum()))     # two batches fit; later ones evict
    ap = torch.zeros((n_pages, w.d_in), dtype=torch.bfloat16, device="cuda")
    bp = torch.zeros((n_pages, w.d_out), dtype=torch.bfloat16, device="cuda")
    res = B.Residency(B.LORA_BF16, w.d_in, w.d_out, w.rank, store_row, sa, sb, ap, bp, L.scale)
    side = torch.cuda.Stream()
    rng = np.random.default_rng(7)
    batches = [wl.zipf_ids(rng, w.T, w.n_adapters).reshape(w.T, 1) for _ in range(6)]
    oracle = RO.trace(w.rank, n_pages, batches)
    outs, refs = [], []
    plan = torch.empty_like(L.plan)
    for b, ids in enumerate(batches):
        print(f"residency batch {b}", flush=True)
        ids_d = D.to_device(ids, "cuda")
        pool = res.prepare(ids, side)
        Y = torch.empty_like(L.Y)
        B.lora_forward(ids_d, L.gates, w.T, 1, L.X, L.W_t, Y, None, 1.0, pool, plan, L.ws)
        res.finish()
        outs.append(Y)
        Yr = torch.empty_like(L.Y)
        plan_r = torch.empty_like(L.plan)
        ws_r = torch.empty_like(L.ws)
        B.lora_forward(ids_d, L.gates, w.T, 1, L.X, L.W_t, Yr, None, 1.0, L.pool, plan_r, ws_r)
        refs.append(Yr)
        # host tables of the library's policy = the oracle's
        rk, ps, pid = res.page_table().tables()
        assert "error" not in oracle[b]
        assert np.array_equal(rk, oracle[b]["rank"]) and np.array_equal(pid, oracle[b]["page_ids"])
    torch.cuda.synchronize()
    for b in range(len(batches)):
        assert np.array_equal(D.to_host(outs[b]), D.to_host(refs[b])), f"batch {b}"
    # the pool now holds every resident adapter's rows
    rk, ps, pid = res.page_table().tables()
    A, Bh = D.to_host(ap), D.to_host(bp)
    for a in range(w.n_adapters):
        if rk[a] == 0:
            continue
        pg = pid[ps[a]:ps[a + 1]]
        src = w.page_ids[w.page_start[a]:w.page_start[a + 1]]
        assert np.array_equal(A[pg], w.a_pages[src]) and np.array_equal(Bh[pg], w.b_pages[src])
    st = res.stats()
    assert st["batches"] == 6 and st["evictions"] > 0
    res.close()


# ---------------------------------------------------------------- tall-skinny QR

def _tsqr_gpu(src, dtype, cols, M, m, n):
    Qt = torch.full((M, n, m), float("nan"), dtype=torch.float32, device="cuda")
    R = torch.full((M, n, n), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.lora_tsqr_workspace_bytes(M, m, n), dtype=torch.uint8, device="cuda")
    B.lora_tsqr(src, dtype, cols, M, m, n, Qt, R, ws)
    torch.cuda.synchronize()
    return Qt.cpu().numpy().astype(np.float64), R.cpu().numpy().astype(np.float64)


TSQR_TOL = 1e-5


@pytest.mark.parametrize("M,m,n", [(5, 1000, 16), (3, 300, 64), (2, 11008, 64), (4, 4096, 1),
                                   (3, 512, 2), (6, 64, 64), (2, 257, 33)])
def test_tsqr_fp32_matches_oracle(M, m, n):
    """Level counts 1..4, ragged last tiles, square and one-column matrices."""
    from oracle import tsqr as TQ
    rng = np.random.default_rng(M * 1000 + m + n)
    A = rng.standard_normal((M, n, m)).astype(np.float32)
    cols = D.to_device(np.arange(M * n, dtype=np.int32), "cuda")
    print(f"tsqr fp32 M={M} m={m} n={n}", flush=True)
    Qt, R = _tsqr_gpu(D.to_device(A.reshape(M * n, m), "cuda"), B.LORA_F32, cols, M, m, n)
    Qo, Ro = TQ.batched_thin_qr(A)
    assert rel_err(R, Ro) <= TSQR_TOL
    assert rel_err(Qt, Qo) <= TSQR_TOL
    assert np.all(np.tril(R, -1) == 0) and np.all(np.diagonal(R, axis1=1, axis2=2) >= 0)


def test_tsqr_bf16_adapter_pages_in_place():
    """The A factors of a pool's adapters (rank 16, d_in 4096), each matrix's
    columns gathered from its pages; the B^T factors likewise (d_out 11008)."""
    from oracle import tsqr as TQ
    w = wl.config(4, T=64, d_in=4096, d_out=11008, seed=41)
    L = D.DeviceLayer(w)
    M, n = w.n_adapters, 16
    cols_h = np.concatenate([w.page_ids[w.page_start[a]:w.page_start[a + 1]] for a in range(M)])
    cols = D.to_device(cols_h.astype(np.int32), "cuda")
    for pages, d, host in ((L.a_pages, w.d_in, w.a_pages), (L.b_pages, w.d_out, w.b_pages)):
        Qt, R = _tsqr_gpu(pages, B.LORA_BF16, cols, M, d, n)
        At = wl.to_f32(host[cols_h]).reshape(M, n, d)
        Qo, Ro = TQ.batched_thin_qr(At)
        assert rel_err(R, Ro) <= TSQR_TOL
        assert rel_err(Qt, Qo) <= TSQR_TOL


def test_tsqr_zero_column():
    """A zero column takes no reflection: R's column is zero there and
    Q.R still equals A."""
    rng = np.random.default_rng(5)
    M, m, n = 2, 700, 8
    A = rng.standard_normal((M, n, m)).astype(np.float32)
    A[1, 3] = 0.0
    cols = D.to_device(np.arange(M * n, dtype=np.int32), "cuda")
    Qt, R = _tsqr_gpu(D.to_device(A.reshape(M * n, m), "cuda"), B.LORA_F32, cols, M, m, n)
    assert np.all(R[1][:, 3] == 0)
    for i in range(M):
        assert rel_err(Qt[i].T @ R[i], A[i].T.astype(np.float64)) <= TSQR_TOL


# ---------------------------------------------------------------- recompression

def _spectral_fleet(dtype, M=12, n=16, d_in=512, d_out=704, seed=61):
    """M adapters of rank n whose products A.B have prescribed, decaying
    spectra (A = P.diag(s), B = Q^T, P and Q with orthonormal columns), plus
    one adapter of another rank (its compression is refused: rank 0)."""
    rng = np.random.default_rng(seed)
    rank = np.full(M + 1, n, np.int32)
    rank[M] = n // 2
    w = wl.build("spectral-fleet", seed, dtype, 4, 1, d_in, d_out, rank,
                 np.zeros((4, 1), np.int32), np.ones((4, 1), np.float32),
                 x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02)
    to = (lambda v: v.astype(np.float32)) if dtype == "f32" else \
        (lambda v: wl.f32_to_bf16_bits(v.astype(np.float32)))
    for a in range(M):
        P, _ = np.linalg.qr(rng.standard_normal((d_in, n)))
        Q, _ = np.linalg.qr(rng.standard_normal((d_out, n)))
        s = 2.0 * 0.5 ** (np.arange(n) * rng.uniform(0.4, 1.2))
        A, Bm = P * s[None, :], Q.T
        pages = w.page_ids[w.page_start[a]:w.page_start[a + 1]]
        w.a_pages[pages] = to(A.T)
        w.b_pages[pages] = to(Bm)
    return w, M + 1, n


@pytest.mark.parametrize("dtype,policy", [("bf16", 1), ("bf16", 0), ("f32", 1)])
def test_compress_matches_oracle(dtype, policy):
    from oracle import tsqr as TQ
    w, M, n = _spectral_fleet(dtype)
    L = D.DeviceLayer(w)
    ratio, energy, floor_rank = 0.3, 0.97, 2
    ad = D.to_device(np.arange(M, dtype=np.int32), "cuda")
    et = torch.float32 if dtype == "f32" else torch.bfloat16
    oa = torch.zeros((M * n, w.d_in), dtype=et, device="cuda")
    ob = torch.zeros((M * n, w.d_out), dtype=et, device="cuda")
    ork = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    osg = torch.zeros((M, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.lora_compress_workspace_bytes(M, w.d_in, w.d_out, n), dtype=torch.uint8,
                     device="cuda")
    B.lora_compress(L.pool, ad, M, n, policy, ratio, energy, floor_rank, oa, ob, ork, osg, ws)
    torch.cuda.synchronize()
    k_gpu, sig = ork.cpu().numpy(), osg.cpu().numpy().astype(np.float64)
    A2, B2 = D.as_f64(D.to_host(oa)), D.as_f64(D.to_host(ob))
    tol = TOL[dtype]
    for a in range(M):
        if w.rank[a] != n:
            assert k_gpu[a] == 0
            continue
        Ad, Bd = O.factors(a, w.rank, w.page_start, w.page_ids, w.a_pages, w.b_pages)
        k, s, Ao, Bo = TQ.compress(Ad, Bd, policy, ratio, energy, floor_rank)
        # the decision has margin: the oracle's cumulative energy is not at the threshold
        cum = np.cumsum(s ** 2) / np.sum(s ** 2)
        assert policy == 0 or np.min(np.abs(cum - np.float32(energy))) > 1e-4
        assert k_gpu[a] == k, (a, k_gpu[a], k)
        assert rel_err(sig[a], s) <= 1e-5
        prod = A2[a * n:a * n + k].T @ B2[a * n:a * n + k]
        assert rel_err(prod, Ao @ Bo) <= tol, a


# ---------------------------------------------------------------- output rounding

RNE_CASES = {
    # 256 x 256 tiles: the rounding in the fused epilogue
    "fused_tiles": (2100, 8192),
    # decode tile, split-K partials: the rounding in the epilogue kernel
    "decode": (64, 640),
    # 256 x 128 tiles: the rounding in the epilogue kernel after the tile GEMM
    "tiles_split": (300, 2048),
}


@pytest.mark.parametrize("case", sorted(RNE_CASES))
def test_output_rounding_is_nearest_even(case):
    """Every output is rounded once to bf16, to nearest with ties to even.
    Inputs make each pre-rounding value exact in fp32 and place it on a bf16
    tie, just above or below one, or on a bf16 value: X rows [1, e, d, 0..],
    W rows [a, 1, 1, 0..] with a of 7 fraction bits in [1, 2) (ulp 2^-7), e
    in {0, 2^-9, +-2^-8, +-3*2^-9} and d in {0, +-2^-16}, so Y = a + e + d
    (every partial sum exact).  Expected bits from torch's own float32 to
    bfloat16 conversion; no slot is active (gates 0), so Y is the base
    product alone."""
    T, d_out = RNE_CASES[case]
    d_in = 64
    ids = np.full((T, 1), -1, np.int32)
    gates = np.zeros((T, 1), np.float32)
    w = wl.build("rne-" + case, 5, "bf16", T, 1, d_in, d_out, np.array([4], np.int32), ids, gates,
                 x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02)
    j = np.arange(d_out)
    a = (1.0 + (j % 128) / 128.0) * np.where((j // 128) % 2 == 0, 1.0, -1.0)
    e_set = np.array([0.0, 2.0 ** -9, 2.0 ** -8, -2.0 ** -8, 3 * 2.0 ** -9, -3 * 2.0 ** -9])
    d_set = np.array([0.0, 2.0 ** -16, -2.0 ** -16])
    t = np.arange(T)
    e = e_set[t % len(e_set)]
    d = d_set[(t // len(e_set)) % len(d_set)]
    X = np.zeros((T, d_in), np.float32)
    X[:, 0], X[:, 1], X[:, 2] = 1.0, e, d
    Wt = np.zeros((d_out, d_in), np.float32)
    Wt[:, 0], Wt[:, 1], Wt[:, 2] = a, 1.0, 1.0
    bits = lambda f: (np.asarray(f, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for arr in (X, Wt):   # every input value is a bf16 value
        assert np.array_equal(wl.bf16_bits_to_f32(bits(arr)), arr)
    w.X, w.W_t = bits(X), bits(Wt)
    L = run(w)
    assert L.read_plan()["header"][B.PH_PAIRS] == 0
    exact = (a[None, :] + e[:, None] + d[:, None]).astype(np.float32)
    assert np.array_equal(exact.astype(np.float64), a[None, :] + e[:, None] + d[:, None])
    want = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = L.Y_host()
    bad = np.argwhere(got != want)
    assert bad.size == 0, (len(bad), bad[:4].tolist())
    # the ties to even were reached: some outputs sit exactly half-way
    half = np.abs(exact - wl.bf16_bits_to_f32(bits(exact))) == 2.0 ** -8
    assert half.any()


def test_merge_rounding_is_nearest_even():
    """lora_merge_delta rounds W + delta once to bf16, to nearest with ties to
    even: one rank-2 adapter of scale 1 with A rows e and d and B rows of
    ones makes delta[n][i] = e_i + d_i, and W[n][i] = a_n of 7 fraction bits,
    so W + delta is exact in fp32 and sits on, near or off bf16 ties.
    Expected bits from torch's float32 to bfloat16 conversion."""
    d_in, d_out = 256, 512
    ids = np.zeros((1, 1), np.int32)
    w = wl.build("rne-merge", 6, "bf16", 1, 1, d_in, d_out, np.array([2], np.int32), ids,
                 np.ones((1, 1), np.float32), x_var=1.0, w_var=0.02, a_var=1 / 64, b_var=0.02,
                 scale=np.ones(1, np.float32))
    n = np.arange(d_out)
    a = (1.0 + (n % 128) / 128.0) * np.where((n // 128) % 2 == 0, 1.0, -1.0)
    i = np.arange(d_in)
    e = np.array([0.0, 2.0 ** -9, 2.0 ** -8, -2.0 ** -8, 3 * 2.0 ** -9, -3 * 2.0 ** -9])[i % 6]
    d = np.array([0.0, 2.0 ** -16, -2.0 ** -16])[(i // 6) % 3]
    bits = lambda f: (np.asarray(f, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    Wt = np.repeat(a[:, None], d_in, axis=1).astype(np.float32)
    a_pages, b_pages = w.a_pages.copy(), w.b_pages.copy()
    p0, p1 = int(w.page_ids[w.page_start[0]]), int(w.page_ids[w.page_start[0] + 1])
    a_pages[p0], a_pages[p1] = bits(e), bits(d)
    b_pages[p0], b_pages[p1] = bits(np.ones(d_out)), bits(np.ones(d_out))
    for v in (Wt, e, d):   # every input value is a bf16 value
        assert np.array_equal(wl.bf16_bits_to_f32(bits(v)), np.asarray(v, np.float32))
    w.W_t, w.a_pages, w.b_pages = bits(Wt), a_pages, b_pages
    L = D.DeviceLayer(w)
    W = L.W_t.clone()
    L.run_merge(W, np.zeros(1, np.int32), np.ones(1, np.float32))
    torch.cuda.synchronize()
    exact64 = a[:, None] + e[None, :] + d[None, :]
    exact = exact64.astype(np.float32)
    assert np.array_equal(exact.astype(np.float64), exact64)
    want = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = D.to_host(W)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (len(bad), bad[:4].tolist())
    assert (np.abs(exact - wl.bf16_bits_to_f32(bits(exact))) == 2.0 ** -8).any()
