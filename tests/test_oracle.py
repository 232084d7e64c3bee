"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, never against the oracle's own formulas retyped.

  * a hand-worked example (tests/golden/tiny_layer.json);
  * brute force with pure-Python loops over the paged layout on tiny shapes;
  * closed forms: one adapter for every token equals the merged weight
    X.(W + g.s.A.B); inactive rows equal X.W exactly;
  * invariants: linearity in the gates, token-permutation equivariance,
    duplicate slots = summed gate, mask of ones = no mask;
  * merge followed by unmerge restores W once rounded to the storage dtype;
    the fused switch equals unmerge-then-merge;
  * gradients: <dY, Y> is linear in A for fixed B (and vice versa), so a
    finite difference along a random direction is exact up to rounding; and
    CPU torch.autograd in float64 on the dense form of the layer;
  * the input gradient dX: <dY, Y> is linear in X (mask fixed), so the same
    directional difference pins it through the forward; torch.autograd; one
    adapter for every token gives dY times the merged weight's transpose;
    inactive rows give dY.W^T exactly.
"""
import json
import os

import numpy as np
import pytest

from oracle import lora_oracle as O
from lora_adapter_amd import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden", "tiny_layer.json")


def _gold():
    with open(GOLD) as f:
        return json.load(f)


def _gold_arrays(g):
    f32 = lambda v: np.asarray(v, dtype=np.float32)
    i32 = lambda v: np.asarray(v, dtype=np.int32)
    return dict(X=f32(g["X"]), W_t=f32(g["W_t"]), rank=i32(g["rank"]), scale=f32(g["scale"]),
                page_start=i32(g["page_start"]), page_ids=i32(g["page_ids"]),
                a_pages=f32(g["a_pages"]), b_pages=f32(g["b_pages"]), ids=i32(g["ids"]),
                gates=f32(g["gates"]))


# ---------------------------------------------------------------- golden

def test_golden_apply():
    g = _gold()
    a = _gold_arrays(g)
    Y = O.apply(**a)
    np.testing.assert_array_equal(Y, np.asarray(g["expected_Y"], dtype=np.float64))


def test_golden_plan():
    g = _gold()
    a = _gold_arrays(g)
    p = O.plan(a["ids"], a["gates"], a["rank"], a["page_start"], a["page_ids"], a["a_pages"].shape[0])
    exp = g["expected_plan"]
    np.testing.assert_array_equal(p["header"][:8], exp["header"])
    for k in ("pair_tk", "seg_adapter", "seg_off", "seg_row_off", "bucket_seg_off", "u_off", "slot_pos",
              "pair_adapter"):
        np.testing.assert_array_equal(p[k], exp[k], err_msg=k)


def test_golden_merge():
    g = _gold()
    a = _gold_arrays(g)
    Wm = O.merge(a["W_t"], a["rank"], a["scale"], a["page_start"], a["page_ids"], a["a_pages"],
                 a["b_pages"], np.asarray(g["merge_ids"]), np.asarray(g["merge_coeffs"], np.float32))
    np.testing.assert_array_equal(Wm, np.asarray(g["expected_merged_W_t"], dtype=np.float64))


def test_golden_merge_layers():
    g = _gold()
    a = _gold_arrays(g)
    f32 = lambda v: np.asarray(v, dtype=np.float32)
    i32 = lambda v: np.asarray(v, dtype=np.int32)
    l1 = g["layer1"]
    layers = [dict(W_t=a["W_t"], rank=a["rank"], scale=a["scale"], page_start=a["page_start"],
                   page_ids=a["page_ids"], a_pages=a["a_pages"], b_pages=a["b_pages"]),
              dict(W_t=f32(l1["W_t"]), rank=i32(l1["rank"]), scale=f32(l1["scale"]),
                   page_start=i32(l1["page_start"]), page_ids=i32(l1["page_ids"]),
                   a_pages=f32(l1["a_pages"]), b_pages=f32(l1["b_pages"]))]
    out = O.merge_layers(layers, np.asarray(g["merge_ids"]), np.asarray(g["merge_coeffs"], np.float32))
    np.testing.assert_array_equal(out[0], np.asarray(g["expected_merged_W_t"], dtype=np.float64))
    np.testing.assert_array_equal(out[1], np.asarray(g["expected_merged_W_t_layer1"], dtype=np.float64))
    # layers do not interact: changing layer 1's pool leaves layer 0's result
    layers[1]["a_pages"] = layers[1]["a_pages"] * 3
    out2 = O.merge_layers(layers, np.asarray(g["merge_ids"]), np.asarray(g["merge_coeffs"], np.float32))
    np.testing.assert_array_equal(out2[0], out[0])
    assert not np.array_equal(out2[1], out[1])


def test_golden_grad():
    g = _gold()
    a = _gold_arrays(g)
    dY = np.asarray(g["dY"], dtype=np.float32)
    gr = O.grad(a["X"], None, 1.0, dY, a["rank"], a["scale"], a["page_start"], a["page_ids"],
                a["a_pages"], a["b_pages"], a["ids"], a["gates"])
    assert sorted(gr) == [0, 1]
    for ad in (0, 1):
        np.testing.assert_array_equal(gr[ad][0], np.asarray(g["expected_dA"][str(ad)], dtype=np.float64))
        np.testing.assert_array_equal(gr[ad][1], np.asarray(g["expected_dB"][str(ad)], dtype=np.float64))


# ---------------------------------------------------------------- brute force

def _rand_tiny(seed, with_mask=False):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 6)); K = int(rng.integers(1, 3))
    d_in = int(rng.integers(1, 13)); d_out = int(rng.integers(1, 13))
    N = int(rng.integers(1, 5))
    rank = rng.integers(0, 4, size=N).astype(np.int32)
    total = int(rank.sum())
    n_pages = total + 2
    perm = rng.permutation(n_pages).astype(np.int32)
    page_ids = perm[:total]
    page_start = np.concatenate([[0], np.cumsum(rank)]).astype(np.int32)
    a_pages = rng.standard_normal((n_pages, d_in)).astype(np.float32)
    b_pages = rng.standard_normal((n_pages, d_out)).astype(np.float32)
    X = rng.standard_normal((T, d_in)).astype(np.float32)
    W_t = rng.standard_normal((d_out, d_in)).astype(np.float32)
    ids = rng.integers(-1, N, size=(T, K)).astype(np.int32)
    gates = rng.standard_normal((T, K)).astype(np.float32)
    gates[rng.random((T, K)) < 0.2] = 0.0
    scale = rng.uniform(0.5, 2.0, size=N).astype(np.float32)
    mask = (rng.random((T, d_in)) < 0.7).astype(np.uint8) if with_mask else None
    kappa = float(np.float32(1 / 0.7)) if with_mask else 1.0
    return dict(X=X, W_t=W_t, rank=rank, scale=scale, page_start=page_start, page_ids=page_ids,
                a_pages=a_pages, b_pages=b_pages, ids=ids, gates=gates, keep_mask=mask,
                keep_scale=kappa)


def _brute_apply(d):
    """Pure-Python loops straight from the paged layout."""
    X, W_t = d["X"].tolist(), d["W_t"].tolist()
    T, d_in = len(X), len(X[0])
    d_out = len(W_t)
    K = d["ids"].shape[1]
    Y = [[sum(float(X[t][i]) * float(W_t[n][i]) for i in range(d_in)) for n in range(d_out)]
         for t in range(T)]
    for t in range(T):
        for k in range(K):
            a = int(d["ids"][t][k]); g = float(d["gates"][t][k])
            if a < 0 or int(d["rank"][a]) == 0 or g == 0.0:
                continue
            r = int(d["rank"][a])
            xt = [float(X[t][i]) for i in range(d_in)]
            if d["keep_mask"] is not None:
                xt = [xt[i] * float(d["keep_mask"][t][i]) * float(d["keep_scale"]) for i in range(d_in)]
            for j in range(r):
                page = int(d["page_ids"][int(d["page_start"][a]) + j])
                u = sum(xt[i] * float(d["a_pages"][page][i]) for i in range(d_in))
                for n in range(d_out):
                    Y[t][n] += g * float(d["scale"][a]) * u * float(d["b_pages"][page][n])
    return np.asarray(Y)


@pytest.mark.parametrize("seed", range(25))
def test_brute_force_tiny(seed):
    d = _rand_tiny(seed, with_mask=(seed % 2 == 1))
    Y = O.apply(**d)
    Yb = _brute_apply(d)
    np.testing.assert_allclose(Y, Yb, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def _dense_factors_by_indexing(w, a):
    """A_a and B_a gathered with numpy fancy indexing (a route independent of
    the oracle's page walk)."""
    pages = w.page_ids[w.page_start[a]:w.page_start[a + 1]]
    A = wl.to_f32(w.a_pages[pages]).astype(np.float64).T
    B = wl.to_f32(w.b_pages[pages]).astype(np.float64)
    return A, B


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_single_adapter_equals_merged_weight(cfg):
    w = wl.small(cfg)
    a = int(np.argmax(w.rank))
    gval = np.float32(0.75)
    ids = np.full((w.T, w.K), -1, dtype=np.int32)
    ids[:, 0] = a
    gates = np.zeros((w.T, w.K), dtype=np.float32)
    gates[:, 0] = gval
    Y = O.apply(w.X, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages,
                ids, gates)
    A, B = _dense_factors_by_indexing(w, a)
    Wm = wl.to_f32(w.W_t).astype(np.float64).T + float(gval) * float(w.scale[a]) * (A @ B)
    Yref = wl.to_f32(w.X).astype(np.float64) @ Wm
    assert np.max(np.abs(Y - Yref)) <= 1e-10 * np.max(np.abs(Yref))
    # and through the oracle's own merge (a different code path than apply)
    Wm2 = O.merge(w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages,
                  np.array([a]), np.array([gval]))
    Yref2 = wl.to_f32(w.X).astype(np.float64) @ Wm2.T
    assert np.max(np.abs(Y - Yref2)) <= 1e-10 * np.max(np.abs(Yref2))


def test_inactive_rows_equal_base_exactly():
    w = wl.small(3)
    ids = w.ids.copy(); gates = w.gates.copy(); rank = w.rank.copy()
    ids[0, 0] = -1                     # empty slot
    gates[1, 0] = 0.0                  # zero gate
    gates[2, 0] = -0.0                 # negative zero gate
    rank_zero_adapter = int(ids[3, 0])
    rank[rank_zero_adapter] = 0        # rank-0 adapter (pool kept consistent below)
    ps = np.concatenate([[0], np.cumsum(rank)]).astype(np.int32)
    pid = np.concatenate([w.page_ids[w.page_start[a]:w.page_start[a + 1]] if rank[a] else
                          np.zeros(0, np.int32) for a in range(w.n_adapters)]).astype(np.int32)
    Y = O.apply(w.X, w.W_t, rank, w.scale, ps, pid, w.a_pages, w.b_pages, ids, gates)
    base = wl.to_f32(w.X).astype(np.float64) @ wl.to_f32(w.W_t).astype(np.float64).T
    inactive = [t for t in range(w.T) if ids[t, 0] == -1 or gates[t, 0] == 0 or rank[ids[t, 0]] == 0]
    assert {0, 1, 2, 3} <= set(inactive)
    for t in inactive:
        assert np.array_equal(Y[t], base[t])
    active = [t for t in range(w.T) if t not in inactive]
    assert any(not np.array_equal(Y[t], base[t]) for t in active)


def test_linearity_in_gates():
    w = wl.small(5)
    rng = np.random.default_rng(7)
    g1 = rng.standard_normal(w.gates.shape).astype(np.float32)
    g2 = rng.standard_normal(w.gates.shape).astype(np.float32)
    al, be = 0.5, -1.25                      # exact in float32
    g3 = (np.float32(al) * g1 + np.float32(be) * g2).astype(np.float32)
    # g3 is rounded to float32; compare against the fp64 combination of the
    # unrounded gates through the linear term only
    f = lambda g: O.apply(w.X, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages,
                          w.b_pages, w.ids, g)
    base = f(np.zeros_like(g1))
    L1, L2, L3 = f(g1) - base, f(g2) - base, f(g3) - base
    g3_64 = al * g1.astype(np.float64) + be * g2.astype(np.float64)
    assert np.max(np.abs(g3.astype(np.float64) - g3_64)) <= 1e-6 * np.max(np.abs(g3_64))
    lhs, rhs = L3, al * L1 + be * L2
    assert np.max(np.abs(lhs - rhs)) <= 1e-6 * np.max(np.abs(rhs))
    # with gates exactly representable (small integers) linearity is exact up to fp64 rounding
    gi1 = rng.integers(-2, 3, size=w.gates.shape).astype(np.float32)
    gi2 = rng.integers(-2, 3, size=w.gates.shape).astype(np.float32)
    Li1, Li2, Li3 = f(gi1) - base, f(gi2) - base, f(gi1 + 2 * gi2) - base
    assert np.max(np.abs(Li3 - (Li1 + 2 * Li2))) <= 1e-9 * np.max(np.abs(Li3))


def test_token_permutation_equivariance():
    w = wl.small(3)
    perm = np.random.default_rng(3).permutation(w.T)
    Y = O.apply_workload(w)
    Yp = O.apply(w.X[perm], w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages,
                 w.b_pages, w.ids[perm], w.gates[perm])
    np.testing.assert_allclose(Yp, Y[perm], rtol=0, atol=1e-9 * np.max(np.abs(Y)))


def test_duplicate_slot_equals_summed_gate():
    w = wl.small(5)
    ids = w.ids.copy(); gates = w.gates.copy()
    ids[:, 1] = ids[:, 0]
    Y2 = O.apply(w.X, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages, ids, gates)
    ids1 = ids.copy(); ids1[:, 1] = -1
    g1 = gates.copy(); g1[:, 0] = gates[:, 0].astype(np.float64) + gates[:, 1].astype(np.float64)
    # the summed gate rounds to float32; use gates whose sum is exact instead
    gates_e = np.round(gates * 8) / 8
    Y2 = O.apply(w.X, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages, ids, gates_e)
    g1 = gates_e.copy(); g1[:, 0] = gates_e[:, 0] + gates_e[:, 1]; g1[:, 1] = 0
    Y1 = O.apply(w.X, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages, ids1, g1)
    np.testing.assert_allclose(Y2, Y1, rtol=0, atol=1e-9 * np.max(np.abs(Y1)))


def test_mask_of_ones_is_no_mask_and_zero_mask_is_base():
    w = wl.small(4)
    ones = np.ones_like(w.keep_mask)
    Ym = O.apply(w.X, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages,
                 w.ids, w.gates, ones, 1.0)
    Yn = O.apply(w.X, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages,
                 w.ids, w.gates)
    assert np.array_equal(Ym, Yn)
    Yz = O.apply(w.X, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages,
                 w.ids, w.gates, np.zeros_like(w.keep_mask), w.keep_scale)
    base = wl.to_f32(w.X).astype(np.float64) @ wl.to_f32(w.W_t).astype(np.float64).T
    assert np.array_equal(Yz, base)
    # the dropout scale multiplies the LoRA term only: mask of ones with kappa
    # doubles the LoRA term when kappa = 2
    Y2 = O.apply(w.X, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages,
                 w.ids, w.gates, ones, 2.0)
    np.testing.assert_allclose(Y2 - base, 2 * (Yn - base), rtol=0, atol=1e-9 * np.max(np.abs(Yn)))


# ---------------------------------------------------------------- merge

@pytest.mark.parametrize("cfg", [1, 5])
def test_merge_then_unmerge_restores_w(cfg):
    w = wl.small(cfg)
    ids = np.arange(min(8, w.n_adapters), dtype=np.int32)
    c = np.ones(len(ids), dtype=np.float32)
    Wp = O.merge_workload(w, ids=ids, coeffs=c)
    # round the merged weight to storage, unmerge, round again
    enc = (lambda v: wl.f32_to_bf16_bits(v.astype(np.float32))) if w.dtype == "bf16" else \
          (lambda v: v.astype(np.float32))
    Wp_st = enc(Wp)
    assert not np.array_equal(Wp_st, w.W_t)
    # fp64 round trip from the exact W returns W bit-for-bit
    Wpp = O.merge_workload(w, W_t=w.W_t, ids=np.concatenate([ids, ids]),
                           coeffs=np.concatenate([c, -c]))
    assert np.array_equal(enc(Wpp), w.W_t)


def test_fused_switch_equals_unmerge_then_merge():
    w = wl.small(5)
    s1 = np.array([1, 4, 9], dtype=np.int32)
    s2 = np.array([2, 7], dtype=np.int32)
    W_s1 = O.merge_workload(w, ids=s1, coeffs=np.ones(3, np.float32))
    fused = O.merge(W_s1, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages,
                    np.concatenate([s1, s2]), np.array([-1, -1, -1, 1, 1], np.float32))
    W_s2 = O.merge_workload(w, ids=s2, coeffs=np.ones(2, np.float32))
    assert np.max(np.abs(fused - W_s2)) <= 1e-12 * np.max(np.abs(W_s2))


# ---------------------------------------------------------------- gradients

def _loss(w, a_pages, b_pages):
    Y = O.apply(w.X, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, a_pages, b_pages,
                w.ids, w.gates, w.keep_mask, w.keep_scale)
    return float(np.sum(Y * wl.to_f32(w.dY).astype(np.float64)))


def test_golden_grad_x():
    g = _gold()
    a = _gold_arrays(g)
    dY = np.asarray(g["dY"], dtype=np.float32)
    dX = O.grad_x(a["X"], None, 1.0, dY, a["W_t"], a["rank"], a["scale"], a["page_start"],
                  a["page_ids"], a["a_pages"], a["b_pages"], a["ids"], a["gates"])
    np.testing.assert_array_equal(dX, np.asarray(g["expected_dX"], dtype=np.float64))


def _f64_pool(w):
    w64 = type("W", (), {})()
    for k in ("X", "W_t", "rank", "scale", "page_start", "page_ids", "ids", "gates", "keep_mask",
              "keep_scale", "dY"):
        setattr(w64, k, getattr(w, k))
    w64.X = wl.to_f32(w.X).astype(np.float64)
    w64.W_t = wl.to_f32(w.W_t).astype(np.float64)
    w64.dY = wl.to_f32(w.dY).astype(np.float64)
    return w64, wl.to_f32(w.a_pages).astype(np.float64), wl.to_f32(w.b_pages).astype(np.float64)


def test_grad_by_directional_difference():
    w = wl.config(4, T=40, d_in=64, d_out=48, seed=41)
    g = O.grad_workload(w)
    w64, A0, B0 = _f64_pool(w)
    rng = np.random.default_rng(5)
    for a, (dA, dB) in g.items():
        pages = w.page_ids[w.page_start[a]:w.page_start[a + 1]]
        dirA = rng.standard_normal((len(pages), w.d_in))
        dirB = rng.standard_normal((len(pages), w.d_out))
        Ap, Am = A0.copy(), A0.copy()
        Ap[pages] += dirA; Am[pages] -= dirA
        fd = (_loss(w64, Ap, B0) - _loss(w64, Am, B0)) / 2.0
        an = float(np.sum(dA.T * dirA))
        assert abs(fd - an) <= 1e-9 * max(1.0, abs(an))
        Bp, Bm = B0.copy(), B0.copy()
        Bp[pages] += dirB; Bm[pages] -= dirB
        fd = (_loss(w64, A0, Bp) - _loss(w64, A0, Bm)) / 2.0
        an = float(np.sum(dB * dirB))
        assert abs(fd - an) <= 1e-9 * max(1.0, abs(an))


def test_grad_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    w = wl.small(4)
    g = O.grad_workload(w)
    X = torch.tensor(wl.to_f32(w.X), dtype=torch.float64)
    M = torch.tensor(w.keep_mask, dtype=torch.float64) * float(np.float32(w.keep_scale))
    dY = torch.tensor(wl.to_f32(w.dY), dtype=torch.float64)
    Wd = torch.tensor(wl.to_f32(w.W_t), dtype=torch.float64).T
    Af, Bf = {}, {}
    for a in range(w.n_adapters):
        A, B = _dense_factors_by_indexing(w, a)
        Af[a] = torch.tensor(A, requires_grad=True)
        Bf[a] = torch.tensor(B, requires_grad=True)
    Y = X @ Wd
    rows = []
    for t in range(w.T):
        extra = torch.zeros(w.d_out, dtype=torch.float64)
        for k in range(w.K):
            a = int(w.ids[t, k])
            if a < 0 or w.gates[t, k] == 0:
                continue
            c = float(w.gates[t, k]) * float(w.scale[a])
            extra = extra + c * ((X[t] * M[t]) @ Af[a]) @ Bf[a]
        rows.append(extra)
    Y = Y + torch.stack(rows)
    (Y * dY).sum().backward()
    for a, (dA, dB) in g.items():
        np.testing.assert_allclose(dA, Af[a].grad.numpy(), rtol=1e-10, atol=1e-9)
        np.testing.assert_allclose(dB, Bf[a].grad.numpy(), rtol=1e-10, atol=1e-9)


def _loss_x(w, X64):
    """<dY, Y> through the (separately pinned) forward, with X replaced."""
    Y = O.apply(X64, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages,
                w.ids, w.gates, w.keep_mask, w.keep_scale)
    return float(np.sum(Y * wl.to_f32(w.dY).astype(np.float64)))


@pytest.mark.parametrize("cfg", [4, 5])
def test_grad_x_by_directional_difference(cfg):
    """<dY, Y> is linear in X for a fixed mask: its central difference along a
    random direction V equals <dX, V> up to rounding."""
    w = wl.config(4, T=40, d_in=64, d_out=48, seed=43) if cfg == 4 else \
        wl.config(5, T=24, d_in=64, d_out=64, n_adapters=10, seed=44)
    if w.dY is None:
        w.dY = wl.f32_to_bf16_bits(np.random.default_rng(7).standard_normal((w.T, w.d_out))
                                   .astype(np.float32))
    dX = O.grad_x_workload(w)
    X0 = wl.to_f32(w.X).astype(np.float64)
    V = np.random.default_rng(9).standard_normal(X0.shape)
    fd = (_loss_x(w, X0 + V) - _loss_x(w, X0 - V)) / 2.0
    an = float(np.sum(dX * V))
    assert abs(fd - an) <= 1e-9 * max(1.0, abs(an))


def test_grad_x_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    w = wl.small(4)
    dXo = O.grad_x_workload(w)
    X = torch.tensor(wl.to_f32(w.X), dtype=torch.float64, requires_grad=True)
    M = torch.tensor(w.keep_mask, dtype=torch.float64) * float(np.float32(w.keep_scale))
    dY = torch.tensor(wl.to_f32(w.dY), dtype=torch.float64)
    Wd = torch.tensor(wl.to_f32(w.W_t), dtype=torch.float64).T
    Y = X @ Wd
    rows = []
    for t in range(w.T):
        extra = torch.zeros(w.d_out, dtype=torch.float64)
        for k in range(w.K):
            a = int(w.ids[t, k])
            if a < 0 or w.gates[t, k] == 0:
                continue
            A, B = _dense_factors_by_indexing(w, a)
            c = float(w.gates[t, k]) * float(w.scale[a])
            extra = extra + c * ((X[t] * M[t]) @ torch.tensor(A)) @ torch.tensor(B)
        rows.append(extra)
    Y = Y + torch.stack(rows)
    (Y * dY).sum().backward()
    np.testing.assert_allclose(dXo, X.grad.numpy(), rtol=1e-10, atol=1e-9)


@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_grad_x_single_adapter_equals_merged_weight(cfg):
    """All tokens on one adapter with gate g and no mask: dX = dY.(W + g.s.A.B)^T,
    with the merged weight from the oracle's merge (pinned on its own)."""
    w = wl.small(cfg)
    a = int(np.argmax(w.rank))
    gval = np.float32(-1.25)
    ids = np.full((w.T, w.K), -1, dtype=np.int32)
    ids[:, 0] = a
    gates = np.zeros((w.T, w.K), dtype=np.float32)
    gates[:, 0] = gval
    dY = np.random.default_rng(3).standard_normal((w.T, w.d_out)).astype(np.float32)
    dX = O.grad_x(w.X, None, 1.0, dY, w.W_t, w.rank, w.scale, w.page_start, w.page_ids,
                  w.a_pages, w.b_pages, ids, gates)
    Wm_t = O.merge(w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages,
                   np.array([a]), np.array([gval]))
    ref = dY.astype(np.float64) @ Wm_t
    assert np.max(np.abs(dX - ref)) <= 1e-10 * np.max(np.abs(ref))


def test_grad_x_inactive_rows_equal_base_exactly():
    w = wl.small(4)
    ids = w.ids.copy(); gates = w.gates.copy()
    ids[0, 0] = -1
    gates[1, 0] = 0.0
    dX = O.grad_x(w.X, w.keep_mask, w.keep_scale, w.dY, w.W_t, w.rank, w.scale, w.page_start,
                  w.page_ids, w.a_pages, w.b_pages, ids, gates)
    base = wl.to_f32(w.dY).astype(np.float64) @ wl.to_f32(w.W_t).astype(np.float64)
    for t in (0, 1):
        assert np.array_equal(dX[t], base[t])
    assert not np.array_equal(dX[2], base[2])


# ---------------------------------------------------------------- generator

def test_generator_is_deterministic_and_distributed():
    a = wl.small(3); b = wl.small(3)
    assert a.digests() == b.digests()
    c = wl.config(3, T=77, d_in=512, d_out=1344, n_adapters=40, seed=999)
    assert c.digests()["X"] != a.digests()["X"]
    w = wl.config(2, T=64, d_in=1024, d_out=1024, n_adapters=8)
    W = wl.to_f32(w.W_t)
    assert abs(W.var() - 0.02) < 0.002 and abs(W.mean()) < 0.002
    A = wl.to_f32(w.a_pages)
    assert abs(A.var() - 1 / 64) < 0.002
    # pages of one adapter are scattered, and spare pages exist
    assert w.n_pages == int(w.rank.sum()) + wl.SPARE_PAGES
    assert len(set(w.page_ids.tolist())) == len(w.page_ids)


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38],
                    dtype=np.float32)
    bits = wl.f32_to_bf16_bits(vals)
    back = wl.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties to even -> 1.0
    assert back[1] == 1.0
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert back[2] == np.float32(1.0 + 2 ** -6)
    assert back[3] == 1.0 and back[4] == -2.5 and back[0] == 1.0
    assert abs(back[5] - 3.0e38) / 3.0e38 < 2 ** -8


def test_workload_shapes_match_the_stated_configs():
    # full sizes are cheap to describe but heavy to draw; check routing recipes at full size
    rng = wl.streams(3)
    ids = wl.zipf_ids(rng["ids"], 200000, 1024)
    frac0 = np.mean(ids == 0)
    H = np.sum(1.0 / np.arange(1, 1025))
    assert abs(frac0 - 1 / H) < 0.01
    lens = wl.dirichlet_segments(np.random.default_rng(0), 8192, 4)
    assert lens.sum() == 8192 and np.all(lens > 0)
    ids2, g2 = wl.top2_softmax(np.random.default_rng(1), 16, 2048)
    assert np.all(ids2[:, 0] != ids2[:, 1])
    np.testing.assert_allclose(g2.sum(1), 1.0, rtol=1e-6)
    assert np.all(g2[:, 0] >= g2[:, 1])
