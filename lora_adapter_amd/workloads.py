"""Seeded synthetic inputs for the batched multi-adapter LoRA layer.

This module only draws numbers and lays them out: it holds none of the layer's
arithmetic.  Both the HIP path (through the tests and the benchmark) and the
CPU oracle consume the arrays it returns, so it must stay free of anything the
layer computes.

Storage conventions (what the C ABI receives):
  * fp32 tensors are numpy float32; bf16 tensors are numpy uint16 holding the
    bf16 bit pattern (top half of the fp32 word, round-to-nearest-even).
  * ``W_t`` is the base weight in nn.Linear layout, ``[d_out][d_in]``.
  * The adapter pool is paged: rank row ``j`` of adapter ``a`` (column ``j`` of
    its down factor A, row ``j`` of its up factor B) lives at page
    ``page_ids[page_start[a] + j]`` of ``a_pages [n_pages][d_in]`` and of
    ``b_pages [n_pages][d_out]``.  Pages of one adapter are scattered by a
    seeded permutation and a few spare pages hold values no adapter owns, as
    in S-LoRA's unified pool ("Unified Paging": one page per rank row, pages
    interleaved and non-contiguous).

Distributions: ``N(mu, v)`` is read with ``v`` the variance.  Draws are made in
float32 (numpy's ziggurat) and rounded to bf16 where the dtype is bf16.
Every role (ranks, W, A, B, X, routing, gates, mask, dY, merge set, pages) has
its own child stream of ``SeedSequence(seed)``, so adding a draw to one role
never shifts another.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

ROLES = ("ranks", "W", "A", "B", "X", "ids", "gates", "mask", "dY", "merge",
         "pages", "spare")

SPARE_PAGES = 3   # pages in the pool that no adapter owns


def streams(seed: int) -> Dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(ROLES))
    return {r: np.random.Generator(np.random.PCG64(c)) for r, c in zip(ROLES, children)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(f)):
        raise ValueError("generator produced a non-finite value")
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f32(arr: np.ndarray) -> np.ndarray:
    """Storage array (float32 or bf16 bits) widened to float32."""
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr)
    return np.asarray(arr, dtype=np.float32)


def _normal(rng: np.random.Generator, shape, var: float, dtype: str, chunk_rows: int = 4096):
    """N(0, var) drawn in float32, stored as float32 or bf16 bits, row chunks."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    std = np.float32(np.sqrt(var))
    if len(shape) == 1:
        shape2 = (1, shape[0])
        view = out.reshape(shape2)
    else:
        view = out
    rows = view.shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        blk = rng.standard_normal((r1 - r0,) + view.shape[1:], dtype=np.float32) * std
        view[r0:r1] = blk if dtype == "f32" else f32_to_bf16_bits(blk)
    return out


@dataclass
class Workload:
    """One synthetic batch for one projection layer (all arrays host-side)."""
    name: str
    dtype: str                 # "f32" or "bf16"
    T: int
    K: int
    d_in: int
    d_out: int
    n_adapters: int
    X: np.ndarray              # [T][d_in]
    W_t: np.ndarray            # [d_out][d_in]
    rank: np.ndarray           # int32 [N]
    scale: np.ndarray          # float32 [N]
    page_start: np.ndarray     # int32 [N+1]
    page_ids: np.ndarray       # int32 [sum(rank)]
    a_pages: np.ndarray        # [n_pages][d_in]
    b_pages: np.ndarray        # [n_pages][d_out]
    ids: np.ndarray            # int32 [T][K], -1 = empty slot
    gates: np.ndarray          # float32 [T][K]
    keep_mask: Optional[np.ndarray] = None   # uint8 [T][d_in] (1 = keep)
    keep_scale: float = 1.0                  # float32 value
    dY: Optional[np.ndarray] = None          # [T][d_out]
    merge_ids: Optional[np.ndarray] = None   # int32 [m]
    merge_coeffs: Optional[np.ndarray] = None  # float32 [m]
    meta: dict = field(default_factory=dict)

    @property
    def n_pages(self) -> int:
        return int(self.a_pages.shape[0])

    @property
    def max_rank(self) -> int:
        return int(self.rank.max()) if self.rank.size else 0

    def arrays(self) -> Dict[str, np.ndarray]:
        out = {k: getattr(self, k) for k in ("X", "W_t", "rank", "scale", "page_start",
                                              "page_ids", "a_pages", "b_pages", "ids", "gates")}
        for k in ("keep_mask", "dY", "merge_ids", "merge_coeffs"):
            v = getattr(self, k)
            if v is not None:
                out[k] = v
        return out

    def digests(self) -> Dict[str, str]:
        return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
                for k, v in self.arrays().items()}


def build(name: str, seed: int, dtype: str, T: int, K: int, d_in: int, d_out: int,
          rank: np.ndarray, ids: np.ndarray, gates: np.ndarray, *,
          x_var: float, w_var: float, a_var: float, b_var: float,
          scale: Optional[np.ndarray] = None, keep_p: Optional[float] = None,
          with_dY: bool = False, merge_ids: Optional[np.ndarray] = None,
          merge_coeffs: Optional[np.ndarray] = None,
          rng: Optional[Dict[str, np.random.Generator]] = None) -> Workload:
    """Lay out one workload from already-drawn ranks and routing."""
    rng = rng or streams(seed)
    rank = np.asarray(rank, dtype=np.int32)
    N = int(rank.size)
    total = int(rank.sum())
    n_pages = total + SPARE_PAGES
    perm = rng["pages"].permutation(n_pages).astype(np.int32)
    page_ids = np.ascontiguousarray(perm[:total])
    page_start = np.zeros(N + 1, dtype=np.int32)
    page_start[1:] = np.cumsum(rank, dtype=np.int64).astype(np.int32)
    W_t = _normal(rng["W"], (d_out, d_in), w_var, dtype)
    a_pages = _normal(rng["A"], (n_pages, d_in), a_var, dtype)
    b_pages = _normal(rng["B"], (n_pages, d_out), b_var, dtype)
    X = _normal(rng["X"], (T, d_in), x_var, dtype)
    keep_mask = None
    keep_scale = 1.0
    if keep_p is not None:
        keep_mask = (rng["mask"].random((T, d_in)) < keep_p).astype(np.uint8)
        keep_scale = float(np.float32(1.0 / keep_p))
    dY = _normal(rng["dY"], (T, d_out), 1.0, dtype) if with_dY else None
    if scale is None:
        scale = np.ones(N, dtype=np.float32)
    return Workload(name=name, dtype=dtype, T=T, K=K, d_in=d_in, d_out=d_out, n_adapters=N,
                    X=X, W_t=W_t, rank=rank, scale=np.asarray(scale, dtype=np.float32),
                    page_start=page_start, page_ids=page_ids, a_pages=a_pages, b_pages=b_pages,
                    ids=np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(T, K)),
                    gates=np.ascontiguousarray(np.asarray(gates, dtype=np.float32).reshape(T, K)),
                    keep_mask=keep_mask, keep_scale=keep_scale, dY=dY,
                    merge_ids=None if merge_ids is None else np.asarray(merge_ids, dtype=np.int32),
                    merge_coeffs=None if merge_coeffs is None else np.asarray(merge_coeffs, dtype=np.float32),
                    meta={"seed": seed})


# --------------------------------------------------------------------------
# Routing and rank samplers (inputs only: the router itself is not modelled)
# --------------------------------------------------------------------------

def zipf_ids(rng: np.random.Generator, n: int, support: int, s: float = 1.0) -> np.ndarray:
    """Finite Zipf: P(k) proportional to 1/k^s on k = 1..support, id = k-1 (inverse CDF)."""
    w = 1.0 / np.arange(1, support + 1, dtype=np.float64) ** s
    cdf = np.cumsum(w) / w.sum()
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), support - 1).astype(np.int32)


def top2_softmax(rng: np.random.Generator, T: int, N: int):
    """Per token: N(0,1) logits over N adapters, top-2 ids (ties: lower id),
    gates = softmax over the two chosen logits."""
    ids = np.empty((T, 2), dtype=np.int32)
    gates = np.empty((T, 2), dtype=np.float32)
    for t in range(T):
        logits = rng.standard_normal(N)
        order = np.argsort(-logits, kind="stable")
        i0, i1 = int(order[0]), int(order[1])
        l0, l1 = logits[i0], logits[i1]
        ids[t] = (i0, i1)
        gates[t] = (1.0 / (1.0 + np.exp(l1 - l0)), 1.0 / (1.0 + np.exp(l0 - l1)))
    return ids, gates


def topk_softmax(rng: np.random.Generator, T: int, N: int, k: int):
    """Per token: N(0,1) logits over N adapters, the top-k ids (ties: lower
    id), gates = softmax over the k chosen logits (top-k routing)."""
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float32)
    for t in range(T):
        logits = rng.standard_normal(N)
        order = np.argsort(-logits, kind="stable")[:k]
        sel = logits[order]
        e = np.exp(sel - sel.max())
        ids[t] = order
        gates[t] = e / e.sum()
    return ids, gates


def dirichlet_segments(rng: np.random.Generator, T: int, n_seg: int) -> np.ndarray:
    """Contiguous segment lengths from Dirichlet(1,...,1) weights, floor for all
    but the last, last takes the rest; resampled until no segment is empty."""
    while True:
        w = rng.dirichlet(np.ones(n_seg))
        n = np.floor(T * w[:-1]).astype(np.int64)
        last = T - int(n.sum())
        lens = np.append(n, last)
        if np.all(lens > 0):
            return lens.astype(np.int32)


# --------------------------------------------------------------------------
# The five named workloads, plus scaled copies for fast tests
# --------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny-fp32-256x256-4seg",
    2: "llama7b-qproj-decode-4096x4096-T64-64xr16",
    3: "hetero-rank-serving-4096x11008-T256-1024ad-zipf",
    4: "finetune-prefill-4096x11008-T8192-4seg-r16-dropout",
    5: "compressed-fleet-top2-5120x5120-T512-2048ad",
}


def config(i: int, *, T: Optional[int] = None, d_in: Optional[int] = None,
           d_out: Optional[int] = None, n_adapters: Optional[int] = None,
           seed: Optional[int] = None) -> Workload:
    """Workload ``i`` (1..5) at full size, or with some sizes overridden (same
    recipe, smaller shapes) for tests the oracle must finish in seconds."""
    seed = i if seed is None else seed
    rng = streams(seed)
    bf = "bf16"
    if i == 1:
        T = T or 64; d_in = d_in or 256; d_out = d_out or 256
        rank = np.array([4, 8, 8, 16], dtype=np.int32)
        N = 4
        seg = max(1, T // 4)
        ids = np.minimum(np.arange(T) // seg, N - 1).astype(np.int32).reshape(T, 1)
        gates = np.ones((T, 1), dtype=np.float32)
        scale = (16.0 / rank).astype(np.float32)
        return build(CONFIG_NAMES[1], seed, "f32", T, 1, d_in, d_out, rank, ids, gates,
                     x_var=1.0, w_var=1.0 / d_in, a_var=1.0 / d_in, b_var=0.01,
                     scale=scale, rng=rng)
    if i == 2:
        T = T or 64; d_in = d_in or 4096; d_out = d_out or 4096; N = n_adapters or 64
        rank = np.full(N, 16, dtype=np.int32)
        ids = rng["ids"].integers(0, N, size=(T, 1)).astype(np.int32)
        gates = np.ones((T, 1), dtype=np.float32)
        return build(CONFIG_NAMES[2], seed, bf, T, 1, d_in, d_out, rank, ids, gates,
                     x_var=1.0, w_var=0.02, a_var=1.0 / 64, b_var=0.02, rng=rng)
    if i == 3:
        T = T or 256; d_in = d_in or 4096; d_out = d_out or 11008; N = n_adapters or 1024
        rank = rng["ranks"].choice(np.array([8, 16, 32, 64, 128]), size=N).astype(np.int32)
        ids = zipf_ids(rng["ids"], T, N).reshape(T, 1)
        gates = np.ones((T, 1), dtype=np.float32)
        return build(CONFIG_NAMES[3], seed, bf, T, 1, d_in, d_out, rank, ids, gates,
                     x_var=1.0, w_var=0.02, a_var=1.0 / 64, b_var=0.02, rng=rng)
    if i == 4:
        T = T or 8192; d_in = d_in or 4096; d_out = d_out or 11008; N = 4
        rank = np.full(N, 16, dtype=np.int32)
        lens = dirichlet_segments(rng["ids"], T, N)
        ids = np.repeat(np.arange(N, dtype=np.int32), lens).reshape(T, 1)
        gates = np.ones((T, 1), dtype=np.float32)
        w = build(CONFIG_NAMES[4], seed, bf, T, 1, d_in, d_out, rank, ids, gates,
                  x_var=1.0, w_var=0.02, a_var=1.0 / 64, b_var=0.02, keep_p=0.9,
                  with_dY=True, rng=rng)
        w.meta["segment_lengths"] = lens.tolist()
        return w
    if i == 5:
        T = T or 512; d_in = d_in or 5120; d_out = d_out or 5120; N = n_adapters or 2048
        rank = np.clip(rng["ranks"].geometric(0.25, size=N), 2, 16).astype(np.int32)
        ids, gates = top2_softmax(rng["gates"], T, N)
        merge_ids = rng["merge"].choice(N, size=8, replace=False).astype(np.int32)
        merge_coeffs = np.ones(8, dtype=np.float32)
        return build(CONFIG_NAMES[5], seed, bf, T, 2, d_in, d_out, rank, ids, gates,
                     x_var=1.0, w_var=0.02, a_var=1.0 / 64, b_var=0.02,
                     merge_ids=merge_ids, merge_coeffs=merge_coeffs, rng=rng)
    raise ValueError(f"unknown workload {i}")


def small(i: int) -> Workload:
    """The recipe of workload ``i`` at sizes the oracle finishes in about a
    second, still spanning several GEMM tiles and a ragged token tail."""
    if i == 1:
        return config(1, T=61)
    if i == 2:
        return config(2, T=45, d_in=512, d_out=768, n_adapters=12, seed=102)
    if i == 3:
        return config(3, T=77, d_in=512, d_out=1344, n_adapters=40, seed=103)
    if i == 4:
        return config(4, T=333, d_in=512, d_out=704, seed=104)
    if i == 5:
        return config(5, T=70, d_in=640, d_out=640, n_adapters=48, seed=105)
    raise ValueError(i)


def subset(w: Workload, rows) -> Workload:
    """The same layer (weights, pool, routing of the chosen tokens) restricted
    to the token rows ``rows``, in that order: a bounded sample of a large
    batch for timing the CPU oracle."""
    rows = np.asarray(rows, dtype=np.int64)
    take = lambda a: None if a is None else np.ascontiguousarray(a[rows])
    return Workload(name=f"{w.name}-rows{len(rows)}", dtype=w.dtype, T=int(len(rows)), K=w.K,
                    d_in=w.d_in, d_out=w.d_out, n_adapters=w.n_adapters, X=take(w.X), W_t=w.W_t,
                    rank=w.rank, scale=w.scale, page_start=w.page_start, page_ids=w.page_ids,
                    a_pages=w.a_pages, b_pages=w.b_pages, ids=take(w.ids), gates=take(w.gates),
                    keep_mask=take(w.keep_mask), keep_scale=w.keep_scale, dY=take(w.dY),
                    merge_ids=w.merge_ids, merge_coeffs=w.merge_coeffs, meta=dict(w.meta))
