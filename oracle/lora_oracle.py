"""CPU oracle for the batched multi-adapter LoRA layer.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import or call this module.  It shares no
code with the HIP library (no kernels, headers, helpers, tables or pre/post
processing); the only module both sides consume is the seeded input generator,
which holds none of the layer's arithmetic.

Everything here is the plain definition in float64, slow and obviously
correct: no sorting, blocking, fusion or paging tricks beyond what the
definition states.  Pages cited (by title and section):

  [LoRAFusion]  "LoRAFusion：消除冗余内存访问的多 LoRA 高效微调系统",
                section 解决什么真问题 (factor shapes A in R^{d x r},
                B in R^{r x k}; the forward Y = X.W + X.(A.B) with dropout
                among the small ops between the GEMMs).
  [S-LoRA]      "S-LoRA：一个GPU运行数千大模型成为可能", section 批处理
                (merged weight for one adapter vs computing xAB on the fly for
                a batch of adapters, no padding) and section Unified Paging
                (one page per rank row; a rank-R adapter takes R pages).
  [AdaFuse]     "AdaFuse: Accelerating Dynamic Adapter Inference via
                Token-Level Pre-Gating and Fused Kernel Optimization",
                section 关键设计 item 1 (gate-weighted sum over experts,
                y = f(x) + sum_i G_i . E_i(x), top-2) and item 2 (fused
                switch: un-merge the previous adapters with negated
                weights and merge the new ones in one operation).
  [LoRAForge]   "LoRAForge：压缩与执行协同，让多LoRA服务更高效", section
                LoRAForge的核心设计 (explicit retained rank, no padding) and
                the rank-specialised-kernel note (kernels specialised per
                rank value, e.g. 4, 8, 16).

Readings where the pages are silent (the plainest one the rest supports):
  * Factor orientation: x.A shrinks d_in -> r, then .B expands r -> d_out.
    W is d_in x d_out mathematically and stored transposed, W_t[d_out][d_in].
  * Each adapter carries a scale s_a; a slot's coefficient is c = g * s_a
    and multiplies the whole adapter output (the gate in [AdaFuse] item 1).
  * Dropout acts on the LoRA branch input only: x~ = x * m * kappa with a
    supplied 0/1 keep mask m and kappa = 1/keep probability.
  * A slot is active when its id is a valid adapter of rank > 0 and its gate
    is non-zero; inactive slots contribute exactly nothing.
  * Plan order: active (token, slot) pairs sorted by (rank bucket, adapter,
    token, slot); bucket(r) = smallest b in 0..7 with r <= 2^b, else 8.
  * Gradients (the pages give none; only A and B train, [LoRAFusion]) are the
    derivatives of <dY, Y> with respect to A_a and B_a, and, for the layer
    below, with respect to X.
"""
from __future__ import annotations

import numpy as np

MAX_RANK = 1024
N_BUCKETS = 9              # 1, 2, 4, ..., 128, and "more than 128"
HEADER_LEN = 16

ERR_BAD_ID = 1             # id < -1 or id >= n_adapters
ERR_BAD_RANK = 2           # referenced adapter with rank < 0 or > MAX_RANK
ERR_BAD_POOL = 4           # used adapter whose page_start/page_ids are inconsistent

H_P, H_S, H_ERR, H_RPAIRS, H_RUSED, H_T, H_K, H_N = range(8)


def widen(arr) -> np.ndarray:
    """Storage array -> float64.  bf16 is stored as its 16-bit pattern, the top
    half of an IEEE float32, so widening it is a shift; float32 widens exactly."""
    a = np.asarray(arr)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rank_bucket(r: int) -> int:
    """Rank-specialisation bucket ([LoRAForge], rank-specialised kernels)."""
    for b in range(8):
        if r <= (1 << b):
            return b
    return 8


def _pool_ok(a, rank, page_start, page_ids, n_pages) -> bool:
    r = int(rank[a])
    s0, s1 = int(page_start[a]), int(page_start[a + 1])
    if s0 < 0 or s1 - s0 != r or s1 > len(page_ids):
        return False
    return all(0 <= int(page_ids[s0 + j]) < n_pages for j in range(r))


def _classify(ids, gates, rank, page_start, page_ids, n_pages):
    """Per slot: adapter id if the slot is active, else -1; plus the error word."""
    ids = np.asarray(ids).reshape(-1)
    gates = np.asarray(gates, dtype=np.float32).reshape(-1)
    N = len(rank)
    err = 0
    cand = []
    for i, a in enumerate(ids.tolist()):
        if a == -1:
            cand.append(-1)
            continue
        if a < -1 or a >= N:
            err |= ERR_BAD_ID
            cand.append(-1)
            continue
        r = int(rank[a])
        if r < 0 or r > MAX_RANK:
            err |= ERR_BAD_RANK
            cand.append(-1)
            continue
        cand.append(a if (r > 0 and gates[i] != 0.0) else -1)
    used = sorted(set(a for a in cand if a >= 0))
    bad = set(a for a in used if not _pool_ok(a, rank, page_start, page_ids, n_pages))
    if bad:
        err |= ERR_BAD_POOL
    act = [a if (a >= 0 and a not in bad) else -1 for a in cand]
    return act, err


def plan(ids, gates, rank, page_start, page_ids, n_pages) -> dict:
    """Segment plan of one batch ([AdaFuse] item 3: rows grouped by adapter into
    segments for one gathered launch; [LoRAForge]: rank buckets; [S-LoRA]
    批处理: no padding, so offsets are prefix sums of the true ranks)."""
    ids = np.asarray(ids, dtype=np.int32)
    T, K = ids.shape
    act, err = _classify(ids, gates, rank, page_start, page_ids, n_pages)
    pairs = [(rank_bucket(int(rank[a])), a, i // K, i % K) for i, a in enumerate(act) if a >= 0]
    pairs = sorted(pairs)
    P = len(pairs)
    pair_tk = [t * K + k for (_, _, t, k) in pairs]
    seg_adapter, seg_off, seg_bucket = [], [], []
    for p, (b, a, _, _) in enumerate(pairs):
        if p == 0 or a != pairs[p - 1][1]:
            seg_adapter.append(a)
            seg_off.append(p)
            seg_bucket.append(b)
    S = len(seg_adapter)
    seg_off.append(P)
    seg_row_off = [0]
    for a in seg_adapter:
        seg_row_off.append(seg_row_off[-1] + int(rank[a]))
    bucket_seg_off = []
    for b in range(N_BUCKETS + 1):
        first = S
        for s in range(S):
            if seg_bucket[s] >= b:
                first = s
                break
        bucket_seg_off.append(first)
    u_off = [0]
    for (_, a, _, _) in pairs:
        u_off.append(u_off[-1] + int(rank[a]))
    pair_adapter = [a for (_, a, _, _) in pairs]
    slot_pos = [-1] * (T * K)
    for p, tk in enumerate(pair_tk):
        slot_pos[tk] = p
    header = [0] * HEADER_LEN
    header[H_P], header[H_S], header[H_ERR] = P, S, err
    header[H_RPAIRS], header[H_RUSED] = u_off[-1], seg_row_off[-1]
    header[H_T], header[H_K], header[H_N] = T, K, len(rank)
    i32 = lambda v: np.asarray(v, dtype=np.int32)
    return {"header": i32(header), "pair_tk": i32(pair_tk), "seg_adapter": i32(seg_adapter),
            "seg_off": i32(seg_off), "seg_row_off": i32(seg_row_off),
            "bucket_seg_off": i32(bucket_seg_off), "u_off": i32(u_off), "slot_pos": i32(slot_pos),
            "pair_adapter": i32(pair_adapter)}


def factors(a, rank, page_start, page_ids, a_pages, b_pages):
    """Adapter a's factors from the paged pool ([S-LoRA] Unified Paging: a rank-R
    adapter occupies R pages).  A_a is d_in x r (page j = column j), B_a is
    r x d_out (page j = row j)."""
    r = int(rank[a])
    pages = [int(page_ids[int(page_start[a]) + j]) for j in range(r)]
    A = np.stack([widen(a_pages[p]) for p in pages], axis=1) if r else np.zeros((a_pages.shape[1], 0))
    B = np.stack([widen(b_pages[p]) for p in pages], axis=0) if r else np.zeros((0, b_pages.shape[1]))
    return A, B


def apply(X, W_t, rank, scale, page_start, page_ids, a_pages, b_pages, ids, gates,
          keep_mask=None, keep_scale=1.0, rows=None) -> np.ndarray:
    """Y = X.W + sum over a token's active slots of g.s.(x~.A).B, float64, unrounded.

    The forward of [LoRAFusion] 解决什么真问题 (Y = X.W + X.(A.B), dropout on the
    LoRA input), batched over adapters as in [S-LoRA] 批处理 (base computed for
    all rows, each row's x.A.B added on its own) and gate-weighted as in
    [AdaFuse] 关键设计 item 1.  ``rows`` restricts the output to those tokens."""
    ids = np.asarray(ids, dtype=np.int32)
    T, K = ids.shape
    n_pages = a_pages.shape[0]
    act, _ = _classify(ids, gates, rank, page_start, page_ids, n_pages)
    g64 = np.asarray(gates, dtype=np.float32).astype(np.float64).reshape(T, K)
    s64 = np.asarray(scale, dtype=np.float32).astype(np.float64)
    kappa = float(np.float32(keep_scale))
    rows = list(range(T)) if rows is None else [int(t) for t in rows]
    X64 = widen(X)
    W64 = widen(W_t).T                        # d_in x d_out
    Y = X64[rows] @ W64
    cache = {}
    for out_row, t in enumerate(rows):
        for k in range(K):
            a = act[t * K + k]
            if a < 0:
                continue
            if a not in cache:
                cache[a] = factors(a, rank, page_start, page_ids, a_pages, b_pages)
            A, B = cache[a]
            x = X64[t]
            if keep_mask is not None:
                x = x * np.asarray(keep_mask[t], dtype=np.float64) * kappa
            u = x @ A
            Y[out_row] += (g64[t, k] * s64[a]) * (u @ B)
    return Y


def merge(W_t, rank, scale, page_start, page_ids, a_pages, b_pages, merge_ids, coeffs) -> np.ndarray:
    """W_t + sum_i c_i.s_i.(A_i.B_i)^T in float64, unrounded, [d_out][d_in].

    One adapter merged into the weight as in [S-LoRA] 批处理 (formula 1 there);
    signed coefficients give [AdaFuse] 关键设计 item 2's fused switch
    (previous adapters with negative weight, new ones with positive).
    Invalid ids are skipped."""
    W = widen(W_t).copy()
    n_pages = a_pages.shape[0]
    s64 = np.asarray(scale, dtype=np.float32).astype(np.float64)
    for a, c in zip(np.asarray(merge_ids).tolist(), np.asarray(coeffs, dtype=np.float32).tolist()):
        if not (0 <= a < len(rank)) or not (0 < int(rank[a]) <= MAX_RANK):
            continue
        if not _pool_ok(a, rank, page_start, page_ids, n_pages):
            continue
        A, B = factors(a, rank, page_start, page_ids, a_pages, b_pages)
        W += (float(c) * s64[a]) * (A @ B).T
    return W


def merge_layers(layers, merge_ids, coeffs) -> list:
    """The same signed merge applied to every layer, each against its own pool:
    [AdaFuse] 关键设计 item 3 packs the merges of all layers into one batched
    operation (its inference flow switches the chosen adapters in every layer
    at once).  ``layers`` is a list of dicts with W_t, rank, scale, page_start,
    page_ids, a_pages, b_pages; returns each layer's merged W_t (float64,
    unrounded), in order.  Layers do not interact."""
    return [merge(L["W_t"], L["rank"], L["scale"], L["page_start"], L["page_ids"], L["a_pages"],
                  L["b_pages"], merge_ids, coeffs) for L in layers]


def grad(X, keep_mask, keep_scale, dY, rank, scale, page_start, page_ids, a_pages, b_pages,
         ids, gates) -> dict:
    """Gradients of L = <dY, Y> with respect to every used adapter's factors.

    The pages train only A and B with W frozen ([LoRAFusion] 解决什么真问题) and
    give no backward formula; differentiating the forward above gives, per
    active slot with c = g.s and x~ the (masked) token row:
        dB_a += c . outer(x~.A_a, dY_t)        (r x d_out)
        dA_a += c . outer(x~, dY_t.B_a^T)      (d_in x r)
    Returns {a: (dA_a, dB_a)} in float64."""
    ids = np.asarray(ids, dtype=np.int32)
    T, K = ids.shape
    n_pages = a_pages.shape[0]
    act, _ = _classify(ids, gates, rank, page_start, page_ids, n_pages)
    g64 = np.asarray(gates, dtype=np.float32).astype(np.float64).reshape(T, K)
    s64 = np.asarray(scale, dtype=np.float32).astype(np.float64)
    kappa = float(np.float32(keep_scale))
    X64 = widen(X)
    dY64 = widen(dY)
    out = {}
    for t in range(T):
        for k in range(K):
            a = act[t * K + k]
            if a < 0:
                continue
            if a not in out:
                A, B = factors(a, rank, page_start, page_ids, a_pages, b_pages)
                out[a] = [np.zeros_like(A), np.zeros_like(B), A, B]
            dA, dB, A, B = out[a]
            c = g64[t, k] * s64[a]
            x = X64[t]
            if keep_mask is not None:
                x = x * np.asarray(keep_mask[t], dtype=np.float64) * kappa
            dB += c * np.outer(x @ A, dY64[t])
            dA += c * np.outer(x, dY64[t] @ B.T)
    return {a: (v[0], v[1]) for a, v in out.items()}


def grad_x(X, keep_mask, keep_scale, dY, W_t, rank, scale, page_start, page_ids, a_pages,
           b_pages, ids, gates) -> np.ndarray:
    """Gradient of L = <dY, Y> with respect to the layer input X, float64,
    unrounded: the input gradient a fine-tune backward hands to the layer
    below ([LoRAFusion] 解决什么真问题: W frozen, A and B trained, dropout on
    the LoRA branch).  The pages give no formula; differentiating the forward
    above, per token t:
        dX_t = dY_t.W^T  +  sum over t's active slots of  c . kappa . m_t * ((dY_t.B_a^T).A_a^T)
    with W^T = W_t (stored [d_out][d_in]) and m_t the keep mask row (the base
    path sees X itself, so the mask and kappa touch only the LoRA term)."""
    ids = np.asarray(ids, dtype=np.int32)
    T, K = ids.shape
    n_pages = a_pages.shape[0]
    act, _ = _classify(ids, gates, rank, page_start, page_ids, n_pages)
    g64 = np.asarray(gates, dtype=np.float32).astype(np.float64).reshape(T, K)
    s64 = np.asarray(scale, dtype=np.float32).astype(np.float64)
    kappa = float(np.float32(keep_scale))
    dY64 = widen(dY)
    dX = dY64 @ widen(W_t)                    # (T x d_out) . (d_out x d_in)
    cache = {}
    for t in range(T):
        for k in range(K):
            a = act[t * K + k]
            if a < 0:
                continue
            if a not in cache:
                cache[a] = factors(a, rank, page_start, page_ids, a_pages, b_pages)
            A, B = cache[a]
            v = (g64[t, k] * s64[a]) * ((dY64[t] @ B.T) @ A.T)
            if keep_mask is not None:
                v = v * np.asarray(keep_mask[t], dtype=np.float64) * kappa
            dX[t] += v
    return dX


def grad_pages(grads: dict, rank, page_start, page_ids, n_pages, d_in, d_out):
    """Scatter per-adapter gradients into the pool's page layout; pages of
    adapters without gradients are NaN (the kernel leaves them untouched)."""
    dA_pages = np.full((n_pages, d_in), np.nan)
    dB_pages = np.full((n_pages, d_out), np.nan)
    for a, (dA, dB) in grads.items():
        for j in range(int(rank[a])):
            p = int(page_ids[int(page_start[a]) + j])
            dA_pages[p] = dA[:, j]
            dB_pages[p] = dB[j, :]
    return dA_pages, dB_pages


def apply_workload(w, rows=None):
    return apply(w.X, w.W_t, w.rank, w.scale, w.page_start, w.page_ids, w.a_pages, w.b_pages,
                 w.ids, w.gates, w.keep_mask, w.keep_scale, rows=rows)


def plan_workload(w):
    return plan(w.ids, w.gates, w.rank, w.page_start, w.page_ids, w.n_pages)


def merge_workload(w, W_t=None, ids=None, coeffs=None):
    return merge(w.W_t if W_t is None else W_t, w.rank, w.scale, w.page_start, w.page_ids,
                 w.a_pages, w.b_pages, w.merge_ids if ids is None else ids,
                 w.merge_coeffs if coeffs is None else coeffs)


def grad_workload(w):
    return grad(w.X, w.keep_mask, w.keep_scale, w.dY, w.rank, w.scale, w.page_start, w.page_ids,
                w.a_pages, w.b_pages, w.ids, w.gates)


def grad_x_workload(w):
    return grad_x(w.X, w.keep_mask, w.keep_scale, w.dY, w.W_t, w.rank, w.scale, w.page_start,
                  w.page_ids, w.a_pages, w.b_pages, w.ids, w.gates)
