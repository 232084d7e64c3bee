"""CPU oracle for the batched tall-skinny QR (FlashTSQR) and the retained-rank
recompression it serves.

TEST INFRASTRUCTURE.  Only the tests may import or call this module; it
shares no code with the library.

The LoRAForge page ("LoRAForge：压缩与执行协同，让多LoRA服务更高效", section
FlashTSQR：批量因子构造的加速器, and its glossary note on TSQR) names the
operation: the QR factorisation of many tall, skinny matrices (rows far more
than columns), computed by local QRs of row blocks whose results are merged,
parallel over modules and row blocks.  A blocked algorithm only reorders the
same factorisation: for a matrix of full column rank the thin factorisation
A = Q.R with Q^T.Q = I, R upper triangular and a non-negative diagonal is
unique.  So the oracle is that definition: a library QR (one step), then the
signs fixed so that diag(R) >= 0.  Everything is float64.
"""
from __future__ import annotations

import numpy as np


def thin_qr(A):
    """A (m x n, m >= n) = Q (m x n, orthonormal columns) . R (n x n, upper
    triangular, diag >= 0)."""
    A = np.asarray(A, dtype=np.float64)
    Q, R = np.linalg.qr(A, mode="reduced")
    d = np.where(np.diag(R) < 0, -1.0, 1.0)
    return Q * d[None, :], R * d[:, None]


def batched_thin_qr(At):
    """At: [M][n][m], each matrix given by its n columns of length m (the
    layout of a pool's pages: a page is one column of A, or one row of B = one
    column of B^T).  Returns Qt [M][n][m] (Q's columns, the same layout) and
    R [M][n][n]."""
    At = np.asarray(At, dtype=np.float64)
    Qs, Rs = [], []
    for a in At:
        Q, R = thin_qr(a.T)
        Qs.append(Q.T)
        Rs.append(R)
    return np.stack(Qs), np.stack(Rs)


def retained_rank(sigma, n, policy, ratio=1.0, energy=1.0, floor_rank=1):
    """Retained rank of one module ([LoRAForge] 核心设计: LoRAForge-U keeps a
    uniform fraction of each module's rank; LoRAForge-S allocates by the
    module's cumulative spectral-energy curve, energy = squared singular
    values).  Uniform: ceil(ratio * n), the product taken in float32.
    Spectral: the smallest k >= 1 whose leading k energies reach the fraction
    `energy` of the total.  Then at least floor_rank, at most n."""
    if policy == 0:
        k = int(np.ceil(np.float32(ratio) * np.float32(n)))
    else:
        e = np.asarray(sigma, dtype=np.float64) ** 2
        tot = float(np.sum(e))
        target = float(np.float32(energy)) * tot
        k, acc = n, 0.0
        for j in range(n):
            acc += e[j]
            if acc >= target:
                k = j + 1
                break
    return int(min(n, max(int(floor_rank), k, 1)))


def compress(A, B, policy, ratio=1.0, energy=1.0, floor_rank=1):
    """Recompression of one adapter module to its retained rank: the best
    rank-k approximation of the product A.B (A: d_in x n, B: n x d_out), split
    as A' = U_k.sqrt(S_k), B' = sqrt(S_k).V_k^T from the SVD of A.B.  Returns
    (k, the n largest singular values, A', B')."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    n = A.shape[1]
    U, s, Vt = np.linalg.svd(A @ B, full_matrices=False)
    s = s[:n]
    k = retained_rank(s, n, policy, ratio, energy, floor_rank)
    r = np.sqrt(s[:k])
    return k, s, U[:, :k] * r[None, :], r[:, None] * Vt[:k]
