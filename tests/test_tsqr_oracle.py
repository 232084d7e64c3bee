"""Pins for the thin-QR oracle (oracle/tsqr.py): a hand-worked example, the
Cholesky identity A^T.A = R^T.R (R from a different library routine), and
classical Gram-Schmidt written out in plain Python loops on tiny matrices."""
import json
import os

import numpy as np
import pytest

from oracle import tsqr as TQ

GOLD = os.path.join(os.path.dirname(__file__), "golden", "tsqr.json")


def test_golden_qr():
    g = json.load(open(GOLD))
    Q, R = TQ.thin_qr(np.asarray(g["A"], float))
    np.testing.assert_allclose(R, np.asarray(g["expected_R"], float), atol=1e-14)
    np.testing.assert_allclose(3 * Q, np.asarray(g["expected_Q_times_3"], float), atol=1e-14)


@pytest.mark.parametrize("shape", [(300, 16), (1000, 64), (65, 64), (4096, 2)])
def test_r_is_the_cholesky_factor_of_the_gram_matrix(shape):
    rng = np.random.default_rng(shape[0] + shape[1])
    A = rng.standard_normal(shape)
    Q, R = TQ.thin_qr(A)
    L = np.linalg.cholesky(A.T @ A)            # lower, positive diagonal
    np.testing.assert_allclose(R, L.T, rtol=1e-9, atol=1e-9 * np.abs(R).max())
    np.testing.assert_allclose(Q @ R, A, atol=1e-12 * np.abs(A).max() * shape[0])
    np.testing.assert_allclose(Q.T @ Q, np.eye(shape[1]), atol=1e-12)
    assert np.all(np.tril(R, -1) == 0) and np.all(np.diag(R) >= 0)


def _gram_schmidt(A):
    m, n = len(A), len(A[0])
    Q = [[0.0] * n for _ in range(m)]
    R = [[0.0] * n for _ in range(n)]
    for j in range(n):
        v = [A[i][j] for i in range(m)]
        for k in range(j):
            R[k][j] = sum(Q[i][k] * A[i][j] for i in range(m))
            for i in range(m):
                v[i] -= R[k][j] * Q[i][k]
        R[j][j] = sum(x * x for x in v) ** 0.5
        for i in range(m):
            Q[i][j] = v[i] / R[j][j]
    return Q, R


@pytest.mark.parametrize("seed", range(4))
def test_matches_gram_schmidt_on_tiny_matrices(seed):
    rng = np.random.default_rng(seed)
    m, n = int(rng.integers(3, 9)), int(rng.integers(1, 4))
    A = rng.standard_normal((m, n))
    Qg, Rg = _gram_schmidt(A.tolist())
    Q, R = TQ.thin_qr(A)
    np.testing.assert_allclose(R, np.asarray(Rg), atol=1e-12)
    np.testing.assert_allclose(Q, np.asarray(Qg), atol=1e-12)


def test_batched_layout_is_columns_per_row():
    rng = np.random.default_rng(3)
    At = rng.standard_normal((3, 4, 50))       # 3 matrices of 50 x 4, given by columns
    Qt, R = TQ.batched_thin_qr(At)
    for i in range(3):
        np.testing.assert_allclose(Qt[i].T @ R[i], At[i].T, atol=1e-12)


# ---------------------------------------------------------------- recompression

def _gold_module():
    g = json.load(open(GOLD))["compress"]
    P = np.asarray(g["P_columns"], float).T
    Q = np.asarray(g["Q_columns"], float).T
    s = np.asarray(g["s"], float)
    return g, P * s[None, :], Q.T


def test_golden_retained_ranks_and_errors():
    g, A, B = _gold_module()
    for c in g["cases"]:
        k, s, A2, B2 = TQ.compress(A, B, c["policy"], c.get("ratio", 1.0), c.get("energy", 1.0),
                                   c["floor"])
        assert k == c["k"], c
        np.testing.assert_allclose(s, g["s"], atol=1e-12)
        err = np.sum((A @ B - A2 @ B2) ** 2)
        assert abs(err - c["tail_energy"]) <= 1e-12


@pytest.mark.parametrize("seed", range(3))
def test_compression_is_the_best_rank_k_approximation(seed):
    """Eckart-Young: the squared Frobenius error of A'.B' equals the energy of
    the dropped singular values, which equal those of the n x n core
    R_A.R_B^T (from the QRs of A and B^T: a route that never forms A.B)."""
    rng = np.random.default_rng(seed)
    d_in, d_out, n = 96, 80, 12
    A = rng.standard_normal((d_in, n))
    B = rng.standard_normal((n, d_out))
    _, Ra = TQ.thin_qr(A)
    _, Rb = TQ.thin_qr(B.T)
    s_core = np.linalg.svd(Ra @ Rb.T, compute_uv=False)
    for k_pol in ((1, 1.0, 0.8, 1), (0, 0.5, 1.0, 1), (1, 1.0, 0.1, 5)):
        k, s, A2, B2 = TQ.compress(A, B, *k_pol)
        np.testing.assert_allclose(s, s_core, rtol=1e-10)
        err = np.sum((A @ B - A2 @ B2) ** 2)
        np.testing.assert_allclose(err, np.sum(s_core[k:] ** 2), rtol=1e-8, atol=1e-9)
        # the new factors' columns / rows are orthogonal with norms sqrt(sigma)
        np.testing.assert_allclose(A2.T @ A2, np.diag(s[:k]), atol=1e-9 * s[0])
        np.testing.assert_allclose(B2 @ B2.T, np.diag(s[:k]), atol=1e-9 * s[0])
