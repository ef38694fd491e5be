"""Independent checks used to pin the oracle.  None of this calls the oracle's
arithmetic: dense linear algebra (numpy/LAPACK), brute-force enumeration and
closed forms derived by hand from the update rule."""
from __future__ import annotations

import numpy as np


def dense_transition(n: int, row_ptr, col_idx) -> np.ndarray:
    """Column-stochastic P: P[v, u] = #(u->v)/outdeg(u); a vertex with no
    out-edge spreads 1/n to every vertex."""
    P = np.zeros((n, n), dtype=np.float64)
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    for u in range(n):
        deg = rp[u + 1] - rp[u]
        if deg == 0:
            P[:, u] = 1.0 / n
        else:
            for v in ci[rp[u]:rp[u + 1]]:
                P[v, u] += 1.0 / deg
    return P


def dense_pagerank(n: int, row_ptr, col_idx, d: float = 0.85) -> np.ndarray:
    """Solve (I - d P) x = (1 - d)/n * 1 with LAPACK."""
    P = dense_transition(n, row_ptr, col_idx)
    A = np.eye(n) - d * P
    return np.linalg.solve(A, np.full(n, (1.0 - d) / n))


def brute_transpose(n: int, row_ptr, col_idx):
    """In-rows by scanning every (u, v) pair: v's sources u in increasing u,
    repeated once per parallel edge."""
    rows = [[] for _ in range(n)]
    for u in range(n):
        for k in range(row_ptr[u], row_ptr[u + 1]):
            rows[col_idx[k]].append(u)
    in_rp = np.zeros(n + 1, dtype=np.int64)
    for v in range(n):
        in_rp[v + 1] = in_rp[v] + len(rows[v])
    in_ci = np.array([u for r in rows for u in sorted(r)], dtype=np.int64)
    return in_rp, in_ci


def star_in_closed_form(N: int, d: float):
    """Leaves -> hub (hub dangling): (x_hub, x_leaf)."""
    den = N + d * (N - 1)
    return (1 + d * (N - 1)) / den, 1.0 / den


def star_out_closed_form(N: int, d: float):
    """Hub -> leaves (leaves dangling): (x_hub, x_leaf)."""
    return 1.0 / (N + d), (N + d - 1) / ((N + d) * (N - 1))


def chain_closed_form(n: int, d: float) -> np.ndarray:
    """0 -> 1 -> ... -> n-1: x_i = k (1 - d^(i+1)) / (1 - d)."""
    k = (1 - d) / (n - d * (1 - d ** n) / (1 - d))
    i = np.arange(n, dtype=np.float64)
    return k * (1 - d ** (i + 1)) / (1 - d)


def dense_adjacency(n: int, row_ptr, col_idx) -> np.ndarray:
    """Boolean A[u, v] = there is an edge u -> v."""
    A = np.zeros((n, n), dtype=bool)
    for u in range(n):
        for k in range(row_ptr[u], row_ptr[u + 1]):
            A[u, col_idx[k]] = True
    return A


def brute_levels(A: np.ndarray, source: int) -> np.ndarray:
    """Smallest k with a length-k walk source -> v, from successive boolean
    products R_{k+1} = R_k A starting at R_0 = e_source; -1 if none."""
    n = A.shape[0]
    level = np.full(n, -1, dtype=np.int64)
    reach = np.zeros(n, dtype=bool)
    reach[source] = True
    for k in range(n):
        level[(level == -1) & reach] = k
        reach = (reach.astype(np.int64) @ A.astype(np.int64)) > 0
    return level


def brute_weak_labels(A: np.ndarray) -> np.ndarray:
    """Smallest vertex id connected to v once directions are ignored, from the
    transitive closure (Warshall) of the symmetrised adjacency."""
    n = A.shape[0]
    C = A | A.T | np.eye(n, dtype=bool)
    for k in range(n):
        C = C | (C[:, k:k + 1] & C[k:k + 1, :])
    return np.array([int(np.flatnonzero(C[v])[0]) for v in range(n)], dtype=np.int64)
