"""fp64 oracle of two-sided adaptive rounding (GPTQ-2D).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's
CPU-baseline leg, never by the GPU library or its binding.

Source: blog.secrett2633.cloud, "[논문리뷰] GPTQ-2D: Cubic-Time Two-Sided Adaptive
Rounding", sections 1-3: round the entries of X in a fixed order, feeding each
entry's error back to the entries not yet rounded, to minimise the two-sided
metric ||A (Z - X) B||_F^2 (A, B fixed and nonsingular); vectorised, the metric is
that of one-sided rounding with the Kronecker-structured matrix built from B^T and
A; entries are grouped by anti-diagonals, which are independent, so the sweep has
depth O(max(m, n)), and the work is O(mn max(m, n)).

The page gives the objective, the Kronecker form, the anti-diagonal grouping and
the complexity but no formulas.  Written out here (and pinned):
  vec(A D B) = (B^T kron A) vec(D) with column-major vec (entry (i, j) at i + m j),
  so the metric is vec(D)^T (P kron Q) vec(D) with Q = A^T A, P = B B^T.  One-sided
  adaptive rounding in the column-major order uses the upper factor of the inverse,
  U = U_P kron U_Q (U_Q^T U_Q = Q^-1, U_P^T U_P = P^-1); entry (i, j) then feeds
  back only to entries (i', j') with i' >= i and j' >= j, so the entries of one
  anti-diagonal i + j = k never feed each other, and sweeping anti-diagonals gives
  exactly the column-major result.  With M = E U_P over the entries already
  rounded, the value entry (i, j) is rounded from is X_ij - (U_Q^T M)_ij (a dot
  product of length i + 1), and its error e_ij = (value - q) / (U_Q[i,i] U_P[j,j])
  adds e_ij U_P[j, j:] to row i of M (length n - j): O(mn (m + n)) in all.

Readings (the page leaves these open): the grid is one asymmetric k-bit min/max grid
for the whole matrix, by the same rule as the one-sided grid (range floored at
1e-8, zero-point round(-min / scale), codes clamped to [0, 2^k - 1]); the factors of
Q and P are given (damping, if any, is the caller's); the error returned is
sum(E^2), which equals the metric for the (possibly damped) Q and P the factors come
from.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

from .gptq_oracle import ReplayMismatch, dequant, grid_params, quant_codes


@dataclasses.dataclass
class Result2D:
    codes: np.ndarray     # uint8 [m x n]
    w_hat: np.ndarray     # fp64 [m x n], scale * (codes - zero)
    E: np.ndarray         # fp64 [m x n], scaled errors
    scale: float
    zero: int
    err: float            # sum(E^2)
    adopted_codes: int = 0


def tensor_grid(X: np.ndarray, bits: int) -> Tuple[float, int]:
    """One grid for the whole matrix, by the one-sided rule applied to all entries."""
    s, z = grid_params(np.asarray(X, dtype=np.float64).reshape(1, -1), bits)
    return float(np.ravel(s)[0]), int(np.ravel(z)[0])


def gptq2d(X: np.ndarray, U_Q: np.ndarray, U_P: np.ndarray, bits: int,
           grid: Optional[Tuple[float, int]] = None, reverse_within_diagonal: bool = False,
           replay_codes: Optional[np.ndarray] = None, replay_tol: float = 1e-3) -> Result2D:
    """Anti-diagonal sweep: for k = 0 .. m + n - 2, round every entry (i, k - i) from
    X_ij - (U_Q^T M)_ij, then add each entry's e_ij U_P[j, j:] to row i of M.

    replay_codes (forced replay, for comparing a path that rounds in another
    precision): where the supplied code differs from this one, it is adopted if
    value / scale lies within replay_tol of a rounding boundary and the code is one
    of the two neighbours; otherwise ReplayMismatch is raised."""
    X = np.asarray(X, dtype=np.float64)
    U_Q = np.asarray(U_Q, dtype=np.float64)
    U_P = np.asarray(U_P, dtype=np.float64)
    m, n = X.shape
    maxq = (1 << bits) - 1
    scale, zero = grid if grid is not None else tensor_grid(X, bits)
    M = np.zeros((m, n))
    E = np.zeros((m, n))
    adopted = 0
    codes = np.zeros((m, n), dtype=np.uint8)
    w_hat = np.zeros((m, n))
    for k in range(m + n - 1):
        rows = range(max(0, k - n + 1), min(k, m - 1) + 1)
        if reverse_within_diagonal:
            rows = reversed(list(rows))
        done = []
        for i in rows:
            j = k - i
            v = X[i, j] - U_Q[:i + 1, i] @ M[:i + 1, j]
            c = quant_codes(np.array([v]), scale, zero, maxq)[0]
            if replay_codes is not None and int(replay_codes[i, j]) != int(c):
                t = v / scale
                near = abs(abs(t - np.floor(t)) - 0.5) <= replay_tol
                cand = {int(np.clip(np.floor(t) + zero, 0, maxq)), int(np.clip(np.ceil(t) + zero, 0, maxq))}
                if not (near and int(replay_codes[i, j]) in cand):
                    raise ReplayMismatch(f"entry ({i}, {j}): code {int(replay_codes[i, j])} vs {int(c)}, "
                                         f"value/scale {t:.6f}")
                c = float(replay_codes[i, j])
                adopted += 1
            q = dequant(float(c), scale, zero)
            codes[i, j] = c
            w_hat[i, j] = q
            E[i, j] = (v - q) / (U_Q[i, i] * U_P[j, j])
            done.append((i, j))
            if reverse_within_diagonal:
                # applying each entry's feedback at once is allowed only because no
                # other entry of the diagonal reads it
                M[i, j:] += E[i, j] * U_P[j, j:]
        if not reverse_within_diagonal:
            for i, j in done:
                M[i, j:] += E[i, j] * U_P[j, j:]
    return Result2D(codes, w_hat, E, scale, zero, float(np.sum(E * E)), adopted)


def two_sided_metric(X: np.ndarray, Z: np.ndarray, A: np.ndarray, B: np.ndarray) -> float:
    """||A (Z - X) B||_F^2."""
    D = np.asarray(Z, dtype=np.float64) - np.asarray(X, dtype=np.float64)
    return float(np.sum((A @ D @ B) ** 2))
