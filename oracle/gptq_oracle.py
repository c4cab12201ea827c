"""Plain fp64 CPU oracle for GPTQ's per-layer solver.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code with it.

Sources (the pages this follows; cited by page, section and equation):

* itwiki "GPTQ" page, section "문제 설정" (problem setting): the layer objective
  argmin over the grid of ||W X - What X||^2.
* same page, section "OBQ에서 GPTQ로" (from OBQ to GPTQ): the OBQ compensation
  delta_F and the Gaussian-elimination downdate of H_F^-1 (the two displayed
  equations), and the three-changes table (fixed column order, lazy batch
  B = 128, Cholesky form of H^-1 with 1% damping).
* same page, section "알고리즘" (Algorithm 1): Q, E; the upper Cholesky factor of
  H^-1; block loop, column loop, in-block update, out-of-block update.
* same page, section "최소 구현" (minimal implementation): the asymmetric per-row
  min/max grid, H = 2 X^T X, damping by percdamp * mean(diag H), the factor
  chain cholesky -> cholesky_inverse -> cholesky(upper).
* same page, section "실무 변형" (practical variants): group quantization with
  group parameters taken from the latest updated weights.
* molayo1419.me blog "GPTQ를 밑바닥부터 구현하며 배운 것들", section 3
  (implementation): H = 2 X^T X and the per-column update rule.

Readings of points the pages leave open are listed in the repository's design
notes; the ones that change arithmetic are restated next to the code below.

Parity pins: every function here is checked in tests against closed forms,
brute force on tiny inputs, the OBQ explicit-inverse form, or invariants.
"""
from __future__ import annotations

import dataclasses
from typing import Iterable, Optional

import numpy as np
import scipy.linalg as sla


# ---------------------------------------------------------------------------
# Hessian and damping
# ---------------------------------------------------------------------------

def hessian(x_chunks: Iterable[np.ndarray], d_col: Optional[int] = None) -> np.ndarray:
    """H = sum over chunks of 2 * X_c^T X_c, in fp64.

    Blog section 3 and the wiki sketch write H = 2 X^T X with X [n x d_in]; the
    sum (not a mean) over calibration rows is taken.  Chunks are read exactly
    as stored (fp16/fp32 values are exact in fp64).
    """
    H = None
    for xc in x_chunks:
        x = np.asarray(xc, dtype=np.float64)
        if H is None:
            H = np.zeros((x.shape[1], x.shape[1]))
        H += 2.0 * (x.T @ x)
    if H is None:
        if d_col is None:
            raise ValueError("no chunks")
        H = np.zeros((d_col, d_col))
    return H


def damp(H: np.ndarray, percdamp: float = 0.01):
    """H_lambda = H + lambda I with lambda = percdamp * mean(diag H).

    Wiki sketch (damping line) and the three-changes table (1% of the mean
    diagonal).  lambda is taken from the undamped diagonal.
    """
    lam = float(percdamp) * float(np.mean(np.diag(H)))
    return H + lam * np.eye(H.shape[0]), lam


# ---------------------------------------------------------------------------
# inverse-Hessian factor
# ---------------------------------------------------------------------------

class NotPositiveDefinite(ArithmeticError):
    pass


def inv_hessian_factor(H_lam: np.ndarray) -> np.ndarray:
    """U upper triangular with U^T U = H_lam^-1, by the sketch's route.

    Wiki "최소 구현": L = cholesky(H); Hinv = cholesky_inverse(L) = L^-T L^-1;
    U = cholesky(Hinv, upper).  Algorithm 1 writes the same object as
    Cholesky(H^-1)^T (the transpose of the lower factor).
    """
    try:
        L = np.linalg.cholesky(H_lam)
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from exc
    Linv = sla.solve_triangular(L, np.eye(L.shape[0]), lower=True)
    Hinv = Linv.T @ Linv
    Hinv = 0.5 * (Hinv + Hinv.T)
    try:
        Lh = np.linalg.cholesky(Hinv)
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from exc
    return Lh.T.copy()


def inv_hessian_factor_reverse(H_lam: np.ndarray) -> np.ndarray:
    """Same U by the reverse-order route: H_lam = Ut Ut^T with Ut upper, U = Ut^-1.

    By uniqueness of the Cholesky factor of H_lam^-1 (positive diagonal) this
    equals :func:`inv_hessian_factor`.  Ut is the lower Cholesky factor of the
    row/column-reversed matrix, reversed back.
    """
    J = H_lam[::-1, ::-1]
    Lr = np.linalg.cholesky(J)
    Ut = Lr[::-1, ::-1]
    return sla.solve_triangular(Ut, np.eye(Ut.shape[0]), lower=False)


# ---------------------------------------------------------------------------
# grid and quantizer (wiki "최소 구현": quantize(), per-row min/max grid)
# ---------------------------------------------------------------------------

def grid_params(w: np.ndarray, bits: int):
    """Asymmetric min/max grid over the last axis of w.

    scale = max(max - min, 1e-8) / maxq; zero = round(-min / scale), with the
    range floor 1e-8 as written; zero is an integer and is not clamped.
    Rounding is round-half-to-even, as torch.round.
    """
    maxq = (1 << bits) - 1
    wmin = np.min(w, axis=-1)
    wmax = np.max(w, axis=-1)
    scale = np.maximum(wmax - wmin, 1e-8) / maxq
    zero = np.rint(-wmin / scale)
    return scale, zero


def quant_codes(w, scale, zero, maxq):
    """c = clamp(round(w / scale) + zero, 0, maxq) -- the sketch's quantize()."""
    return np.clip(np.rint(w / scale) + zero, 0, maxq)


def dequant(c, scale, zero):
    """What = scale * (c - zero)."""
    return scale * (c - zero)


# ---------------------------------------------------------------------------
# GPTQ lazy-batch loop (Algorithm 1 + the sketch's loop + grouping)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class GPTQResult:
    codes: np.ndarray        # uint8 [d_row x d_col]
    scales: np.ndarray       # fp64 [d_row x n_groups]
    zeros: np.ndarray        # int64 [d_row x n_groups]
    w_hat: np.ndarray        # fp64 [d_row x d_col]
    err_sq_sum: float        # sum of squared scaled errors E over all columns
    adopted_codes: int = 0   # forced-replay statistics
    adopted_zeros: int = 0
    max_boundary_dist: float = 0.0


class ReplayMismatch(AssertionError):
    pass


def check_alignment(block_size: int, group_size: int):
    if block_size <= 0:
        raise ValueError("block_size must be positive")
    if group_size < 0:
        raise ValueError("group_size must be >= 0")
    if group_size and not (group_size % block_size == 0 or block_size % group_size == 0):
        raise ValueError("group_size and block_size must divide one another")


def gptq_quantize(W0: np.ndarray, U: np.ndarray, bits: int, group_size: int = 0,
                  block_size: int = 128, replay_codes: Optional[np.ndarray] = None,
                  replay_zeros: Optional[np.ndarray] = None,
                  replay_tol: float = 1e-3) -> GPTQResult:
    """Quantize W0 [d_row x d_col] given U (upper, U^T U = H_lambda^-1).

    Derivation (wiki "OBQ에서 GPTQ로": the compensation equation, and its
    three-changes table; "알고리즘": Algorithm 1).  In the fixed natural order,
    the OBS step for column j has remaining set F = {j, j+1, ..} and moves the
    remaining weights by -(w_j - q_j) / [H_F^-1]_jj * H_F^-1[:, j], with H_F
    the rows and columns F of H_lambda.  For an upper U with U^T U =
    H_lambda^-1 the trailing block satisfies U[F, F]^T U[F, F] = H_F^-1, so
    H_F^-1[:, j] = U[j, j] U[j, F]^T and [H_F^-1]_jj = U[j, j]^2: the step
    reads w_k -= e_j U[j, k] for k > j with the scaled error
    e_j = (w_j - q_j) / U[j, j].  Unrolled, the
    value of column j at its turn is

        w_j = W0_j - sum_{i < j} e_i U[i, j]           (column recursion)

    The lazy batch (change 2) splits this sum at block boundaries: the terms
    of finished blocks are applied to every later column at once as the
    product E_blk U[blk, later], and the terms of the current block are
    gathered when column j is reached (a left-looking evaluation: columns of
    the block are never updated before their turn).  Both orders give the
    same value up to fp64 rounding.

    Grid: per row from W0, or per group at the group's first column from the
    then-current values of the group's columns (wiki "실무 변형": parameters
    from the latest updated weights); block and group sizes divide one another,
    so those columns are the ones inside the block (brought up to date the
    same way) or, for a group wider than the block, fully updated columns at a
    block start.

    Forced replay (``replay_codes`` given): wherever the supplied code differs
    from this oracle's, the difference is accepted only if it is 1 and
    w / scale lies within ``replay_tol`` of the half-integer between the two
    candidates; the supplied code is then adopted and the loop continues.  The
    same applies to zero-points with -min / scale.  Any other difference
    raises ReplayMismatch.
    """
    check_alignment(block_size, group_size)
    U = np.asarray(U, dtype=np.float64)
    Wr = np.array(W0, dtype=np.float64, copy=True)   # W0 minus finished blocks' terms
    d_row, d_col = Wr.shape
    maxq = (1 << bits) - 1
    g = group_size if group_size else d_col
    n_groups = (d_col + g - 1) // g
    codes = np.zeros((d_row, d_col))
    scales = np.zeros((d_row, n_groups))
    zeros = np.zeros((d_row, n_groups))
    stats = {"codes": 0, "zeros": 0, "dist": 0.0}

    def set_grid(gi, cols):
        s, z = grid_params(cols, bits)
        z = _replay_zero(z, -np.min(cols, axis=1) / s, replay_zeros, gi, replay_tol, stats)
        scales[:, gi], zeros[:, gi] = s, z

    if not group_size:
        set_grid(0, Wr)

    err_sq = 0.0
    for b0 in range(0, d_col, block_size):
        b1 = min(b0 + block_size, d_col)
        Eb = np.zeros((d_row, b1 - b0))          # scaled errors of this block so far

        def current(k0, k1, done):
            # columns [k0, k1) after the block's first `done` columns' OBS steps
            return Wr[:, k0:k1] - Eb[:, :done] @ U[b0:b0 + done, k0:k1]

        for j in range(b0, b1):
            done = j - b0
            gi = j // g
            if group_size and j % g == 0:
                set_grid(gi, current(j, min(j + g, d_col), done))
            s, z = scales[:, gi], zeros[:, gi]
            w = current(j, j + 1, done)[:, 0]
            c = _replay_code(quant_codes(w, s, z, maxq), w / s, z, replay_codes, j,
                             replay_tol, stats)
            codes[:, j] = c
            Eb[:, done] = (w - dequant(c, s, z)) / U[j, j]
        err_sq += float(np.sum(Eb * Eb))
        Wr[:, b1:] -= Eb @ U[b0:b1, b1:]

    gidx = np.arange(d_col) // g
    w_hat = dequant(codes, scales[:, gidx], zeros[:, gidx])
    return GPTQResult(codes.astype(np.uint8), scales, zeros.astype(np.int64), w_hat, err_sq,
                      stats["codes"], stats["zeros"], stats["dist"])


def _replay_code(c, v, z, replay_codes, col, tol, stats):
    """Adopt a supplied code that differs by one where v = w / scale lies within
    tol of the half-integer tie between the two candidates (c - zero being the
    rounded value of v); raise ReplayMismatch for any other difference."""
    if replay_codes is None:
        return c
    rc = np.asarray(replay_codes[:, col], dtype=np.float64)
    diff = rc != c
    if not np.any(diff):
        return c
    tie = np.minimum(rc[diff], c[diff]) - z[diff] + 0.5
    dist = np.abs(v[diff] - tie)
    bad = (np.abs(rc[diff] - c[diff]) != 1) | (dist > tol)
    if np.any(bad):
        rows = np.nonzero(diff)[0][bad][:8]
        raise ReplayMismatch(
            f"code mismatch at column {col}, rows {rows.tolist()}: given {rc[rows].tolist()} "
            f"oracle {c[rows].tolist()} w/scale {v[rows].tolist()}")
    stats["dist"] = max(stats["dist"], float(np.max(dist)))
    stats["codes"] += int(np.sum(diff))
    return np.where(diff, rc, c)


def _replay_zero(z, v, replay_zeros, gi, tol, stats):
    """Adopt a supplied zero-point that differs by one where v = -min / scale lies
    within tol of the half-integer tie between the two candidates; raise
    ReplayMismatch for any other difference."""
    if replay_zeros is None:
        return z
    rz = np.asarray(replay_zeros[:, gi], dtype=np.float64)
    diff = rz != z
    if not np.any(diff):
        return z
    tie = np.minimum(rz[diff], z[diff]) + 0.5
    bad = (np.abs(rz[diff] - z[diff]) != 1) | (np.abs(v[diff] - tie) > tol)
    if np.any(bad):
        rows = np.nonzero(diff)[0][bad][:8]
        raise ReplayMismatch(f"zero-point mismatch in group {gi}, rows {rows.tolist()}: "
                             f"given {rz[rows].tolist()} oracle {z[rows].tolist()} "
                             f"-min/scale {v[rows].tolist()}")
    stats["zeros"] += int(np.sum(diff))
    return np.where(diff, rz, z)


# ---------------------------------------------------------------------------
# act-order (wiki "실무 변형": an option of later implementations quantizes the
# columns with the largest Hessian diagonal -- the largest input activations --
# first; with groups it needs a column-to-group map at inference)
# ---------------------------------------------------------------------------

def act_order_perm(H: np.ndarray) -> np.ndarray:
    """Quantization order: position i takes original column perm[i].

    Columns by descending diag(H), compared in H's own precision; equal
    diagonals keep ascending column index (a stable sort), and a NaN diagonal
    counts as -inf.  (Readings: the pages name the criterion only.)
    """
    dg = np.array(np.diag(np.asarray(H)), copy=True)
    dg[np.isnan(dg)] = -np.inf
    return np.argsort(-dg, kind="stable")


@dataclasses.dataclass
class ActOrderResult:
    perm: np.ndarray         # int64 [d_col]: position i quantizes original column perm[i]
    g_idx: np.ndarray        # int64 [d_col]: group of original column j
    codes: np.ndarray        # uint8 [d_row x d_col], original column order
    scales: np.ndarray       # fp64 [d_row x n_groups], groups of consecutive positions
    zeros: np.ndarray        # int64 [d_row x n_groups]
    w_hat: np.ndarray        # fp64 [d_row x d_col], original column order
    err_sq_sum: float
    in_order: GPTQResult     # the loop's own result, in quantization order


def gptq_quantize_act_order(W0: np.ndarray, U_perm: np.ndarray, perm: np.ndarray, bits: int,
                            group_size: int = 0, block_size: int = 128,
                            replay_codes: Optional[np.ndarray] = None,
                            replay_zeros: Optional[np.ndarray] = None,
                            replay_tol: float = 1e-3) -> ActOrderResult:
    """The lazy-batch loop over the columns in the order ``perm``.

    U_perm is the factor of the Hessian with rows and columns in that order
    (H[perm][:, perm]).  Groups are runs of ``group_size`` consecutive
    positions of the quantization order (their parameters come from the
    then-current weights as in natural order), so original column j belongs to
    group g_idx[j] = (position of j) // group_size.  ``replay_codes`` is in the
    original column order; ``replay_zeros`` per group as returned.
    """
    perm = np.asarray(perm, dtype=np.int64)
    d_col = W0.shape[1]
    if sorted(perm.tolist()) != list(range(d_col)):
        raise ValueError("perm is not a permutation of the columns")
    inv = np.empty_like(perm)
    inv[perm] = np.arange(d_col)
    rc = None if replay_codes is None else np.asarray(replay_codes)[:, perm]
    res = gptq_quantize(np.asarray(W0)[:, perm], U_perm, bits, group_size, block_size,
                        replay_codes=rc, replay_zeros=replay_zeros, replay_tol=replay_tol)
    g = group_size if group_size else d_col
    return ActOrderResult(perm, inv // g, res.codes[:, inv], res.scales, res.zeros,
                          res.w_hat[:, inv], res.err_sq_sum, res)


# ---------------------------------------------------------------------------
# packed low-bit codes and the dequantizing product (the consumer of the codes:
# wiki "결과" reports the speed of such kernels; the pages fix no format)
# ---------------------------------------------------------------------------

def pack_codes(codes: np.ndarray, bits: int, perm: Optional[np.ndarray] = None) -> np.ndarray:
    """Row-major bitstream of ``bits``-bit fields in little-endian uint32 words.

    Position i of a row holds column perm[i] (or column i): its field occupies
    bits [bits*i, bits*i + bits) of the row's stream, bit b of the stream being
    bit b % 32 of word b // 32.  Rows are padded to whole 32-code chunks, so a
    row takes ceil(d_col / 32) * bits words.  (Reading: the pages name packed
    low-bit storage but no layout.)
    """
    c = np.asarray(codes, dtype=np.uint64)
    d_row, d_col = c.shape
    if perm is not None:
        c = c[:, np.asarray(perm, dtype=np.int64)]
    if np.any(c >> np.uint64(bits)):
        raise ValueError("code does not fit in the field width")
    words = -(-d_col // 32) * bits
    out = np.zeros((d_row, words), dtype=np.uint64)
    for i in range(d_col):
        off = bits * i
        w, sh = off // 32, off % 32
        out[:, w] |= (c[:, i] << np.uint64(sh)) & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:                       # the field runs into the next word
            out[:, w + 1] |= c[:, i] >> np.uint64(32 - sh)
    return out.astype(np.uint32)


def unpack_codes(packed: np.ndarray, bits: int, d_col: int) -> np.ndarray:
    """Inverse of pack_codes (codes by position)."""
    p = np.asarray(packed, dtype=np.uint64)
    out = np.zeros((p.shape[0], d_col), dtype=np.uint64)
    mask = np.uint64((1 << bits) - 1)
    for i in range(d_col):
        off = bits * i
        w, sh = off // 32, off % 32
        v = p[:, w] >> np.uint64(sh)
        if sh + bits > 32:
            v |= p[:, w + 1] << np.uint64(32 - sh)
        out[:, i] = v & mask
    return out.astype(np.uint8)


def dequant_matmul(packed: np.ndarray, bits: int, scales: np.ndarray, zeros: np.ndarray,
                   group_size: int, X: np.ndarray, d_col: int,
                   perm: Optional[np.ndarray] = None) -> np.ndarray:
    """Y = X What^T with What dequantized from packed codes, in fp64.

    What by position i: scale[:, g] * (code_i - zero[:, g]) with g = i // group_size
    (one group when group_size == 0); position i multiplies column perm[i] of X
    (or column i).  X is [m x d_col]; Y is [m x d_row].
    """
    c = unpack_codes(packed, bits, d_col).astype(np.float64)
    g = group_size if group_size else d_col
    gi = np.arange(d_col) // g
    w_hat = np.asarray(scales, dtype=np.float64)[:, gi] * (c - np.asarray(zeros, dtype=np.float64)[:, gi])
    Xp = np.asarray(X, dtype=np.float64)
    if perm is not None:
        Xp = Xp[:, np.asarray(perm, dtype=np.int64)]
    return Xp @ w_hat.T


# ---------------------------------------------------------------------------
# output error (wiki "문제 설정": ||W X - What X||^2)
# ---------------------------------------------------------------------------

def output_error(W0: np.ndarray, W_hat: np.ndarray, H: np.ndarray) -> float:
    """||X dW^T||_F^2 = 1/2 sum_r dW_r H dW_r^T with H = 2 X^T X undamped."""
    D = np.asarray(W0, dtype=np.float64) - np.asarray(W_hat, dtype=np.float64)
    return 0.5 * float(np.sum((D @ H) * D))


def output_error_direct(W0: np.ndarray, W_hat: np.ndarray, X: np.ndarray) -> float:
    """||W X - What X||^2 evaluated from the calibration rows themselves."""
    D = np.asarray(W0, dtype=np.float64) - np.asarray(W_hat, dtype=np.float64)
    Y = np.asarray(X, dtype=np.float64) @ D.T
    return float(np.sum(Y * Y))


# ---------------------------------------------------------------------------
# RTN baseline (wiki "문제 설정": nearest grid point, no error feedback)
# ---------------------------------------------------------------------------

def rtn(W0: np.ndarray, bits: int, group_size: int = 0):
    """Round-to-nearest on the same grid structure, parameters from W0."""
    W = np.asarray(W0, dtype=np.float64)
    d_row, d_col = W.shape
    maxq = (1 << bits) - 1
    g = group_size if group_size else d_col
    codes = np.zeros_like(W)
    w_hat = np.zeros_like(W)
    for g0 in range(0, d_col, g):
        blk = W[:, g0:g0 + g]
        s, z = grid_params(blk, bits)
        c = quant_codes(blk, s[:, None], z[:, None], maxq)
        codes[:, g0:g0 + g] = c
        w_hat[:, g0:g0 + g] = dequant(c, s[:, None], z[:, None])
    return codes.astype(np.uint8), w_hat


# ---------------------------------------------------------------------------
# OBQ form in the same fixed order (wiki "OBQ에서 GPTQ로", both equations)
# ---------------------------------------------------------------------------

def obq_fixed_order(W0: np.ndarray, H_lam: np.ndarray, bits: int, group_size: int = 0,
                    downdate: str = "inverse"):
    """Per row: quantize weights in natural order with the OBQ compensation.

    For weight q with remaining set F: delta_F = -(w_q - quant(w_q)) /
    [H_F^-1]_qq * (H_F^-1)[:, q]; then q leaves F.  ``downdate="inverse"``
    recomputes H_F^-1 by direct inversion of H_lam[F, F] at every step (brute
    force); ``downdate="gauss"`` removes q's row and column from H^-1 by the
    Gaussian-elimination step H^-1 - H^-1[:, q] H^-1[q, :] / H^-1[q, q].
    Group parameters (if any) come from the current weights at group starts.
    Returns (codes, w_hat).
    """
    W = np.array(W0, dtype=np.float64, copy=True)
    d_row, d_col = W.shape
    maxq = (1 << bits) - 1
    g = group_size if group_size else d_col
    codes = np.zeros((d_row, d_col))
    w_hat = np.zeros((d_row, d_col))
    for r in range(d_row):
        w = W[r].copy()
        if not group_size:
            s, z = grid_params(w, bits)
        Hinv = np.linalg.inv(H_lam)
        for q in range(d_col):
            F = np.arange(q, d_col)
            if downdate == "inverse":
                HF = np.linalg.inv(H_lam[np.ix_(F, F)])
            else:
                HF = Hinv[np.ix_(F, F)]
            if group_size and q % g == 0:
                s, z = grid_params(w[q:q + g], bits)
            c = quant_codes(w[q], s, z, maxq)
            qv = dequant(c, s, z)
            delta = -(w[q] - qv) / HF[0, 0] * HF[:, 0]
            w[F] += delta
            w[q] = qv
            codes[r, q] = c
            w_hat[r, q] = qv
            if downdate == "gauss":
                Hinv = Hinv - np.outer(Hinv[:, q], Hinv[q, :]) / Hinv[q, q]
    return codes.astype(np.uint8), w_hat


def exhaustive_optimum(W0: np.ndarray, H: np.ndarray, bits: int) -> float:
    """Exact minimum of 1/2 sum_r dW_r H dW_r^T over the per-row grid (tiny only)."""
    W = np.asarray(W0, dtype=np.float64)
    d_row, d_col = W.shape
    maxq = (1 << bits) - 1
    if (maxq + 1) ** d_col > 1 << 16:
        raise ValueError("too large for enumeration")
    grid = np.array(np.meshgrid(*[np.arange(maxq + 1)] * d_col, indexing="ij"))
    grid = grid.reshape(d_col, -1).T.astype(np.float64)
    total = 0.0
    for r in range(d_row):
        s, z = grid_params(W[r], bits)
        cand = dequant(grid, s, z)
        D = W[r][None, :] - cand
        total += float(np.min(0.5 * np.sum((D @ H) * D, axis=1)))
    return total


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class LayerSolution:
    H: np.ndarray
    lam: float
    U: np.ndarray
    result: GPTQResult
    err: float


def solve_layer(W0: np.ndarray, x_chunks: Iterable[np.ndarray], bits: int,
                group_size: int = 0, block_size: int = 128,
                percdamp: float = 0.01) -> LayerSolution:
    """H -> damping -> U -> lazy-batch loop -> output error (undamped H)."""
    H = hessian(x_chunks, W0.shape[1])
    H_lam, lam = damp(H, percdamp)
    U = inv_hessian_factor(H_lam)
    res = gptq_quantize(W0, U, bits, group_size, block_size)
    return LayerSolution(H, lam, U, res, output_error(W0, res.w_hat, H))


def solve_layer_act_order(W0: np.ndarray, x_chunks: Iterable[np.ndarray], bits: int,
                          group_size: int = 0, block_size: int = 128,
                          percdamp: float = 0.01) -> LayerSolution:
    """As solve_layer, quantizing the columns in act-order.

    H -> order by its diagonal -> damping of H[perm][:, perm] -> its factor ->
    the loop in that order -> error against W0 with the undamped H (an order-free
    quantity).  ``result`` is an ActOrderResult.
    """
    H = hessian(x_chunks, W0.shape[1])
    perm = act_order_perm(H)
    H_lam, lam = damp(H[np.ix_(perm, perm)], percdamp)
    U = inv_hessian_factor(H_lam)
    res = gptq_quantize_act_order(W0, U, perm, bits, group_size, block_size)
    return LayerSolution(H, lam, U, res, output_error(W0, res.w_hat, H))
