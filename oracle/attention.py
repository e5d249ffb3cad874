"""Exact attention by its plain definition, in float64.  TEST INFRASTRUCTURE ONLY.

Sources are cited as P1..P4 (addresses in ``oracle/__init__.py``).

The pages state that the tiled method reaches exactly the result of standard
attention (P1 §2.3, last paragraph; P1 §4.1 table; P4 "principle" section and
conclusion), so the oracle computes that definition and not the tiled
algorithm: S = scale * Q K^T, P = softmax(S) row-wise, O = P V (P1 §1 and the
naive listing of P1 §2.1; P2 "where attention is stuck"; P4 "principle"), with S
and P materialised, plus

* the mask variants of P4 "usage" (none / causal / sliding window), whose bounds
  the pages leave open.  Reading adopted: key j is allowed for query i iff
  none:    always;
  causal:  j <= i;
  sliding: i - window_left <= j <= i + window_right (both ends inclusive).
  Windows are >= 0, so the diagonal is always allowed and no row is empty;
* the per-row statistic saved for the recomputation backward (P1 §2.4 saves O,
  m and l).  Reading adopted: lse = m + ln(l), natural log.

Inputs are the exact fp16/bf16 values the GPU receives, widened to float64
(exact).  The scale is widened from the float32 value the GPU receives.
"""
from __future__ import annotations

import numpy as np

MASK_MODES = ("none", "causal", "sliding")


def _check_mode(mode: str, wl: int, wr: int) -> None:
    if mode not in MASK_MODES:
        raise ValueError(f"unknown mask mode {mode!r}")
    if mode == "sliding" and (wl < 0 or wr < 0):
        raise ValueError("sliding windows must be >= 0")


def _sigma(scale: float) -> np.float64:
    """The scale as the GPU sees it: a float32, widened exactly."""
    return np.float64(np.float32(scale))


def allowed_matrix(rows: np.ndarray, cols: np.ndarray, N: int, mode: str, wl: int = 0,
                   wr: int = 0) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: is key ``cols[c]`` allowed for query ``rows[r]``.

    Mask rules of P4 "usage" under the reading in the module docstring; keys
    at or beyond N are never allowed (the ragged-tail pitfall of P2 "pitfall 1"
    is about tiles, not about the result, which only involves real keys).
    """
    _check_mode(mode, wl, wr)
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    ok = (j >= 0) & (j < N) & (i >= 0) & (i < N)
    if mode == "causal":
        ok &= j <= i
    elif mode == "sliding":
        ok &= (j >= i - wl) & (j <= i + wr)
    return ok


def allowed_count(N: int, mode: str, wl: int = 0, wr: int = 0) -> np.ndarray:
    """#A_i for every query row i, counted from ``allowed_matrix``."""
    r = np.arange(N)
    return allowed_matrix(r, r, N, mode, wl, wr).sum(axis=1)


def _softmax_rows(S: np.ndarray, A: np.ndarray):
    """Two-pass row softmax of the masked scores (P1 §2.1 / §2.3's definition).

    Returns P, m, l with P = exp(S - m) / l, m the row max over allowed keys and
    l the row sum of exp(S - m).  Self-checks the properties every P must have.
    """
    S = np.where(A, S, -np.inf)
    m = S.max(axis=1)
    if not np.all(np.isfinite(m)):
        raise AssertionError("oracle: a query row has no allowed key")
    E = np.exp(S - m[:, None])          # exp(-inf) = 0 for masked keys
    l = E.sum(axis=1)
    P = E / l[:, None]
    # Properties of a softmax row (checked on every block).
    if np.max(np.abs(P.sum(axis=1) - 1.0)) > 1e-12:
        raise AssertionError("oracle: rows of P do not sum to 1")
    if np.any(P < 0.0) or np.any(P[~A] != 0.0):
        raise AssertionError("oracle: P negative or non-zero on a masked key")
    return P, m, l


def _key_hull(rows: np.ndarray, N: int, mode: str, wl: int, wr: int):
    """[lo, hi): the smallest key range holding every allowed key of ``rows``."""
    r0, r1 = int(np.min(rows)), int(np.max(rows))
    if mode == "none":
        return 0, N
    if mode == "causal":
        return 0, r1 + 1
    return max(0, r0 - wl), min(N, r1 + wr + 1)


def forward_rows(rows, q, k, v, scale: float, mode: str = "none", wl: int = 0, wr: int = 0):
    """O and lse of the query rows ``rows`` of one head (float64).

    q, k, v: float64 [N, d].  Only the key hull of the rows is materialised;
    every allowed key lies in that hull, so this equals the full definition.
    Returns (o [len(rows), d], lse [len(rows)]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    N = k.shape[0]
    lo, hi = _key_hull(rows, N, mode, wl, wr)
    cols = np.arange(lo, hi)
    S = _sigma(scale) * (q[rows] @ k[lo:hi].T)
    A = allowed_matrix(rows, cols, N, mode, wl, wr)
    P, m, l = _softmax_rows(S, A)
    return P @ v[lo:hi], m + np.log(l)


def forward_head(q, k, v, scale: float, mode: str = "none", wl: int = 0, wr: int = 0):
    """O [N, d] and lse [N] of one head by the definition, S and P materialised."""
    N = q.shape[0]
    return forward_rows(np.arange(N), q, k, v, scale, mode, wl, wr)


def forward(Q, K, V, scale: float, mode: str = "none", wl: int = 0, wr: int = 0,
            heads=None, row_block: int = 0):
    """All heads (or the listed (b, h) pairs) of [B, H, N, d] float64 inputs.

    ``row_block`` > 0 materialises S in blocks of that many query rows over
    their key hull (needed for long sequences).  Returns (O, lse) float64 of
    shape [B, H, N, d] and [B, H, N]; heads not listed stay NaN.
    """
    B, H, N, d = Q.shape
    O = np.full((B, H, N, d), np.nan)
    L = np.full((B, H, N), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    rb = row_block if row_block > 0 else N
    for b, h in todo:
        for r0 in range(0, N, rb):
            rows = np.arange(r0, min(N, r0 + rb))
            o, lse = forward_rows(rows, Q[b, h], K[b, h], V[b, h], scale, mode, wl, wr)
            O[b, h, rows] = o
            L[b, h, rows] = lse
    return O, L


def backward_head(q, k, v, do, scale: float, mode: str = "none", wl: int = 0, wr: int = 0):
    """Exact gradients of O = softmax(scale Q K^T + mask) V for one head.

    The pages only say that the backward rebuilds S and P from the saved O, m
    and l (P1 §2.4; P3 §4).  The oracle takes the plain gradient of the
    definition instead, with the exact P:
      dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij (= dO_i . O_i),
      dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
    Returns (dq, dk, dv), float64 [N, d] each.
    """
    N = q.shape[0]
    r = np.arange(N)
    sigma = _sigma(scale)
    A = allowed_matrix(r, r, N, mode, wl, wr)
    P, _, _ = _softmax_rows(sigma * (q @ k.T), A)
    o = P @ v
    dv = P.T @ do
    dP = do @ v.T
    D = (P * dP).sum(axis=1)
    D_from_o = (do * o).sum(axis=1)
    if np.max(np.abs(D - D_from_o)) > 1e-10 * max(1.0, float(np.max(np.abs(D)))):
        raise AssertionError("oracle: rowsum(P * dP) differs from rowsum(dO * O)")
    dS = P * (dP - D[:, None])
    return sigma * (dS @ k), sigma * (dS.T @ q), dv

