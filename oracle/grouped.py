"""Grouped-query and packed variable-length attention by the plain definition.
TEST INFRASTRUCTURE ONLY.

Sources are cited as P1..P4 (addresses in ``oracle/__init__.py``).  P1 §5 lists
grouped-query / multi-query attention and variable-length (packed) sequences
among FlashAttention's extensions and gives no formula for either.  Readings
adopted (the plainest ones):

* grouped-query attention: H query heads and H_kv key/value heads, H a multiple
  of H_kv; query head h uses key/value head h // (H // H_kv), so consecutive
  query heads share one (multi-query attention is H_kv = 1, standard attention
  H_kv = H).  Each query head's result is the definition of ``attention.py``
  on its own Q and its key/value head's K and V; the gradient of a shared K or
  V is the sum over the query heads that read it (chain rule through the
  sharing).
* packed variable length: Q is [H, T, d], K and V are [H_kv, T, d]; sequence s
  is rows cu[s] .. cu[s+1] - 1; its rows attend only to its own rows, and the
  mask rule applies to positions counted from the sequence's first row.  Rows
  outside every sequence have no defined result (left NaN here).

Each function only selects heads and row ranges and calls the single-head
definition (``forward_rows`` / ``backward_head``), whose arithmetic is pinned
in ``tests/test_oracle_forward.py`` and ``tests/test_oracle_backward.py``.
"""
from __future__ import annotations

import numpy as np

from .attention import backward_head, forward_rows


def group_size(H: int, H_kv: int) -> int:
    """Query heads per key/value head; H must be a multiple of H_kv >= 1."""
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError(f"H = {H} is not a multiple of H_kv = {H_kv}")
    return H // H_kv


def forward_gqa(Q, K, V, scale: float, mode: str = "none", wl: int = 0, wr: int = 0,
                heads=None, row_block: int = 0):
    """O [B, H, N, d] and lse [B, H, N] for Q [B, H, N, d], K, V [B, H_kv, N, d].

    ``heads`` lists the (b, h) query heads to compute (others stay NaN);
    ``row_block`` > 0 materialises S in blocks of that many query rows.
    """
    B, H, N, d = Q.shape
    g = group_size(H, K.shape[1])
    O = np.full((B, H, N, d), np.nan)
    L = np.full((B, H, N), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    rb = row_block if row_block > 0 else N
    for b, h in todo:
        kv = h // g
        for r0 in range(0, N, rb):
            rows = np.arange(r0, min(N, r0 + rb))
            O[b, h, rows], L[b, h, rows] = forward_rows(rows, Q[b, h], K[b, kv], V[b, kv], scale,
                                                        mode, wl, wr)
    return O, L


def backward_gqa(Q, K, V, dO, scale: float, mode: str = "none", wl: int = 0, wr: int = 0):
    """(dQ [B, H, N, d], dK, dV [B, H_kv, N, d]): dK, dV sum over each group."""
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    g = group_size(H, H_kv)
    dQ = np.empty_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for h in range(H):
            kv = h // g
            dq, dk, dv = backward_head(Q[b, h], K[b, kv], V[b, kv], dO[b, h], scale, mode, wl, wr)
            dQ[b, h] = dq
            dK[b, kv] += dk
            dV[b, kv] += dv
    return dQ, dK, dV


def _sequences(cu, T: int):
    cu = [int(x) for x in cu]
    if cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])) or cu[-1] > T:
        raise ValueError("row offsets must start at 0, not decrease and end at most at T")
    return [(lo, hi) for lo, hi in zip(cu, cu[1:]) if hi > lo]


def forward_varlen(Q, K, V, cu, scale: float, mode: str = "none", wl: int = 0, wr: int = 0,
                   heads=None):
    """O [H, T, d] and lse [H, T] of a packed batch (rows outside sequences: NaN).

    ``heads`` lists the query heads to compute (others stay NaN).
    """
    H, T, d = Q.shape
    g = group_size(H, K.shape[0])
    O = np.full((H, T, d), np.nan)
    L = np.full((H, T), np.nan)
    todo = heads if heads is not None else range(H)
    for lo, hi in _sequences(cu, T):
        rows = np.arange(hi - lo)
        for h in todo:
            kv = h // g
            O[h, lo:hi], L[h, lo:hi] = forward_rows(rows, Q[h, lo:hi], K[kv, lo:hi], V[kv, lo:hi],
                                                    scale, mode, wl, wr)
    return O, L


def backward_varlen(Q, K, V, dO, cu, scale: float, mode: str = "none", wl: int = 0, wr: int = 0):
    """(dQ [H, T, d], dK, dV [H_kv, T, d]) of a packed batch (rows outside sequences: NaN)."""
    H, T, d = Q.shape
    H_kv = K.shape[0]
    g = group_size(H, H_kv)
    dQ = np.full(Q.shape, np.nan)
    dK = np.full(K.shape, np.nan)
    dV = np.full(V.shape, np.nan)
    for lo, hi in _sequences(cu, T):
        dK[:, lo:hi] = 0.0
        dV[:, lo:hi] = 0.0
        for h in range(H):
            kv = h // g
            dq, dk, dv = backward_head(Q[h, lo:hi], K[kv, lo:hi], V[kv, lo:hi], dO[h, lo:hi],
                                       scale, mode, wl, wr)
            dQ[h, lo:hi] = dq
            dK[kv, lo:hi] += dk
            dV[kv, lo:hi] += dv
    return dQ, dK, dV
