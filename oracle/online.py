"""The tiled online-softmax method itself, in float64.  TEST INFRASTRUCTURE ONLY.

Sources are cited as P1..P4 (addresses in ``oracle/__init__.py``).

This is not what the GPU is compared against (that is the definition in
``attention.py``).  It exists so that a test can check the pages' central claim
-- the block-by-block online softmax equals the two-pass softmax -- under the
readings adopted for the GPU kernels, before any kernel is trusted:

* blocks: Q in Br-row blocks, K/V in Bc-row blocks (P1 §2.2);
* per key block, per row (P1 §2.3 update equations; P3 §2):
    m_new = max(m, rowmax S_blk)
    corr  = exp(m - m_new)             -- applied once per key block
    l_new = corr * l + rowsum exp(S_blk - m_new)
    normalised form (P1 §2.3):   O = (corr * l * O + exp(S_blk - m_new) V) / l_new
    deferred form   (P3 §2/§3):  acc = corr * acc + exp(S_blk - m_new) V,
                                  O = acc / l at the end;
* masked keys score -inf (P4 "usage" variants, bounds as in ``attention.py``);
  while a row has seen no allowed key its max is -inf, and the exponent base
  is taken as 0 so that exp(-inf - base) = 0 and no NaN appears (the NaN
  hazard P4 "performance data" reports at window/tile boundaries);
* lse = m + ln(l) (P1 §2.4 keeps m and l for the backward).
"""
from __future__ import annotations

import numpy as np

from .attention import allowed_matrix, _sigma


def online_forward_head(q, k, v, scale: float, mode: str = "none", wl: int = 0, wr: int = 0,
                        Br: int = 64, Bc: int = 64, deferred: bool = True):
    """One head by the tiled online softmax; returns (o [N, d], lse [N])."""
    N, d = q.shape
    sigma = _sigma(scale)
    O = np.zeros((N, d))
    lse = np.zeros(N)
    for i0 in range(0, N, Br):
        rows = np.arange(i0, min(N, i0 + Br))
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), d))
        for j0 in range(0, N, Bc):
            cols = np.arange(j0, min(N, j0 + Bc))
            s = sigma * (q[rows] @ k[cols].T)
            s = np.where(allowed_matrix(rows, cols, N, mode, wl, wr), s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            base = np.where(np.isfinite(m_new), m_new, 0.0)
            corr = np.exp(m - base)
            p = np.exp(s - base[:, None])
            l_new = corr * l + p.sum(axis=1)
            if deferred:
                acc = corr[:, None] * acc + p @ v[cols]
            else:
                num = (corr * l)[:, None] * acc + p @ v[cols]
                acc = np.divide(num, l_new[:, None], out=np.zeros_like(num),
                                where=l_new[:, None] > 0)
            m, l = m_new, l_new
        O[rows] = acc / l[:, None] if deferred else acc
        lse[rows] = m + np.log(l)
    return O, lse
