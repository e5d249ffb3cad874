"""Decoding over a paged K/V cache by the plain definition.  TEST INFRASTRUCTURE ONLY.

Sources are cited as P1..P4 (addresses in ``oracle/__init__.py``).  P1 §5 names
split-KV decoding and paged K/V caches among FlashAttention's extensions; it
gives no layout.  Readings adopted (the plainest ones):

* the cache is a pool of pages, K and V each [n_pages, H_kv, page_size, d];
  key j of sequence s is row j % page_size of page block_table[s][j //
  page_size], for j < seq_lens[s];
* the n_q query tokens of a sequence are its last n_q positions
  L - n_q .. L - 1, and the mask rule of ``attention.py`` applies to those
  positions over the L cached keys (none: all keys; causal: keys up to the
  query's position; sliding: the window around it);
* query head h reads key/value head h // (H // H_kv) (``grouped.py``).

The result is the definition itself: gather the sequence's keys and values
from its pages, then the single-head definition of ``attention.py`` for the
query rows at those positions.  Splitting the keys over workgroups is the
GPU's business and does not appear here.
"""
from __future__ import annotations

import numpy as np

from .attention import forward_rows
from .grouped import group_size


def gather(pool, table_row, L: int, page_size: int):
    """[H_kv, L, d]: the sequence's first L cached rows, page by page."""
    rows = [pool[int(table_row[j // page_size]), :, j % page_size, :] for j in range(L)]
    return np.stack(rows, axis=1) if rows else np.zeros((pool.shape[1], 0, pool.shape[3]))


def forward_decode(Q, K_pool, V_pool, block_table, seq_lens, scale: float, mode: str = "none",
                   wl: int = 0, wr: int = 0):
    """O [n_seqs, H, n_q, d] and lse [n_seqs, H, n_q] (float64).

    Q: [n_seqs, H, n_q, d]; pools [n_pages, H_kv, page_size, d]; each
    seq_lens[s] must be at least n_q.
    """
    n_seqs, H, n_q, d = Q.shape
    page_size = K_pool.shape[2]
    g = group_size(H, K_pool.shape[1])
    O = np.empty((n_seqs, H, n_q, d))
    Lse = np.empty((n_seqs, H, n_q))
    for s in range(n_seqs):
        L = int(seq_lens[s])
        if L < n_q:
            raise ValueError("a sequence's cache must hold at least its n_q query tokens")
        K = gather(K_pool, block_table[s], L, page_size)
        V = gather(V_pool, block_table[s], L, page_size)
        pos = np.arange(L - n_q, L)
        for h in range(H):
            q = np.zeros((L, d))
            q[pos] = Q[s, h]
            O[s, h], Lse[s, h] = forward_rows(pos, q, K[h // g], V[h // g], scale, mode, wl, wr)
    return O, Lse
