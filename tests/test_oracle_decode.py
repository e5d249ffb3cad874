"""Pins of the paged-cache decoding oracle (oracle/decode.py).

Routes other than the oracle's own: the standard-attention oracle on a dense
sequence whose last n_q query rows are the decode queries; torch's CPU
float64 SDPA (grouped-query support, explicit position masks) on keys and
values gathered by torch indexing; invariance under reordering the pages of
the pool; n_q = 1 under a causal mask equals no mask.  A planted mistake (row
and page index swapped when reading the pool) must fail the pins.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

MASKS = [("none", 0, 0), ("causal", 0, 0), ("sliding", 5, 0), ("sliding", 2, 3)]


def make_cache(rng, lens, H_kv, d, page_size, spare=3):
    """A shuffled pool holding each sequence's rows; unused rows and pages are NaN."""
    n_pages_seq = [max(1, -(-L // page_size)) for L in lens]
    n_pages = sum(n_pages_seq) + spare
    perm = rng.permutation(n_pages)
    K = np.full((n_pages, H_kv, page_size, d), np.nan)
    V = np.full((n_pages, H_kv, page_size, d), np.nan)
    table = np.zeros((len(lens), max(n_pages_seq)), dtype=np.int64)
    dense_k, dense_v = [], []
    used = 0
    for s, L in enumerate(lens):
        k = rng.standard_normal((H_kv, L, d))
        v = rng.standard_normal((H_kv, L, d))
        dense_k.append(k)
        dense_v.append(v)
        for pg in range(n_pages_seq[s]):
            phys = perm[used]
            used += 1
            table[s, pg] = phys
            rows = slice(pg * page_size, min(L, (pg + 1) * page_size))
            n = rows.stop - rows.start
            K[phys, :, :n] = k[:, rows]
            V[phys, :, :n] = v[:, rows]
    return K, V, table, dense_k, dense_v


@pytest.mark.parametrize("mode,wl,wr", MASKS)
@pytest.mark.parametrize("n_q", [1, 3])
def test_decode_equals_last_rows_of_dense_attention(mode, wl, wr, n_q):
    rng = np.random.default_rng(1)
    lens, H, H_kv, d, P = [7, 16, 23], 4, 2, 8, 4
    K, V, table, dk, dv = make_cache(rng, lens, H_kv, d, P)
    Q = rng.standard_normal((len(lens), H, n_q, d))
    O, L = oracle.forward_decode(Q, K, V, table, lens, 0.3, mode, wl, wr)
    for s, Ls in enumerate(lens):
        for h in range(H):
            q = rng.standard_normal((Ls, d))  # other rows do not matter
            q[Ls - n_q:] = Q[s, h]
            o_full, l_full = oracle.forward_head(q, dk[s][h // 2], dv[s][h // 2], 0.3, mode, wl, wr)
            assert np.max(np.abs(O[s, h] - o_full[Ls - n_q:])) < 1e-13
            assert np.max(np.abs(L[s, h] - l_full[Ls - n_q:])) < 1e-13


@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_decode_matches_torch_sdpa_on_torch_gathered_pages(mode, wl, wr):
    rng = np.random.default_rng(2)
    lens, H, H_kv, d, P, n_q = [9, 4, 20], 6, 3, 8, 4, 2
    K, V, table, _, _ = make_cache(rng, lens, H_kv, d, P)
    Q = rng.standard_normal((len(lens), H, n_q, d))
    O, _ = oracle.forward_decode(Q, K, V, table, lens, -0.45, mode, wl, wr)
    tK, tV, tT = torch.from_numpy(K), torch.from_numpy(V), torch.from_numpy(table)
    for s, Ls in enumerate(lens):
        j = torch.arange(Ls)
        pages = tT[s, j // P]
        ks = tK[pages, :, j % P].permute(1, 0, 2).contiguous()  # [H_kv, L, d]
        vs = tV[pages, :, j % P].permute(1, 0, 2).contiguous()
        pos = torch.arange(Ls - n_q, Ls)[:, None]
        if mode == "none":
            mask = torch.ones(n_q, Ls, dtype=torch.bool)
        elif mode == "causal":
            mask = j[None, :] <= pos
        else:
            mask = (j[None, :] >= pos - wl) & (j[None, :] <= pos + wr)
        ref = F.scaled_dot_product_attention(torch.from_numpy(Q[s])[None], ks[None], vs[None],
                                             attn_mask=mask, scale=float(np.float32(-0.45)),
                                             enable_gqa=True)[0]
        assert np.max(np.abs(O[s] - ref.numpy())) < 1e-12


def test_page_order_does_not_matter():
    rng = np.random.default_rng(3)
    lens, H, d, P = [13, 5], 2, 8, 4
    K, V, table, _, _ = make_cache(rng, lens, 1, d, P)
    Q = rng.standard_normal((2, H, 1, d))
    O, L = oracle.forward_decode(Q, K, V, table, lens, 0.5, "causal")
    perm = rng.permutation(K.shape[0])
    inv = np.argsort(perm)
    O2, L2 = oracle.forward_decode(Q, K[perm], V[perm], inv[table], lens, 0.5, "causal")
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_single_token_causal_equals_no_mask():
    rng = np.random.default_rng(4)
    K, V, table, _, _ = make_cache(rng, [11, 30], 2, 8, 8)
    Q = rng.standard_normal((2, 4, 1, 8))
    a = oracle.forward_decode(Q, K, V, table, [11, 30], 0.4, "causal")
    b = oracle.forward_decode(Q, K, V, table, [11, 30], 0.4, "none")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_planted_page_misread_fails_the_pin():
    """Reading row j // page_size of page table[j % page_size] gives another result (under a
    window: without a mask it only permutes K and V together, which attention cannot see)."""
    rng = np.random.default_rng(5)
    lens, d, P = [16], 8, 4
    K, V, table, dk, dv = make_cache(rng, lens, 1, d, P, spare=0)
    Q = rng.standard_normal((1, 1, 1, d))
    wrong_k = np.stack([K[table[0, j % P], 0, j // P] for j in range(16)])
    wrong_v = np.stack([V[table[0, j % P], 0, j // P] for j in range(16)])
    q = np.zeros((16, d))
    q[15] = Q[0, 0, 0]
    o_wrong, _ = oracle.forward_rows(np.array([15]), q, wrong_k, wrong_v, 0.5, "sliding", 3, 0)
    O, _ = oracle.forward_decode(Q, K, V, table, lens, 0.5, "sliding", 3, 0)
    assert np.max(np.abs(O[0, 0] - o_wrong)) > 1e-3


def test_short_cache_is_rejected():
    rng = np.random.default_rng(6)
    K, V, table, _, _ = make_cache(rng, [2], 1, 8, 4)
    with pytest.raises(ValueError):
        oracle.forward_decode(rng.standard_normal((1, 1, 3, 8)), K, V, table, [2], 0.5)
