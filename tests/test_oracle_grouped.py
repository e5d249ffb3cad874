"""Pins of the grouped-query and packed variable-length oracle (oracle/grouped.py).

Each pin reaches the expected value by another route than the oracle:
  * torch's CPU float64 scaled-dot-product attention with its own grouped-query
    support (``enable_gqa``) and its autograd, for the forward and backward of
    shared key/value heads;
  * the standard-attention oracle on key/value heads repeated along the head
    axis (what sharing means), with the plain special case H_kv = H;
  * for packed batches, one softmax over the whole packed T x T score matrix
    under a block-diagonal mask (scipy's softmax and logsumexp), torch
    autograd through the same masked matrix, and finite differences;
  * closed forms for one-row sequences.
Planted mistakes (the wrong key/value head, attention across sequence
boundaries) must make the matching pin fail.
"""
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle

MASKS = [("none", 0, 0), ("causal", 0, 0), ("sliding", 3, 1), ("sliding", 0, 5)]


def rand(rng, *shape):
    return rng.standard_normal(shape)


def torch_mask(N, mode, wl, wr):
    r = np.arange(N)
    return torch.from_numpy(oracle.allowed_matrix(r, r, N, mode, wl, wr))


@pytest.mark.parametrize("H,H_kv", [(4, 4), (4, 2), (6, 3), (8, 1)])
@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_gqa_matches_torch_sdpa_grouped(H, H_kv, mode, wl, wr):
    rng = np.random.default_rng(11)
    B, N, d = 2, 13, 8
    Q, K, V = rand(rng, B, H, N, d), rand(rng, B, H_kv, N, d), rand(rng, B, H_kv, N, d)
    scale = 0.37
    O, L = oracle.forward_gqa(Q, K, V, scale, mode, wl, wr)
    tq, tk, tv = (torch.from_numpy(x) for x in (Q, K, V))
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch_mask(N, mode, wl, wr),
                                         scale=float(np.float32(scale)), enable_gqa=True)
    assert np.max(np.abs(O - ref.numpy())) < 1e-12
    # lse by the library's logsumexp over the masked scores of each head
    for b in range(B):
        for h in range(H):
            S = float(np.float32(scale)) * Q[b, h] @ K[b, h // (H // H_kv)].T
            S[~torch_mask(N, mode, wl, wr).numpy()] = -np.inf
            assert np.max(np.abs(L[b, h] - scipy.special.logsumexp(S, axis=1))) < 1e-12


def test_gqa_equals_standard_attention_on_repeated_kv_heads():
    rng = np.random.default_rng(12)
    B, H, H_kv, N, d = 2, 6, 2, 9, 8
    Q, K, V = rand(rng, B, H, N, d), rand(rng, B, H_kv, N, d), rand(rng, B, H_kv, N, d)
    O, L = oracle.forward_gqa(Q, K, V, 0.5, "causal")
    Kr, Vr = np.repeat(K, H // H_kv, axis=1), np.repeat(V, H // H_kv, axis=1)
    O2, L2 = oracle.forward(Q, Kr, Vr, 0.5, "causal")
    assert np.array_equal(O, O2) and np.array_equal(L, L2)
    # H_kv = H is standard attention
    O3, L3 = oracle.forward_gqa(Q, Kr, Vr, 0.5, "causal")
    assert np.array_equal(O3, O2) and np.array_equal(L3, L2)


def test_planted_wrong_kv_head_fails_the_pin():
    """Reading key/value head h % H_kv instead of h // group changes the result."""
    rng = np.random.default_rng(13)
    B, H, H_kv, N, d = 1, 4, 2, 7, 8
    Q, K, V = rand(rng, B, H, N, d), rand(rng, B, H_kv, N, d), rand(rng, B, H_kv, N, d)
    O, _ = oracle.forward_gqa(Q, K, V, 0.5)
    wrong = np.stack([np.stack([oracle.forward_head(Q[0, h], K[0, h % H_kv], V[0, h % H_kv], 0.5)[0]
                                for h in range(H)])])
    assert np.max(np.abs(O - wrong)) > 1e-3


@pytest.mark.parametrize("H,H_kv", [(4, 2), (3, 1)])
@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_gqa_backward_matches_torch_autograd(H, H_kv, mode, wl, wr):
    rng = np.random.default_rng(14)
    B, N, d = 2, 11, 8
    Q, K, V = rand(rng, B, H, N, d), rand(rng, B, H_kv, N, d), rand(rng, B, H_kv, N, d)
    dO = rand(rng, B, H, N, d)
    scale = -0.3
    dQ, dK, dV = oracle.backward_gqa(Q, K, V, dO, scale, mode, wl, wr)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (Q, K, V))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch_mask(N, mode, wl, wr),
                                       scale=float(np.float32(scale)), enable_gqa=True)
    o.backward(torch.from_numpy(dO))
    for mine, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) < 1e-11


def test_gqa_backward_finite_differences():
    """d(sum(dO * O)) / dK and / dV of a shared head, by central differences."""
    rng = np.random.default_rng(15)
    B, H, H_kv, N, d = 1, 4, 2, 5, 4
    Q, K, V = rand(rng, B, H, N, d), rand(rng, B, H_kv, N, d), rand(rng, B, H_kv, N, d)
    dO = rand(rng, B, H, N, d)
    _, dK, dV = oracle.backward_gqa(Q, K, V, dO, 0.5, "causal")

    def f(K_, V_):
        return float(np.sum(dO * oracle.forward_gqa(Q, K_, V_, 0.5, "causal")[0]))

    eps = 1e-6
    for (b, h, i, j) in [(0, 0, 0, 0), (0, 1, 3, 2), (0, 1, 4, 3), (0, 0, 2, 1)]:
        Kp, Km = K.copy(), K.copy()
        Kp[b, h, i, j] += eps
        Km[b, h, i, j] -= eps
        assert abs((f(Kp, V) - f(Km, V)) / (2 * eps) - dK[b, h, i, j]) < 1e-7
        Vp, Vm = V.copy(), V.copy()
        Vp[b, h, i, j] += eps
        Vm[b, h, i, j] -= eps
        assert abs((f(K, Vp) - f(K, Vm)) / (2 * eps) - dV[b, h, i, j]) < 1e-7


def packed_allowed(cu, T, mode, wl, wr):
    """T x T: same sequence and the mask rule on positions within the sequence."""
    seq = np.full(T, -1)
    start = np.zeros(T, dtype=np.int64)
    for s, (lo, hi) in enumerate(zip(cu, cu[1:])):
        seq[lo:hi] = s
        start[lo:hi] = lo
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    ok = (seq[:, None] == seq[None, :]) & (seq[:, None] >= 0)
    pi, pj = i - start[:, None], j - start[None, :]
    if mode == "causal":
        ok &= pj <= pi
    elif mode == "sliding":
        ok &= (pj >= pi - wl) & (pj <= pi + wr)
    return ok


CUS = [[0, 5, 6, 6, 14, 20], [0, 20], [0, 1, 2, 3, 17]]


@pytest.mark.parametrize("cu", CUS)
@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_varlen_matches_one_block_diagonal_softmax(cu, mode, wl, wr):
    rng = np.random.default_rng(16)
    H, H_kv, T, d = 4, 2, cu[-1], 8
    Q, K, V = rand(rng, H, T, d), rand(rng, H_kv, T, d), rand(rng, H_kv, T, d)
    scale = 0.41
    O, L = oracle.forward_varlen(Q, K, V, cu, scale, mode, wl, wr)
    A = packed_allowed(cu, T, mode, wl, wr)
    s32 = float(np.float32(scale))
    for h in range(H):
        S = s32 * Q[h] @ K[h // 2].T
        S[~A] = -np.inf
        P = scipy.special.softmax(S, axis=1)
        lse = scipy.special.logsumexp(S, axis=1)
        assert np.max(np.abs(O[h] - P @ V[h // 2])) < 1e-12
        assert np.max(np.abs(L[h] - lse)) < 1e-12


def test_planted_attention_across_sequences_fails_the_pin():
    """Softmax over the whole packed row (no block-diagonal mask) is a different result."""
    rng = np.random.default_rng(17)
    cu, T = [0, 6, 13], 13
    Q, K, V = rand(rng, 1, T, 8), rand(rng, 1, T, 8), rand(rng, 1, T, 8)
    O, _ = oracle.forward_varlen(Q, K, V, cu, 0.5)
    leak, _ = oracle.forward_head(Q[0], K[0], V[0], 0.5)
    assert np.max(np.abs(O[0] - leak)) > 1e-3


def test_varlen_single_sequence_is_the_fixed_length_result():
    rng = np.random.default_rng(18)
    H, H_kv, T, d = 4, 1, 17, 8
    Q, K, V = rand(rng, H, T, d), rand(rng, H_kv, T, d), rand(rng, H_kv, T, d)
    O, L = oracle.forward_varlen(Q, K, V, [0, T], 0.3, "causal")
    O2, L2 = oracle.forward_gqa(Q[None], K[None], V[None], 0.3, "causal")
    assert np.array_equal(O, O2[0]) and np.array_equal(L, L2[0])


def test_varlen_one_row_and_empty_sequences():
    """A one-row sequence returns its own V row and lse = scale q.k; empty ones change nothing."""
    rng = np.random.default_rng(19)
    T, d = 6, 8
    Q, K, V = rand(rng, 2, T, d), rand(rng, 2, T, d), rand(rng, 2, T, d)
    cu = [0, 0, 1, 1, 6, 6]
    O, L = oracle.forward_varlen(Q, K, V, cu, 0.25, "causal")
    s32 = float(np.float32(0.25))
    for h in range(2):
        assert np.array_equal(O[h, 0], V[h, 0])
        assert abs(L[h, 0] - s32 * Q[h, 0] @ K[h, 0]) < 1e-14
    O2, _ = oracle.forward_varlen(Q, K, V, [0, 1, 6], 0.25, "causal")
    assert np.array_equal(O, O2)
    # rows outside every sequence stay undefined
    O3, _ = oracle.forward_varlen(Q, K, V, [0, 2, 4], 0.25)
    assert np.all(np.isnan(O3[:, 4:])) and not np.any(np.isnan(O3[:, :4]))


@pytest.mark.parametrize("cu", CUS)
@pytest.mark.parametrize("mode,wl,wr", MASKS[:3])
def test_varlen_backward_matches_torch_autograd_on_the_packed_matrix(cu, mode, wl, wr):
    rng = np.random.default_rng(20)
    H, H_kv, T, d = 4, 2, cu[-1], 8
    Q, K, V, dO = rand(rng, H, T, d), rand(rng, H_kv, T, d), rand(rng, H_kv, T, d), rand(rng, H, T, d)
    scale = 0.35
    dQ, dK, dV = oracle.backward_varlen(Q, K, V, dO, cu, scale, mode, wl, wr)
    tq, tk, tv = (torch.from_numpy(x[None]).requires_grad_(True) for x in (Q, K, V))
    A = torch.from_numpy(packed_allowed(cu, T, mode, wl, wr))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=A, scale=float(np.float32(scale)),
                                       enable_gqa=True)
    o.backward(torch.from_numpy(dO[None]))
    covered = np.zeros(T, dtype=bool)
    covered[cu[0]:cu[-1]] = True
    for mine, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
        assert np.max(np.abs(mine[:, covered] - ref.numpy()[0][:, covered])) < 1e-11


def test_bad_offsets_and_groups_are_rejected():
    z = np.zeros((4, 5, 8))
    with pytest.raises(ValueError):
        oracle.forward_varlen(z, z[:3], z[:3], [0, 5], 0.5)
    with pytest.raises(ValueError):
        oracle.forward_varlen(z, z, z, [0, 3, 2], 0.5)
    with pytest.raises(ValueError):
        oracle.forward_varlen(z, z, z, [1, 5], 0.5)
    with pytest.raises(ValueError):
        oracle.forward_varlen(z, z, z, [0, 6], 0.5)
