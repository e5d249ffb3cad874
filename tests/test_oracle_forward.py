"""Pins of the fp64 oracle's forward (runs on the CPU).

Each test ties the oracle to something other than itself: brute force with
scalar loops, torch's own float64 scaled-dot-product attention (masks built
independently with tril/triu or ``is_causal``), closed forms that follow from
the definition (constant V, Q = 0, a single allowed key, equal keys) with the
allowed-key count written out per mask, and invariants (key permutation, a
common shift of every key, mask equivalences).  Sources: P1 §1/§2.1/§2.3,
P4 "usage" (mask variants); addresses in ``oracle/__init__.py``.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import draw, to_f64

MASKS = [("none", 0, 0), ("causal", 0, 0), ("sliding", 0, 0), ("sliding", 1, 0),
         ("sliding", 3, 2), ("sliding", 0, 5), ("sliding", 7, 1000)]


def head(N, d, seed, dtype="f16"):
    t = draw(1, 1, N, d, dtype, seed)
    return to_f64(t["q"][0, 0]), to_f64(t["k"][0, 0]), to_f64(t["v"][0, 0])


def count_allowed(i, N, mode, wl, wr):
    """#A_i written out per mask rule (independent of oracle.allowed_matrix)."""
    if mode == "none":
        return N
    if mode == "causal":
        return i + 1
    return min(i, wl) + 1 + min(N - 1 - i, wr)


# ---------------------------------------------------------------- brute force
def brute_force(q, k, v, scale, mode, wl, wr):
    """Scalar loops with math.fsum/math.exp: the definition on tiny inputs."""
    N, d = q.shape
    sigma = float(np.float32(scale))
    O = [[0.0] * d for _ in range(N)]
    L = [0.0] * N
    for i in range(N):
        keys = []
        for j in range(N):
            if mode == "causal" and j > i:
                continue
            if mode == "sliding" and not (i - wl <= j <= i + wr):
                continue
            keys.append(j)
        s = {j: sigma * math.fsum(float(q[i, t]) * float(k[j, t]) for t in range(d)) for j in keys}
        mx = max(s.values())
        e = {j: math.exp(s[j] - mx) for j in keys}
        tot = math.fsum(e.values())
        for t in range(d):
            O[i][t] = math.fsum(e[j] * float(v[j, t]) for j in keys) / tot
        L[i] = mx + math.log(tot)
    return np.array(O), np.array(L)


@pytest.mark.parametrize("N,d", [(1, 1), (2, 3), (5, 8), (16, 4), (13, 8)])
@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_brute_force_tiny(N, d, mode, wl, wr):
    q, k, v = head(N, d, seed=100 + N * 7 + d)
    scale = 0.37
    o, lse = oracle.forward_head(q, k, v, scale, mode, wl, wr)
    ob, lb = brute_force(q, k, v, scale, mode, wl, wr)
    np.testing.assert_allclose(o, ob, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lb, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------- library routine (torch)
def torch_mask(N, mode, wl, wr):
    if mode == "none":
        return None
    ones = torch.ones(N, N, dtype=torch.bool)
    if mode == "causal":
        return ones.tril()
    return ones.tril(diagonal=wr).triu(diagonal=-wl)


@pytest.mark.parametrize("N,d", [(64, 64), (197, 128), (300, 16)])
@pytest.mark.parametrize("mode,wl,wr", MASKS + [("sliding", 40, 0)])
def test_matches_torch_sdpa(N, d, mode, wl, wr):
    q, k, v = head(N, d, seed=N + d, dtype="bf16")
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.forward_head(q, k, v, scale, mode, wl, wr)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    sig = float(np.float32(scale))
    if mode == "causal":
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=sig)
    else:
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=torch_mask(N, mode, wl, wr), scale=sig)
    np.testing.assert_allclose(o, ref[0, 0].numpy(), rtol=0, atol=1e-12)
    # lse via torch.logsumexp over the masked scores (mask from tril/triu)
    s = sig * (torch.from_numpy(q) @ torch.from_numpy(k).T)
    msk = torch_mask(N, mode, wl, wr)
    if msk is not None:
        s = s.masked_fill(~msk, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_constant_v_gives_that_constant(mode, wl, wr):
    N, d = 90, 16
    q, k, _ = head(N, d, seed=7)
    c = np.linspace(-3.0, 5.0, d)
    v = np.tile(c, (N, 1))
    o, _ = oracle.forward_head(q, k, v, 0.5, mode, wl, wr)
    np.testing.assert_allclose(o, v, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("N", [1, 17, 128])
@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_zero_q_gives_mean_of_allowed_v(N, mode, wl, wr):
    d = 8
    _, k, v = head(N, d, seed=11)
    q = np.zeros((N, d))
    o, lse = oracle.forward_head(q, k, v, 0.125, mode, wl, wr)
    for i in range(N):
        n = count_allowed(i, N, mode, wl, wr)
        assert lse[i] == pytest.approx(math.log(n), abs=1e-13)
        if mode == "none":
            lo, hi = 0, N
        elif mode == "causal":
            lo, hi = 0, i + 1
        else:
            lo, hi = max(0, i - wl), min(N, i + wr + 1)
        assert hi - lo == n
        np.testing.assert_allclose(o[i], v[lo:hi].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_single_allowed_key():
    N, d = 40, 32
    q, k, v = head(N, d, seed=12)
    o, lse = oracle.forward_head(q, k, v, 0.3, "sliding", 0, 0)
    np.testing.assert_array_equal(o, v)
    sig = np.float64(np.float32(0.3))
    np.testing.assert_allclose(lse, sig * np.einsum("nd,nd->n", q, k), rtol=1e-14, atol=1e-14)
    for mode in ("none", "causal", "sliding"):
        o1, l1 = oracle.forward_head(q[:1], k[:1], v[:1], 0.3, mode, 2, 2)
        np.testing.assert_array_equal(o1, v[:1])
        assert l1[0] == pytest.approx(sig * float(q[0] @ k[0]), abs=1e-14)


@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_equal_keys_give_uniform_weights(mode, wl, wr):
    N, d = 70, 8
    q, k, v = head(N, d, seed=13)
    k[:] = k[5]
    o, lse = oracle.forward_head(q, k, v, 0.7, mode, wl, wr)
    sig = np.float64(np.float32(0.7))
    for i in range(N):
        n = count_allowed(i, N, mode, wl, wr)
        assert lse[i] == pytest.approx(sig * float(q[i] @ k[0]) + math.log(n), abs=1e-12)
        A = oracle.allowed_matrix([i], np.arange(N), N, mode, wl, wr)[0]
        np.testing.assert_allclose(o[i], v[A].mean(axis=0), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- invariants
def test_key_permutation_invariance():
    N, d = 150, 32
    q, k, v = head(N, d, seed=14)
    perm = np.random.default_rng(0).permutation(N)
    o, lse = oracle.forward_head(q, k, v, 0.2)
    o2, lse2 = oracle.forward_head(q, k[perm], v[perm], 0.2)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_common_key_shift(mode, wl, wr):
    """K -> K + 1 u^T adds scale*q_i.u to every score of row i: O fixed, lse shifted."""
    N, d = 80, 16
    q, k, v = head(N, d, seed=15)
    u = np.linspace(-1, 1, d)
    o, lse = oracle.forward_head(q, k, v, 0.25, mode, wl, wr)
    o2, lse2 = oracle.forward_head(q, k + u, v, 0.25, mode, wl, wr)
    sig = np.float64(np.float32(0.25))
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + sig * (q @ u), rtol=0, atol=1e-12)


def test_mask_equivalences():
    N, d = 100, 16
    q, k, v = head(N, d, seed=16)
    oc, lc = oracle.forward_head(q, k, v, 0.3, "causal")
    for wl in (N - 1, 10 * N):
        os_, ls = oracle.forward_head(q, k, v, 0.3, "sliding", wl, 0)
        np.testing.assert_array_equal(os_, oc)
        np.testing.assert_array_equal(ls, lc)
    on, ln_ = oracle.forward_head(q, k, v, 0.3, "none")
    os_, ls = oracle.forward_head(q, k, v, 0.3, "sliding", N - 1, N - 1)
    np.testing.assert_array_equal(os_, on)
    np.testing.assert_array_equal(ls, ln_)


def test_row_blocks_over_key_hull_equal_full_head():
    N, d = 333, 16
    t = draw(2, 1, N, d, "bf16", 17)
    Q, K, V = (to_f64(t[x]) for x in ("q", "k", "v"))
    for mode, wl, wr in [("none", 0, 0), ("causal", 0, 0), ("sliding", 40, 0), ("sliding", 5, 9)]:
        Of, Lf = oracle.forward(Q, K, V, 0.2, mode, wl, wr)
        Ob, Lb = oracle.forward(Q, K, V, 0.2, mode, wl, wr, row_block=64)
        np.testing.assert_allclose(Ob, Of, rtol=0, atol=1e-13)
        np.testing.assert_allclose(Lb, Lf, rtol=0, atol=1e-13)


def test_invalid_mask_arguments_are_rejected():
    q, k, v = head(4, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.forward_head(q, k, v, 1.0, "sliding", -1, 0)
    with pytest.raises(ValueError):
        oracle.forward_head(q, k, v, 1.0, "diagonal")


# ------------------------------------------------------------ allowed counts
@pytest.mark.parametrize("N", [1, 2, 7, 64, 65, 300])
@pytest.mark.parametrize("mode,wl,wr", MASKS + [("sliding", 400, 400), ("sliding", 64, 0)])
def test_allowed_count_closed_forms(N, mode, wl, wr):
    """#A_i from oracle.allowed_count equals the count written out per mask
    rule: N without a mask, i + 1 under causal, min(i, wl) + 1 + min(N-1-i, wr)
    for a sliding window (P4 "usage" variants, both window ends inclusive)."""
    got = oracle.allowed_count(N, mode, wl, wr)
    want = np.array([count_allowed(i, N, mode, wl, wr) for i in range(N)])
    assert got.shape == (N,)
    assert np.array_equal(got, want)


def test_allowed_count_catches_a_transposed_sum():
    """Planted mistake: counting per key (columns) instead of per query row.
    Causal column counts are N - j, not i + 1, so the closed form rejects it;
    an asymmetric sliding window is caught the same way."""
    for N, mode, wl, wr in [(50, "causal", 0, 0), (40, "sliding", 5, 1)]:
        r = np.arange(N)
        wrong = oracle.allowed_matrix(r, r, N, mode, wl, wr).sum(axis=0)
        want = np.array([count_allowed(i, N, mode, wl, wr) for i in range(N)])
        assert not np.array_equal(wrong, want)
        assert np.array_equal(oracle.allowed_count(N, mode, wl, wr), want)


@pytest.mark.parametrize("mode,wl,wr", [("none", 0, 0), ("causal", 0, 0), ("sliding", 6, 3)])
def test_multi_head_forward_matches_torch_sdpa(mode, wl, wr):
    """The [B, H, N, d] wrapper (every head, and a listed subset) against
    torch's float64 SDPA over the whole batch at once, with its lse from
    torch.logsumexp: a head written to the wrong (b, h) slot or a subset that
    leaks into unlisted heads fails here."""
    B, H, N, d = 2, 3, 70, 16
    t = draw(B, H, N, d, "bf16", 31)
    Q, K, V = (to_f64(t[x]) for x in ("q", "k", "v"))
    scale = 0.3
    sig = float(np.float32(scale))
    tq, tk, tv = (torch.from_numpy(x) for x in (Q, K, V))
    msk = torch_mask(N, mode, wl, wr)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=msk, scale=sig)
    s = sig * (tq @ tk.transpose(-1, -2))
    if msk is not None:
        s = s.masked_fill(~msk, float("-inf"))
    lref = torch.logsumexp(s, dim=-1).numpy()
    O, L = oracle.forward(Q, K, V, scale, mode, wl, wr)
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, lref, rtol=0, atol=1e-12)
    O2, L2 = oracle.forward(Q, K, V, scale, mode, wl, wr, heads=[(1, 2), (0, 1)])
    for b in range(B):
        for h in range(H):
            if (b, h) in [(1, 2), (0, 1)]:
                np.testing.assert_array_equal(O2[b, h], O[b, h])
                np.testing.assert_array_equal(L2[b, h], L[b, h])
            else:
                assert np.all(np.isnan(O2[b, h])) and np.all(np.isnan(L2[b, h]))
