"""CPU checks of the backward rounding model that sets the relaxed gradient bars.

The model (``bwd_rounding``) applies the GPU backward's 16-bit roundings to exact
fp64 quantities.  These tests pin it: without rounding it reproduces the
oracle's exact gradient; it reproduces the ~6.6e-2 error of bf16 with two
allowed keys per row that motivates a wider bar there; and it stays well below
1e-2 wherever rows see many keys, so every such case keeps the 1e-2 bar.
"""
import numpy as np
import pytest

import oracle
from bwd_rounding import BASE_BAR, grad_bar, modelled_error, modelled_grads
from workloads import draw, to_f64


def head(B, H, N, d, dtype, seed, b=0, h=0):
    t = draw(B, H, N, d, dtype, seed, with_do=True)
    return tuple(to_f64(t[x][b, h]) for x in ("q", "k", "v", "do"))


@pytest.mark.parametrize("mode,wl,wr", [("none", 0, 0), ("causal", 0, 0), ("sliding", 3, 1)])
def test_no_rounding_is_the_exact_gradient(mode, wl, wr):
    q, k, v, do = head(1, 1, 40, 16, "f16", 5)
    got = modelled_grads(q, k, v, do, 0.4, mode, wl, wr, None)
    exact = oracle.backward_head(q, k, v, do, 0.4, mode, wl, wr)
    for g, e in zip(got, exact):
        np.testing.assert_allclose(g, e, rtol=0, atol=1e-12)


def test_two_keys_per_row_in_bf16_is_far_above_1e_2():
    """N = 2 causal, bf16, d = 64 (the ragged backward case with seed N + d):
    the rounding of the stored O alone puts dQ/dK near 6.6e-2, which the GPU
    also shows (6.5e-2), so that case needs its own bar."""
    worst = 0.0
    for hh in range(2):
        q, k, v, do = head(1, 2, 2, 64, "bf16", 66, h=hh)
        worst = max(worst, max(modelled_error(q, k, v, do, 1 / 8, "causal", 0, 0, "bf16")))
    assert 4e-2 <= worst <= 1e-1, worst


def test_same_case_in_fp16_keeps_1e_2():
    q, k, v, do = head(1, 2, 2, 64, "f16", 66)
    assert max(modelled_error(q, k, v, do, 1 / 8, "causal", 0, 0, "f16")) < BASE_BAR


@pytest.mark.parametrize("N,mode,wl,wr", [(300, "causal", 0, 0), (300, "none", 0, 0),
                                          (1000, "sliding", 100, 0), (129, "sliding", 9, 4)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_many_keys_per_row_keep_the_base_bar(N, mode, wl, wr, dtype):
    q, k, v, do = head(1, 1, N, 64, dtype, 7)
    assert max(modelled_error(q, k, v, do, 1 / 8, mode, wl, wr, dtype)) < 0.5 * BASE_BAR
    assert grad_bar(q, k, v, do, 1 / 8, mode, wl, wr, dtype) == BASE_BAR


def test_planted_rounding_of_d_is_visible():
    """A model that forgets the rounding of O (D from the exact O) would
    predict a tiny error for the two-key bf16 case: the error really comes
    from D, and the model must carry it."""
    q, k, v, do = head(1, 2, 2, 64, "bf16", 66)
    exact = oracle.backward_head(q, k, v, do, 1 / 8, "causal", 0, 0)
    with_d = modelled_error(q, k, v, do, 1 / 8, "causal", 0, 0, "bf16")
    # Without the rounding of O: only the products' operands and outputs are rounded.
    from bwd_rounding import rnd
    r = np.arange(2)
    A = oracle.allowed_matrix(r, r, 2, "causal")
    S = np.where(A, np.float64(np.float32(1 / 8)) * (q @ k.T), -np.inf)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    P = E / E.sum(axis=1, keepdims=True)
    D = (do * (P @ v)).sum(axis=1)
    dS = rnd(P * (do @ v.T - D[:, None]), "bf16")
    dq = rnd(np.float64(np.float32(1 / 8)) * (dS @ k), "bf16")
    without_d = np.linalg.norm(dq - exact[0]) / np.linalg.norm(exact[0])
    assert with_d[0] > 5 * without_d
