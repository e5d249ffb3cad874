"""Pins of the fp64 oracle's backward (runs on the CPU).

The backward is the exact gradient of the forward definition (P1 §2.4 and P3 §4
only say that it rebuilds P by recomputation).  It is pinned by central finite
differences, by torch autograd through its own float64 attention, and by
invariants that hold for any mask: the rows of dS sum to zero (so the key
gradients sum to zero), the rows of P sum to one (so sum_j dV_j = sum_i dO_i),
a constant V gives zero dQ and dK, and dO = 0 gives zero gradients.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import draw, to_f64

MASKS = [("none", 0, 0), ("causal", 0, 0), ("sliding", 2, 1), ("sliding", 0, 0)]


def head(N, d, seed):
    t = draw(1, 1, N, d, "f16", seed, with_do=True)
    return tuple(to_f64(t[x][0, 0]) for x in ("q", "k", "v", "do"))


@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_finite_differences(mode, wl, wr):
    N, d = 7, 3
    q, k, v, do = head(N, d, seed=31)
    scale = 0.8
    dq, dk, dv = oracle.backward_head(q, k, v, do, scale, mode, wl, wr)

    def f(q_, k_, v_):
        o, _ = oracle.forward_head(q_, k_, v_, scale, mode, wl, wr)
        return float(np.sum(do * o))

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        err = np.linalg.norm(num - grad) / max(np.linalg.norm(grad), 1e-30)
        assert err < 1e-6, (which, err)


@pytest.mark.parametrize("N,d", [(96, 32), (203, 64)])
@pytest.mark.parametrize("mode,wl,wr", MASKS + [("sliding", 30, 0)])
def test_matches_torch_autograd(N, d, mode, wl, wr):
    q, k, v, do = head(N, d, seed=N + d)
    scale = 1.0 / math.sqrt(d)
    sig = float(np.float32(scale))
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    if mode == "causal":
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=sig)
    else:
        m = None
        if mode == "sliding":
            m = torch.ones(N, N, dtype=torch.bool).tril(diagonal=wr).triu(diagonal=-wl)
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=sig)
    o.backward(torch.from_numpy(do))
    dq, dk, dv = oracle.backward_head(q, k, v, do, scale, mode, wl, wr)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=0, atol=1e-10)


@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_invariants(mode, wl, wr):
    N, d = 120, 16
    q, k, v, do = head(N, d, seed=41)
    dq, dk, dv = oracle.backward_head(q, k, v, do, 0.3, mode, wl, wr)
    tol = 1e-10
    assert np.linalg.norm(dk.sum(axis=0)) <= tol * np.linalg.norm(dk)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=0,
                               atol=tol * np.linalg.norm(do))
    vc = np.tile(np.linspace(-1, 2, d), (N, 1))
    dq2, dk2, dv2 = oracle.backward_head(q, k, vc, do, 0.3, mode, wl, wr)
    assert np.linalg.norm(dq2) <= tol * np.linalg.norm(dv2)
    assert np.linalg.norm(dk2) <= tol * np.linalg.norm(dv2)
    z = oracle.backward_head(q, k, v, np.zeros_like(do), 0.3, mode, wl, wr)
    for g in z:
        assert np.all(g == 0.0)
