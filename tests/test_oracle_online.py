"""The pages' online softmax equals the two-pass definition (CPU, float64).

P1 §2.3 and P3 §2 claim that the block-by-block update with the rescale
factor exp(m - m_new) reproduces the full softmax exactly.  This checks that
claim, under the readings the GPU kernels use (rescale once per key block,
-inf for masked and out-of-range keys, base 0 while a row has seen no allowed
key), for many block shapes including ones that do not divide N and windows
whose leading key blocks are fully masked.

Negative control: P1's CUDA teaching listing applies the rescale inside the
loop over the keys of a block, so history is multiplied by the factor once per
key.  That variant is planted here (CPU only) and must fail.
"""
import numpy as np
import pytest

import oracle
from workloads import draw, to_f64

MASKS = [("none", 0, 0), ("causal", 0, 0), ("sliding", 5, 0), ("sliding", 0, 0),
         ("sliding", 17, 3), ("sliding", 2, 40)]


def head(N, d, seed, outliers=0.0):
    t = draw(1, 1, N, d, "bf16", seed, outlier_frac=outliers, outlier_mul=8.0)
    return to_f64(t["q"][0, 0]), to_f64(t["k"][0, 0]), to_f64(t["v"][0, 0])


@pytest.mark.parametrize("Br", [1, 3, 16, 64])
@pytest.mark.parametrize("Bc", [1, 3, 16, 64])
@pytest.mark.parametrize("mode,wl,wr", MASKS)
def test_online_equals_two_pass(Br, Bc, mode, wl, wr):
    N, d = 100, 8
    q, k, v = head(N, d, seed=Br * 100 + Bc)
    o, lse = oracle.forward_head(q, k, v, 0.4, mode, wl, wr)
    for deferred in (True, False):
        o2, lse2 = oracle.online_forward_head(q, k, v, 0.4, mode, wl, wr, Br=Br, Bc=Bc,
                                              deferred=deferred)
        np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)


def test_online_equals_two_pass_with_outlier_keys():
    """Keys scaled x8 move the running max late in the sequence."""
    N, d = 512, 64
    q, k, v = head(N, d, seed=3, outliers=0.01)
    for mode in ("none", "causal"):
        o, lse = oracle.forward_head(q, k, v, 0.125, mode)
        o2, lse2 = oracle.online_forward_head(q, k, v, 0.125, mode, Br=128, Bc=64)
        np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)


def per_key_rescale_variant(q, k, v, scale, Bc):
    """Planted mistake: the rescale applied once per key inside a block."""
    N, d = q.shape
    sigma = np.float64(np.float32(scale))
    O = np.zeros((N, d))
    for i in range(N):
        m, l, acc = -np.inf, 0.0, np.zeros(d)
        for j0 in range(0, N, Bc):
            s = sigma * (k[j0:j0 + Bc] @ q[i])
            m_new = max(m, s.max())
            corr = np.exp(m - m_new)
            l = l * corr
            for c in range(len(s)):
                p = np.exp(s[c] - m_new)
                l += p
                acc = acc * corr + p * v[j0 + c]
            m = m_new
        O[i] = acc / l
    return O


def test_negative_control_per_key_rescale_fails():
    N, d = 64, 8
    q, k, v = head(N, d, seed=21)
    o, _ = oracle.forward_head(q, k, v, 1.0)
    bad = per_key_rescale_variant(q, k, v, 1.0, Bc=16)
    assert np.max(np.abs(bad - o)) > 1e-3
    # The correct per-block rescale of the same loop structure agrees.
    o2, _ = oracle.online_forward_head(q, k, v, 1.0, Br=1, Bc=16)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-12)
