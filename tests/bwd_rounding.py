"""A model of the recomputation backward's inherent rounding error.  TEST INFRASTRUCTURE.

The GPU backward rebuilds P from the saved lse and forms D_i = dO_i . O_i from
the forward's stored O, which is rounded once to the 16-bit input type (P1
§2.4 recomputation; P3 §4 on the backward).  Its products take 16-bit operands:
P for dV = P^T dO, dS = P * (dP - D) for dQ = scale dS K and dK = scale dS^T Q,
and the fp32 results are rounded once to the input type.  This module applies
exactly those roundings to the exact fp64 quantities and reports how far the
result lands from the exact gradient.  When every row has only one or two
allowed keys, dP - D nearly cancels and the rounding of O dominates dS, so the
relative error of dQ and dK can be far above the 1e-2 that holds otherwise;
the parity tests take their per-case bar from this model.

It computes P with its own masked softmax (mask from ``oracle.allowed_matrix``)
and shares no code with the GPU path.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

_DT = {"f16": torch.float16, "bf16": torch.bfloat16}

BASE_BAR = 1e-2    # relative Frobenius bar of every gradient where rounding is not dominant
MARGIN = 1.5       # the GPU's own fp32 summation orders and exp2 on top of the model


def rnd(x: np.ndarray, dtype: str | None) -> np.ndarray:
    """x rounded to nearest-even in the 16-bit type (via float32), back to fp64."""
    if dtype is None:
        return x
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.float32)
    return t.to(_DT[dtype]).to(torch.float64).numpy()


def modelled_grads(q, k, v, do, scale, mode, wl, wr, dtype):
    """(dQ, dK, dV) with the GPU backward's roundings applied to exact fp64 values.

    dtype None applies no rounding and gives the exact gradient.
    """
    N = q.shape[0]
    r = np.arange(N)
    sigma = np.float64(np.float32(scale))
    A = oracle.allowed_matrix(r, r, N, mode, wl, wr)
    S = np.where(A, sigma * (q @ k.T), -np.inf)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    P = E / E.sum(axis=1, keepdims=True)
    o_stored = rnd(P @ v, dtype)                  # the forward's rounded output
    D = (do * o_stored).sum(axis=1)
    dP = do @ v.T
    dS = rnd(P * (dP - D[:, None]), dtype)        # 16-bit operand of dQ and dK
    Pr = rnd(P, dtype)                            # 16-bit operand of dV
    return (rnd(sigma * (dS @ k), dtype), rnd(sigma * (dS.T @ q), dtype), rnd(Pr.T @ do, dtype))


def modelled_error(q, k, v, do, scale, mode, wl, wr, dtype):
    """Relative Frobenius error of the modelled dQ, dK, dV against the exact gradient."""
    exact = oracle.backward_head(q, k, v, do, scale, mode, wl, wr)
    got = modelled_grads(q, k, v, do, scale, mode, wl, wr, dtype)
    out = []
    for g, e in zip(got, exact):
        n = np.linalg.norm(e)
        out.append(float(np.linalg.norm(g - e) / n) if n > 0 else float(np.linalg.norm(g)))
    return out


def grad_bar(q, k, v, do, scale, mode, wl, wr, dtype) -> float:
    """The bar a GPU gradient of this head is held to: 1e-2, or MARGIN times the
    modelled error of the worst of dQ, dK, dV where that is larger."""
    return max(BASE_BAR, MARGIN * max(modelled_error(q, k, v, do, scale, mode, wl, wr, dtype)))


def heads_bar(Q, K, V, dO, scale, mode, wl, wr, dtype, group: int = 1) -> float:
    """grad_bar over the query heads of one batch entry or one packed sequence:
    Q, dO [H, n, d] and K, V [H_kv, n, d], query head h reading key/value
    head h // group.  A gradient of a shared key/value head sums its query
    heads' contributions, whose relative errors the worst head bounds."""
    return max(grad_bar(Q[h], K[h // group], V[h // group], dO[h], scale, mode, wl, wr, dtype)
               for h in range(Q.shape[0]))
