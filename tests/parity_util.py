"""Helpers for the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (against the fp64 oracle):
  O:    max abs error <= 2e-2 and mean abs error <= 2e-3 (fp16/bf16 outputs);
  lse:  max abs error <= 1e-3 (fp32 dot products and one exp2/log2 rounding;
        typically ~1e-5);
  dQ, dK, dV: relative Frobenius error <= 1e-2 per tensor, or, where the
        16-bit roundings the backward must apply (the stored O, from which D
        is formed, and the products' operands) alone exceed that, 1.5 times
        the error those roundings give in fp64 (``bwd_rounding``).
"""
from __future__ import annotations

import concurrent.futures
import os
import sys

import numpy as np
import torch

import oracle
import exact_attention_14_amd as ea
from bwd_rounding import grad_bar
from workloads import draw, to_f64

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3
GRAD_REL_FRO = 1e-2

MODE_NAMES = ("none", "causal", "sliding")


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_mask(mask):
    mode, wl, wr = ea.mask_args(mask)
    return MODE_NAMES[mode], wl, wr


def gpu(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda")


def run_fwd(inp, mask, scale):
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    o, lse = ea.attn_fwd(q, k, v, mask=mask, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def fwd_errors(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray):
    e = np.abs(o_gpu - o_ref)
    el = np.abs(lse_gpu - lse_ref)
    return float(e.max()), float(e.mean()), float(el.max())


def check_fwd(o_gpu, lse_gpu, o_ref, lse_ref, label=""):
    mx, mean, lmx = fwd_errors(o_gpu, lse_gpu, o_ref, lse_ref)
    say(f"  {label} O max abs {mx:.3e} mean abs {mean:.3e}  lse max abs {lmx:.3e}")
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu))
    assert mx <= O_MAX_ABS, (label, mx)
    assert mean <= O_MEAN_ABS, (label, mean)
    assert lmx <= LSE_MAX_ABS, (label, lmx)
    return mx, mean, lmx


def fwd_case(B, H, N, d, dtype, mask, seed, scale=None, heads=None, row_block=0, **draw_kw):
    """Draw inputs, run the GPU forward on all heads, compare the listed heads (all by default)."""
    scale = (1.0 / np.sqrt(d)) if scale is None else scale
    inp = draw(B, H, N, d, dtype, seed, **draw_kw)
    o, lse = run_fwd(inp, mask, scale)
    name, wl, wr = oracle_mask(mask)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    o_cpu, l_cpu = o.cpu(), lse.cpu()
    O_ref = np.empty((len(todo), N, d))
    L_ref = np.empty((len(todo), N))
    for n, (b, h) in enumerate(todo):
        q, k, v = (to_f64(inp[x][b, h]) for x in ("q", "k", "v"))
        rb = row_block if row_block > 0 else N
        for r0 in range(0, N, rb):
            rows = np.arange(r0, min(N, r0 + rb))
            O_ref[n, rows], L_ref[n, rows] = oracle.forward_rows(rows, q, k, v, scale, name, wl, wr)
    og = np.stack([to_f64(o_cpu[b, h]) for b, h in todo])
    lg = np.stack([l_cpu[b, h].double().numpy() for b, h in todo])
    return check_fwd(og, lg, O_ref, L_ref, label=f"B{B}H{H}N{N}d{d} {dtype} {mask}")


def rel_fro(x: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))


def bwd_case(B, H, N, d, dtype, mask, seed, scale=None, heads=None, tol=None):
    """Forward + backward on the GPU; gradients of the listed heads vs the oracle.

    tol None: each head's bar comes from the rounding model (1e-2 unless its
    roundings alone exceed that)."""
    scale = (1.0 / np.sqrt(d)) if scale is None else scale
    inp = draw(B, H, N, d, dtype, seed, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, mask=mask, scale=scale)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, mask=mask, scale=scale)
    torch.cuda.synchronize()
    name, wl, wr = oracle_mask(mask)
    g = [t.cpu() for t in (dq, dk, dv)]
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    worst = [0.0, 0.0, 0.0]
    bar = 0.0
    for b, h in todo:
        qh, kh, vh, doh = (to_f64(inp[x][b, h]) for x in ("q", "k", "v", "do"))
        ref = oracle.backward_head(qh, kh, vh, doh, scale, name, wl, wr)
        hb = tol if tol is not None else grad_bar(qh, kh, vh, doh, scale, name, wl, wr, dtype)
        bar = max(bar, hb)
        for i in range(3):
            gi = to_f64(g[i][b, h])
            assert np.all(np.isfinite(gi))
            e = rel_fro(gi, ref[i])
            worst[i] = max(worst[i], e)
            assert e <= hb, ("dQ dK dV"[3 * i:3 * i + 2], (b, h), e, hb)
    say(f"  B{B}H{H}N{N}d{d} {dtype} {mask}: rel fro dQ {worst[0]:.3e} dK {worst[1]:.3e} "
        f"dV {worst[2]:.3e} (bar {bar:.3e})")
    return worst, (q, k, v, o, lse, do, dq, dk, dv)


def oracle_threads() -> int:
    """Worker threads for oracle sweeps over many heads (numpy releases the GIL
    in its matrix products and ufuncs); at most 16, the host share of one GPU."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def map_heads(fn, items):
    """fn over items in parallel threads, one BLAS thread each; results in order."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), concurrent.futures.ThreadPoolExecutor(oracle_threads()) as ex:
        return list(ex.map(fn, items))


def fwd_all_heads(inp, o_gpu, lse_gpu, scale, mode, wl, wr, row_block=0, heads=None, label=""):
    """Compare the GPU's O and lse with the oracle over every head (or the listed
    (b, h) pairs), each head's oracle run in a worker thread.

    Asserts the bars over the whole compared tensor: O max abs and the mean abs
    over all of its B*H*N*d elements, lse max abs.  Returns (O max abs, O mean
    abs, lse max abs).
    """
    B, H, N, d = inp["q"].shape
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    rb = row_block if row_block > 0 else N

    def one(bh):
        b, h = bh
        q, k, v = (to_f64(inp[x][b, h]) for x in ("q", "k", "v"))
        og = to_f64(o_gpu[b, h])
        lg = lse_gpu[b, h].double().numpy()
        emax = esum = lmax = 0.0
        finite = bool(np.all(np.isfinite(og)) and np.all(np.isfinite(lg)))
        for r0 in range(0, N, rb):
            rows = np.arange(r0, min(N, r0 + rb))
            o_ref, l_ref = oracle.forward_rows(rows, q, k, v, scale, mode, wl, wr)
            e = np.abs(og[rows] - o_ref)
            emax = max(emax, float(e.max()))
            esum += float(e.sum())
            lmax = max(lmax, float(np.abs(lg[rows] - l_ref).max()))
        return emax, esum, lmax, finite

    res = map_heads(one, todo)
    mx = max(r[0] for r in res)
    mean = sum(r[1] for r in res) / (len(todo) * N * d)
    lmx = max(r[2] for r in res)
    worst_head = todo[int(np.argmax([r[0] for r in res]))]
    say(f"  {label} {len(todo)} heads: O max abs {mx:.3e} (head {worst_head}) mean abs "
        f"{mean:.3e} over {len(todo) * N * d} elements; lse max abs {lmx:.3e}")
    assert all(r[3] for r in res), (label, "non-finite output")
    assert mx <= O_MAX_ABS, (label, mx)
    assert mean <= O_MEAN_ABS, (label, mean)
    assert lmx <= LSE_MAX_ABS, (label, lmx)
    return mx, mean, lmx
