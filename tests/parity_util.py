"""Helpers for the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (against the fp64 oracle):
  O:    max abs error <= 2e-2 and mean abs error <= 2e-3 (fp16/bf16 outputs);
  lse:  max abs error <= 1e-3 (fp32 dot products and one exp2/log2 rounding;
        typically ~1e-5);
  dQ, dK, dV: relative Frobenius error <= 1e-2 per tensor.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import exact_attention_14_amd as ea
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


def bwd_case(B, H, N, d, dtype, mask, seed, scale=None, heads=None, tol=GRAD_REL_FRO):
    """Forward + backward on the GPU; gradients of the listed heads vs the oracle."""
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
    for b, h in todo:
        qh, kh, vh, doh = (to_f64(inp[x][b, h]) for x in ("q", "k", "v", "do"))
        ref = oracle.backward_head(qh, kh, vh, doh, scale, name, wl, wr)
        for i in range(3):
            gi = to_f64(g[i][b, h])
            assert np.all(np.isfinite(gi))
            worst[i] = max(worst[i], rel_fro(gi, ref[i]))
    say(f"  B{B}H{H}N{N}d{d} {dtype} {mask}: rel fro dQ {worst[0]:.3e} dK {worst[1]:.3e} "
        f"dV {worst[2]:.3e}")
    for i in range(3):
        assert worst[i] <= tol, ("dQ dK dV"[3 * i:3 * i + 2], worst[i])
    return worst, (q, k, v, o, lse, do, dq, dk, dv)
