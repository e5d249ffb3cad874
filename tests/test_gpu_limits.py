"""The longest head the boundary accepts, forward and backward, against the oracle.

At d = 128 one tensor's head holds at most 2^23 - 1 rows (just under 2^31
bytes, the reach of the kernels' 32-bit byte offsets within a head); that
length also leaves a ragged last tile.  A (64, 0) sliding window keeps the
work small.  Inputs are drawn on the GPU (seeded) and the rows compared are
copied back for the oracle.  Blocks of rows at the start, across row 2^22
(byte offset 2^30) and at the very end are compared on their local problem:
the block's rows with the 64 rows before it.  That problem holds every key
the block's rows attend to, so their O, lse and dQ are the full problem's;
keys from the block's first row on that are at least 64 rows before its end
(or anywhere in the last block) also have every query that attends to them
inside the block, so their dK and dV are the full problem's too.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_14_amd as ea
import oracle
from bwd_rounding import grad_bar
from parity_util import check_fwd, rel_fro, say
from workloads import draw_on_device, to_f64

pytestmark = pytest.mark.gpu

D = 128
N_MAX = (1 << 31) // (2 * D) - 1  # 8,388,607
WL = 64
R = 1024


def test_longest_head_forward_and_backward():
    dtype, scale, mask = "bf16", 1.0 / math.sqrt(D), (WL, 0)
    say(f"longest head: B1 H1 N{N_MAX} d{D} {dtype}, sliding ({WL}, 0)")
    inp = draw_on_device(1, 1, N_MAX, D, dtype, seed=11, with_do=True)
    q, k, v, do = (inp[x] for x in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, mask=mask, scale=scale)
    o_p, lse_p = ea.attn_fwd(q, k, v, mask=mask, scale=scale, persistent=True)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, mask=mask, scale=scale)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("lse", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), name
    assert torch.equal(o, o_p) and torch.equal(lse, lse_p)  # device-queue forward, same result
    for a in (0, (1 << 22) - R // 2, N_MAX - R):
        base, end = max(0, a - WL), a + R
        ql, kl, vl, dol = (to_f64(t[0, 0, base:end].cpu()) for t in (q, k, v, do))
        rows = np.arange(a - base, end - base)
        o_ref, l_ref = oracle.forward_rows(rows, ql, kl, vl, scale, "sliding", WL, 0)
        check_fwd(to_f64(o[0, 0, a:end].cpu())[None], lse[0, 0, a:end].cpu().double().numpy()[None],
                  o_ref[None], l_ref[None], label=f"rows {a}..{end - 1}")
        gq, gk, gv = oracle.backward_head(ql, kl, vl, dol, scale, "sliding", WL, 0)
        bar = grad_bar(ql, kl, vl, dol, scale, "sliding", WL, 0, dtype)
        kend = end if end == N_MAX else end - WL
        errs = (rel_fro(to_f64(dq[0, 0, a:end].cpu()), gq[a - base:]),
                rel_fro(to_f64(dk[0, 0, a:kend].cpu()), gk[a - base:kend - base]),
                rel_fro(to_f64(dv[0, 0, a:kend].cpu()), gv[a - base:kend - base]))
        say(f"  rows {a}..{end - 1}: rel fro dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e} "
            f"(bar {bar:.3e})")
        assert max(errs) <= bar, (a, errs, bar)
