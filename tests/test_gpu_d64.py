"""GPU parity at full size for head size 64 (the workloads use d = 128): B4 H32
N4096 bf16, no mask and causal, every head of the forward against the fp64
oracle (max and mean abs over all elements), and the causal backward on
heads that every die runs in both passes."""
import numpy as np
import pytest
import torch

import exact_attention_14_amd as ea
import oracle
from bwd_rounding import grad_bar
from parity_util import fwd_all_heads, gpu, map_heads, rel_fro, say
from test_gpu_workloads import die_covering_heads
from workloads import draw, to_f64

pytestmark = pytest.mark.gpu

B, H, N, D = 4, 32, 4096, 64
SCALE = 1.0 / np.sqrt(D)


@pytest.fixture(scope="module")
def inputs():
    say(f"d = 64 full size: drawing B{B} H{H} N{N} inputs")
    return draw(B, H, N, D, "bf16", seed=21, with_do=True)


@pytest.mark.parametrize("mask", [None, "causal"])
def test_d64_forward_all_heads(inputs, mask):
    q, k, v = (gpu(inputs[x]) for x in ("q", "k", "v"))
    o, lse = ea.attn_fwd(q, k, v, mask=mask, scale=SCALE)
    torch.cuda.synchronize()
    name = "none" if mask is None else "causal"
    fwd_all_heads(inputs, o.cpu(), lse.cpu(), SCALE, name, 0, 0, label=f"d64 {name}")


def test_d64_causal_backward_die_covering_heads(inputs):
    q, k, v, do = (gpu(inputs[x]) for x in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, mask="causal", scale=SCALE)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, mask="causal", scale=SCALE)
    torch.cuda.synchronize()
    for name, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), name
    g = [t.cpu() for t in (dq, dk, dv)]
    heads = die_covering_heads(B, H, 4, 21)
    say(f"d64 causal backward: oracle on heads {heads}")

    def one(bh):
        b, h = bh
        qh, kh, vh, doh = (to_f64(inputs[x][b, h]) for x in ("q", "k", "v", "do"))
        ref = oracle.backward_head(qh, kh, vh, doh, SCALE, "causal")
        bar = grad_bar(qh, kh, vh, doh, SCALE, "causal", 0, 0, "bf16")
        return [rel_fro(to_f64(g[i][b, h]), ref[i]) for i in range(3)], bar

    for bh, (e, bar) in zip(heads, map_heads(one, heads)):
        say(f"  head {bh} rel fro dQ {e[0]:.3e} dK {e[1]:.3e} dV {e[2]:.3e} (bar {bar:.3e})")
        assert max(e) <= bar, (bh, e, bar)
