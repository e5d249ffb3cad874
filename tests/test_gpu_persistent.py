"""GPU parity of the persistent forward (attn_fwd_persistent) with attn_fwd.

The persistent launch runs the same per-item code as the ordered one, so its
outputs must agree bit for bit; outputs are pre-filled with NaN so that an
item the work queues failed to hand out shows.  Back-to-back calls check that
every launch leaves the queues empty for the next (an unreset queue would hand
out nothing), including calls with fewer work items than resident
workgroups, and one call is checked against the oracle directly.
"""
import numpy as np
import pytest
import torch

import exact_attention_14_amd as ea
import oracle
from parity_util import check_fwd, gpu, oracle_mask, say
from workloads import draw, draw_grouped, to_f64

pytestmark = pytest.mark.gpu

CASES = [  # (B, H, H_kv, N, d, dtype, mask)
    (4, 32, 32, 4096, 128, "bf16", None),
    (4, 32, 32, 4096, 128, "bf16", "causal"),
    (2, 8, 2, 3000, 128, "f16", "causal"),
    (1, 6, 6, 5000, 64, "bf16", (700, 0)),
    (2, 4, 1, 777, 128, "bf16", (33, 65)),
    (1, 1, 1, 100, 64, "f16", "causal"),
    (3, 2, 2, 64, 128, "bf16", None),
]


def persistent_pair(q, k, v, mask):
    o1 = torch.full_like(q, float("nan"))
    l1 = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
    ea.attn_fwd(q, k, v, mask=mask, out=o1, lse=l1)
    ea.attn_fwd(q, k, v, mask=mask, out=o2, lse=l2, persistent=True)
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2)


@pytest.mark.parametrize("cfg", CASES, ids=[str(c) for c in CASES])
def test_persistent_equals_ordered(cfg):
    B, H, H_kv, N, d, dtype, mask = cfg
    say(f"persistent fwd {cfg}")
    inp = draw_grouped(B, H, H_kv, N, d, dtype, seed=N + H)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    for rep in range(3):  # the queues must be empty again after every launch
        (o1, l1), (o2, l2) = persistent_pair(q, k, v, mask)
        assert torch.equal(o1, o2), f"O differs (call {rep})"
        assert torch.equal(l1, l2), f"lse differs (call {rep})"


def test_persistent_against_the_oracle():
    B, H, N, d = 2, 3, 1000, 128
    inp = draw(B, H, N, d, "bf16", 17)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    o, lse = ea.attn_fwd(q, k, v, mask="causal", persistent=True)
    torch.cuda.synchronize()
    name, wl, wr = oracle_mask("causal")
    scale = 1.0 / np.sqrt(d)
    O_ref, L_ref = oracle.forward(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]), scale,
                                  name, wl, wr)
    check_fwd(to_f64(o.cpu()), lse.cpu().double().numpy(), O_ref, L_ref, label="persistent")


def test_persistent_interleaved_with_other_launches():
    """Persistent launches between ordered forwards and backwards of other sizes
    on the same stream: each still hands out every item exactly once."""
    big = draw(2, 16, 2048, 128, "f16", 3, with_do=True)
    small = draw(1, 2, 300, 64, "bf16", 4)
    qb, kb, vb, dob = (gpu(big[x]) for x in ("q", "k", "v", "do"))
    qs, ks, vs = (gpu(small[x]) for x in ("q", "k", "v"))
    ref_b = ea.attn_fwd(qb, kb, vb, mask="causal")
    ref_s = ea.attn_fwd(qs, ks, vs)
    for _ in range(2):
        ob, lb = ea.attn_fwd(qb, kb, vb, mask="causal", persistent=True)
        ea.attn_bwd(qb, kb, vb, ob, lb, dob, mask="causal")
        os_, ls = ea.attn_fwd(qs, ks, vs, persistent=True)
        torch.cuda.synchronize()
        assert torch.equal(ob, ref_b[0]) and torch.equal(lb, ref_b[1])
        assert torch.equal(os_, ref_s[0]) and torch.equal(ls, ref_s[1])
