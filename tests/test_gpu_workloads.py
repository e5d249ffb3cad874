"""GPU parity at the full sizes of the named workloads, in the launch
configuration the benchmark times (one attn_fwd / attn_bwd call over all heads).

Every head of every forward output is compared with the fp64 oracle (run head
by head in worker threads): O max abs and mean abs over all B*H*N*d elements,
lse max abs.  The LLaMA-13B-shaped backward is compared on all 320 heads, with
invariants of the exact gradient over every head checked first.
"""
import numpy as np
import pytest
import torch

import exact_attention_14_amd as ea
import oracle
from parity_util import GRAD_REL_FRO, fwd_all_heads, gpu, map_heads, rel_fro, say
from workloads import (CAUSAL_OUTLIERS_N4096, FULL_N4096, LLAMA13B_CAUSAL_FWDBWD, SLIDING_N32768,
                       make_inputs, to_f64)

pytestmark = pytest.mark.gpu

N_DIES = 8


def mask_of(w):
    return None if w.mask == "none" else ("causal" if w.mask == "causal" else
                                          (w.window_left, w.window_right))


def run_workload_fwd(w, row_block=0):
    say(f"workload {w.name}: drawing inputs")
    inp = make_inputs(w)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    say(f"workload {w.name}: attn_fwd on the GPU")
    o, lse = ea.attn_fwd(q, k, v, mask=mask_of(w), scale=w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    say(f"workload {w.name}: oracle over all {w.B * w.H} heads")
    fwd_all_heads(inp, o.cpu(), lse.cpu(), w.scale, w.mask, w.window_left, w.window_right,
                  row_block=row_block, label=w.name)
    return inp, (q, k, v, o, lse)


def test_full_n4096_bf16():
    run_workload_fwd(FULL_N4096)


def test_causal_outlier_keys_n4096_bf16():
    inp, (q, k, v, o, lse) = run_workload_fwd(CAUSAL_OUTLIERS_N4096)
    # the causal and sliding(N-1, 0) instances agree bitwise at full size
    o2, l2 = ea.attn_fwd(q, k, v, mask=(CAUSAL_OUTLIERS_N4096.N - 1, 0),
                         scale=CAUSAL_OUTLIERS_N4096.scale)
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_sliding_n32768_bf16():
    run_workload_fwd(SLIDING_N32768, row_block=1024)


def die_covering_heads(B, H, n_extra, seed):
    """Heads that every die runs in both backward passes, plus seeded extras.

    The dQ pass deals a contiguous run of B*H/8 query heads to each die, the
    causal dK/dV pass deals head x to die x mod 8 (B*H a multiple of 8): head
    x = i*(B*H/8) + i lands on die i in both."""
    n = B * H
    per = n // N_DIES
    pick = {i * per + i for i in range(N_DIES)}
    rng = np.random.default_rng(seed)
    while len(pick) < N_DIES + n_extra:
        pick.add(int(rng.integers(n)))
    return sorted((x // H, x % H) for x in pick)


def test_llama13b_causal_forward_backward_f16():
    w = LLAMA13B_CAUSAL_FWDBWD
    say(f"workload {w.name}: drawing inputs")
    inp = make_inputs(w)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    say(f"workload {w.name}: attn_fwd + attn_bwd on the GPU")
    o, lse = ea.attn_fwd(q, k, v, mask="causal", scale=w.scale)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, mask="causal", scale=w.scale)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("lse", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), f"{name} has non-finite values"
    # Invariants over every head (any size): sum_j dK_j = 0, sum_j dV_j = sum_i dO_i.
    dk_sum = dk.float().sum(dim=2)
    dk_norm = dk.float().norm(dim=(2, 3))
    dk_ok = (dk_sum.norm(dim=2) <= 1e-2 * dk_norm).cpu()
    dv_sum = dv.float().sum(dim=2)
    do_sum = do.float().sum(dim=2)
    dv_ok = ((dv_sum - do_sum).norm(dim=2) <= 1e-2 * do_sum.norm(dim=2)).cpu()
    bad = [tuple(int(x) for x in bh) for bh in torch.nonzero(~(dk_ok & dv_ok)).tolist()]
    if bad:
        say(f"  invariant violated in heads {bad[:8]} (dK ok: {bool(dk_ok.all())}, "
            f"dV ok: {bool(dv_ok.all())})")
    g = [t.cpu() for t in (o, lse, dq, dk, dv)]
    # The forward: every one of the 320 heads.
    say(f"workload {w.name}: forward oracle over all {w.B * w.H} heads")
    fwd_all_heads(inp, g[0], g[1], w.scale, "causal", 0, 0, label=f"{w.name} fwd")
    # The backward: every one of the 320 heads, a head that breaks an
    # invariant first (so that a failure names the gradient that is off).
    heads = bad[:1] + [(b, h) for b in range(w.B) for h in range(w.H) if (b, h) not in bad[:1]]
    say(f"workload {w.name}: backward oracle over all {len(heads)} heads")

    def one(bh):
        b, h = bh
        qh, kh, vh, doh = (to_f64(inp[x][b, h]) for x in ("q", "k", "v", "do"))
        ref = oracle.backward_head(qh, kh, vh, doh, w.scale, "causal")
        return [rel_fro(to_f64(g[2 + i][b, h]), ref[i]) for i in range(3)]

    errs = map_heads(one, heads)
    worst = np.max(np.array(errs), axis=0)
    worst_head = heads[int(np.argmax(np.max(np.array(errs), axis=1)))]
    say(f"  {len(heads)} heads: worst rel fro dQ {worst[0]:.3e} dK {worst[1]:.3e} dV {worst[2]:.3e} "
        f"(worst head {worst_head})")
    assert not bad, f"gradient invariants violated in heads {bad[:8]}"
    assert worst.max() <= GRAD_REL_FRO, worst
    # No atomics anywhere on the path: a second call agrees bitwise over every
    # element (a race between wavefronts would show up here at any size).
    o2, lse2 = ea.attn_fwd(q, k, v, mask="causal", scale=w.scale)
    dq2, dk2, dv2 = ea.attn_bwd(q, k, v, o, lse, do, mask="causal", scale=w.scale)
    torch.cuda.synchronize()
    for name, a, b_ in (("O", o, o2), ("lse", lse, lse2), ("dQ", dq, dq2), ("dK", dk, dk2),
                        ("dV", dv, dv2)):
        assert torch.equal(a, b_), f"{name} differs between two identical calls"


@pytest.mark.parametrize("mask", [None, (512, 0)], ids=["none", "sliding512"])
def test_f16_forward_full_size_all_heads(mask):
    """The fp16 forward at the headline shape (the fp16 workload is causal):
    B4 H32 N4096 d128, no mask and a (512, 0) window, every head."""
    from workloads import draw
    inp = draw(4, 32, 4096, 128, "f16", seed=23)
    scale = 1.0 / np.sqrt(128)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    o, lse = ea.attn_fwd(q, k, v, mask=mask, scale=scale)
    torch.cuda.synchronize()
    name, wl, wr = ("none", 0, 0) if mask is None else ("sliding", mask[0], mask[1])
    fwd_all_heads(inp, o.cpu(), lse.cpu(), scale, name, wl, wr, row_block=1024 if mask else 0,
                  label=f"f16 B4 H32 N4096 {name}")
