"""GPU parity of the forward against the fp64 oracle (element by element).

Small and ragged shapes that span several tiles, every mask, both storage
types and both head sizes are compared in full; the properties that hold at
any size (mask equivalences, determinism, closed forms) are checked on the
GPU's own outputs.  Full-size workloads live in test_gpu_workloads.py.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_14_amd as ea
from parity_util import check_fwd, fwd_case, gpu, oracle_mask, run_fwd, say
from workloads import SINGLE_HEAD_N256, draw, make_inputs, to_f64

import oracle

pytestmark = pytest.mark.gpu

MASKS = [None, "causal", (0, 0), (1, 0), (5, 3), (63, 0), (64, 0), (65, 1), (127, 128),
         (200, 0), (4096, 4096)]


def test_single_head_n256_workload():
    w = SINGLE_HEAD_N256
    say(f"workload {w.name}")
    inp = make_inputs(w)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    o, lse = ea.attn_fwd(q, k, v, mask=None, scale=w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]), w.scale)
    check_fwd(to_f64(o.cpu()), lse.cpu().double().numpy(), o_ref, l_ref, w.name)


@pytest.mark.parametrize("N", [1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 333])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_lengths_all_masks(N, dtype, d):
    for mask in [None, "causal", (5, 3), (64, 0)]:
        say(f"N={N} d={d} {dtype} mask={mask}")
        fwd_case(1, 2, N, d, dtype, mask, seed=N * 31 + d)


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_windows_and_tile_edges(mask, dtype):
    say(f"N=1000 mask={mask} {dtype}")
    fwd_case(2, 2, 1000, 128, dtype, mask, seed=7)


@pytest.mark.parametrize("N", [3333, 4096])
def test_multi_tile_heads(N):
    for mask in [None, "causal", (300, 0)]:
        say(f"N={N} mask={mask}")
        fwd_case(1, 3, N, 128, "bf16", mask, seed=N)


def test_outlier_keys_move_the_running_max():
    say("outlier keys, N=2048 causal and none")
    for mask in [None, "causal"]:
        fwd_case(1, 4, 2048, 128, "bf16", mask, seed=99, outlier_frac=0.01, outlier_mul=8.0)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mask", [None, "causal"])
def test_running_max_jumps_beyond_the_optimistic_bound(dtype, mask):
    """Scores that rise in steps far larger than the optimistic bound on a
    probability (2^32 for bf16, 2^15 for fp16, in exp2 units): every step must
    take the exact-max path (a probability formed against the old max would
    overflow), and smaller steps below the bound must not disturb the result.
    Q rows are all e_0 and K's first column rises in steps within and across
    key tiles, so each row's softmax concentrates on its latest keys."""
    N, d = 700, 64
    inp = draw(1, 2, N, d, dtype, 77)
    q, k, v = inp["q"].clone(), inp["k"].clone(), inp["v"].clone()
    q.zero_()
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    # scale 1: score = k[:, 0]; exp2 units multiply by log2(e) = 1.44
    steps = {100: 30.0, 160: 60.0, 161: 64.0, 300: 120.0, 333: 124.0, 500: 200.0, 640: 204.0}
    level = 0.0
    for j in range(N):
        level = steps.get(j, level)
        k[..., j, 0] = level
    if dtype == "f16":  # keep the largest score (and q.k) inside fp16's range
        k[..., 0] = k[..., 0] / 8.0
    scale = 1.0
    o, lse = run_fwd({"q": q, "k": k, "v": v}, mask, scale)
    name, wl, wr = oracle_mask(mask)
    O_ref = np.empty((2, N, d))
    L_ref = np.empty((2, N))
    for h in range(2):
        O_ref[h], L_ref[h] = oracle.forward_head(to_f64(q[0, h]), to_f64(k[0, h]), to_f64(v[0, h]),
                                                 scale, name, wl, wr)
    check_fwd(to_f64(o[0].cpu()), lse[0].cpu().double().numpy(), O_ref, L_ref,
              label=f"max jumps {dtype} {mask}")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 1.7, 1e-3])
def test_scales(scale):
    say(f"scale={scale}")
    for mask in [None, "causal", (10, 2)]:
        fwd_case(1, 2, 300, 64, "f16", mask, seed=5, scale=scale)


def test_mask_equivalences_are_bitwise():
    N = 777
    inp = draw(2, 3, N, 128, "bf16", 11)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    oc, lc = ea.attn_fwd(q, k, v, mask="causal")
    for wl in (N - 1, N, 10 * N):
        os_, ls = ea.attn_fwd(q, k, v, mask=(wl, 0))
        assert torch.equal(oc, os_) and torch.equal(lc, ls)
    on, ln_ = ea.attn_fwd(q, k, v, mask=None)
    os_, ls = ea.attn_fwd(q, k, v, mask=(N - 1, N - 1))
    assert torch.equal(on, os_) and torch.equal(ln_, ls)


def test_forward_is_deterministic():
    inp = draw(2, 4, 1500, 128, "f16", 12)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    for mask in [None, "causal", (100, 7)]:
        o1, l1 = ea.attn_fwd(q, k, v, mask=mask)
        o2, l2 = ea.attn_fwd(q, k, v, mask=mask)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("mask", [None, "causal", (7, 3), (0, 0)])
def test_closed_forms(mask):
    """Constant V gives that constant; Q = 0 gives lse = ln #A_i and the mean of allowed V."""
    N, d = 500, 64
    inp = draw(1, 2, N, d, "bf16", 13)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    c = torch.linspace(-2, 3, d, dtype=torch.bfloat16, device="cuda")
    vc = c.expand(1, 2, N, d).contiguous()
    o, _ = ea.attn_fwd(q, k, vc, mask=mask)
    assert torch.max(torch.abs(o.float() - vc.float())).item() <= 2e-2
    mode, wl, wr = ea.mask_args(mask)
    name = ["none", "causal", "sliding"][mode]
    count = oracle.allowed_count(N, name, wl, wr)
    o0, l0 = ea.attn_fwd(torch.zeros_like(q), k, v, mask=mask)
    torch.cuda.synchronize()
    np.testing.assert_allclose(l0[0, 0].cpu().double().numpy(), np.log(count), rtol=0, atol=1e-5)
    V64 = to_f64(inp["v"][0, 0])
    A = oracle.allowed_matrix(np.arange(N), np.arange(N), N, name, wl, wr)
    mean_v = (A @ V64) / count[:, None]
    err = np.abs(to_f64(o0[0, 0].cpu()) - mean_v)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_key_permutation_invariance():
    N = 1000
    inp = draw(1, 2, N, 128, "f16", 14)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(0)).cuda()
    o1, l1 = ea.attn_fwd(q, k, v)
    o2, l2 = ea.attn_fwd(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous())
    assert torch.max(torch.abs(o1.float() - o2.float())).item() <= 2e-2
    assert torch.max(torch.abs(l1 - l2)).item() <= 1e-4


def test_single_allowed_key_copies_v():
    N = 300
    inp = draw(1, 1, N, 128, "bf16", 15)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    o, lse = ea.attn_fwd(q, k, v, mask=(0, 0), scale=0.1)
    assert torch.equal(o, v)
    ref = 0.1 * (to_f64(inp["q"][0, 0]) * to_f64(inp["k"][0, 0])).sum(axis=1)
    np.testing.assert_allclose(lse[0, 0].cpu().double().numpy(), ref, rtol=0, atol=1e-4)


def test_output_buffers_and_errors():
    inp = draw(1, 1, 64, 64, "f16", 16)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    with pytest.raises(ea.AttnError):
        ea.attn_fwd(q, k, v, out=q)          # output aliases an input
    with pytest.raises(ea.AttnError):
        ea.attn_fwd(q, k, v, mask=(-1, 0))   # negative window
    with pytest.raises(ea.AttnError):
        ea.attn_fwd(q, k, v, scale=math.inf)


def test_binding_checks_lse_and_workspace():
    inp = draw(1, 2, 100, 64, "f16", 17, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    with pytest.raises(ValueError, match="lse"):
        ea.attn_fwd(q, k, v, lse=torch.empty(1, 2, 100))          # host lse
    o, lse = ea.attn_fwd(q, k, v)
    with pytest.raises(ValueError, match="lse"):
        ea.attn_bwd(q, k, v, o, lse.cpu(), do)
    with pytest.raises(ValueError, match="workspace"):
        ea.attn_bwd(q, k, v, o, lse, do, workspace=torch.empty(4096, dtype=torch.uint8))
    # A workspace of any element type counts in bytes: float32 with exactly enough bytes works
    # and matches the default workspace bitwise.
    need = ea.attn_bwd_workspace_bytes(q.dtype, 1, 2, 100, 64)
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device=q.device)
    g1 = ea.attn_bwd(q, k, v, o, lse, do, workspace=ws)
    g2 = ea.attn_bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


def test_large_values_after_a_max_jump_stay_finite():
    """bf16 V of magnitude 2^70 and one key whose score lies 63.5 (exp2 units)
    above every earlier key of its row: a probability formed against the old
    max would be 2^63.5, and 2^63.5 * 2^70 overflows fp32.  The exact result
    (a convex combination of V rows) is representable; the kernel must take the
    exact-max path before such a product reaches the accumulator."""
    N, d = 1024, 64
    inp = draw(1, 2, N, d, "bf16", 78)
    q, k, v = inp["q"].clone(), inp["k"].clone(), inp["v"].clone()
    q.zero_()
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    k[..., 100, 0] = 44.0  # 44 * log2(e) = 63.5 in exp2 units, scale 1
    v = v * 2.0 ** 70       # a power of two: exact in bf16
    for mask in (None, "causal"):
        o, lse = run_fwd({"q": q, "k": k, "v": v}, mask, 1.0)
        assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), mask
        name, wl, wr = oracle_mask(mask)
        O_ref = np.empty((2, N, d))
        L_ref = np.empty((2, N))
        for h in range(2):
            O_ref[h], L_ref[h] = oracle.forward_head(to_f64(q[0, h]), to_f64(k[0, h]),
                                                     to_f64(v[0, h]), 1.0, name, wl, wr)
        # compare in units of 2^70 (exact rescaling of both sides)
        check_fwd(to_f64(o[0].cpu()) / 2.0 ** 70, lse[0].cpu().double().numpy(), O_ref / 2.0 ** 70,
                  L_ref, label=f"|V| ~ 2^70 after a jump, {mask}")
