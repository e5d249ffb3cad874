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


def test_many_short_heads_forward_and_backward():
    """131,072 heads of 65 rows (two key tiles, the second one row long), causal,
    d = 128 fp16: 2.18 GB per tensor, so the last heads start past byte 2^31.
    Every output is finite; heads at the start, the middle and the end are
    compared with the oracle."""
    B, H, N, d, dtype = 64, 2048, 65, 128, "f16"
    scale = 1.0 / math.sqrt(d)
    say(f"many heads: B{B} H{H} N{N} d{d} {dtype}, causal")
    inp = draw_on_device(B, H, N, d, dtype, seed=12, with_do=True)
    q, k, v, do = (inp[x] for x in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, mask="causal", scale=scale)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, mask="causal", scale=scale)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("lse", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), name
    for b, h in ((0, 0), (0, 1), (31, 1023), (32, 0), (63, 2046), (63, 2047)):
        qh, kh, vh, doh = (to_f64(t[b, h].cpu()) for t in (q, k, v, do))
        o_ref, l_ref = oracle.forward_rows(np.arange(N), qh, kh, vh, scale, "causal")
        check_fwd(to_f64(o[b, h].cpu())[None], lse[b, h].cpu().double().numpy()[None],
                  o_ref[None], l_ref[None], label=f"head ({b}, {h})")
        ref = oracle.backward_head(qh, kh, vh, doh, scale, "causal")
        bar = grad_bar(qh, kh, vh, doh, scale, "causal", 0, 0, dtype)
        errs = [rel_fro(to_f64(g[b, h].cpu()), r) for g, r in zip((dq, dk, dv), ref)]
        assert max(errs) <= bar, ((b, h), errs, bar)


def test_decode_over_a_pool_beyond_4_gib():
    """Paged decoding whose pages lie past byte 2^32 of each pool (5.2 GB pools of
    40,000 64-key pages x 8 key/value heads): every page of the three sequences is
    taken from the last 4,000 pages, shuffled, and the rest of the pool is NaN."""
    n_pages, H, H_kv, page, d, dtype = 40000, 32, 8, 64, 128, "bf16"
    lens = [3000, 64, 1501]
    scale = 1.0 / math.sqrt(d)
    say(f"decode, pools of {n_pages} pages ({n_pages * H_kv * page * d * 2 / 1e9:.1f} GB each)")
    pool_k = torch.full((n_pages, H_kv, page, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    pool_v = torch.full_like(pool_k, float("nan"))
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    q = torch.randn((len(lens), H, 1, d), generator=g, device="cuda").to(torch.bfloat16)
    per = [-(-L // page) for L in lens]
    rng = np.random.default_rng(13)
    phys = rng.permutation(np.arange(n_pages - 4000, n_pages))[:sum(per)]
    assert phys.min() * H_kv * page * d * 2 >= (1 << 32)
    table = np.zeros((len(lens), max(per)), dtype=np.int32)
    used = 0
    for s, n in enumerate(per):
        table[s, :n] = phys[used:used + n]
        used += n
    pages = torch.from_numpy(phys.astype(np.int64)).cuda()
    pool_k[pages] = torch.randn((len(phys), H_kv, page, d), generator=g, device="cuda").to(
        torch.bfloat16)
    pool_v[pages] = torch.randn((len(phys), H_kv, page, d), generator=g, device="cuda").to(
        torch.bfloat16)
    bt = torch.from_numpy(table).cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = ea.attn_decode(q, pool_k, pool_v, bt, sl, max(lens), scale=scale)
    torch.cuda.synchronize()
    # the oracle reads each sequence's own pages, renumbered 0..
    O_ref, L_ref = [], []
    for s, n in enumerate(per):
        own = torch.from_numpy(table[s, :n].astype(np.int64)).cuda()
        o_s, l_s = oracle.forward_decode(to_f64(q[s:s + 1].cpu()), to_f64(pool_k[own].cpu()),
                                         to_f64(pool_v[own].cpu()),
                                         np.arange(n, dtype=np.int32)[None],
                                         np.array([lens[s]], dtype=np.int32), scale)
        O_ref.append(o_s)
        L_ref.append(l_s)
    check_fwd(to_f64(o.cpu()), lse.cpu().double().numpy(), np.concatenate(O_ref),
              np.concatenate(L_ref), label="pool beyond 4 GiB")
