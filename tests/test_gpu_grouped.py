"""GPU parity of the grouped-query and packed variable-length entry points
against the fp64 oracle (oracle/grouped.py), element by element, with the
tolerances of parity_util (reading 19's per-case bars for the backward).

Inputs come from workloads.draw_grouped / draw_packed (seeded N(0, 1),
rounded once to fp16/bf16); packed batches mix empty, one-row, tile-edge and
longer sequences.
"""
import numpy as np
import pytest
import torch

import oracle
import exact_attention_14_amd as ea
from bwd_rounding import heads_bar
from parity_util import GRAD_REL_FRO, check_fwd, gpu, oracle_mask, rel_fro, say
from workloads import draw_grouped, draw_packed, length_mix, packed_offsets, to_f64

pytestmark = pytest.mark.gpu

GQA_FWD = [
    (2, 8, 2, 300, 128, "bf16", None),
    (1, 8, 1, 257, 64, "f16", "causal"),
    (2, 6, 3, 130, 128, "f16", (20, 5)),
    (1, 4, 2, 1, 128, "bf16", "causal"),
    (3, 4, 1, 64, 64, "bf16", None),
    (1, 16, 4, 700, 128, "f16", "causal"),
]


@pytest.mark.parametrize("cfg", GQA_FWD, ids=[str(c) for c in GQA_FWD])
def test_gqa_forward(cfg):
    B, H, H_kv, N, d, dtype, mask = cfg
    say(f"gqa fwd {cfg}")
    scale = 1.0 / np.sqrt(d)
    inp = draw_grouped(B, H, H_kv, N, d, dtype, seed=100 + N)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    o, lse = ea.attn_fwd(q, k, v, mask=mask, scale=scale)
    torch.cuda.synchronize()
    name, wl, wr = oracle_mask(mask)
    Q, K, V = (to_f64(inp[x]) for x in ("q", "k", "v"))
    O_ref, L_ref = oracle.forward_gqa(Q, K, V, scale, name, wl, wr)
    check_fwd(to_f64(o.cpu()), lse.cpu().double().numpy(), O_ref, L_ref, label=str(cfg))


GQA_BWD = [
    (2, 8, 2, 200, 128, "f16", "causal"),
    (1, 8, 1, 300, 64, "bf16", None),
    (2, 6, 3, 150, 128, "bf16", (30, 0)),
    (1, 4, 4, 96, 64, "f16", (5, 9)),
    (1, 12, 2, 520, 128, "f16", "causal"),
    (2, 8, 4, 333, 128, "bf16", None),
    (1, 4, 2, 190, 64, "f16", (40, 3)),
]


@pytest.mark.parametrize("cfg", GQA_BWD, ids=[str(c) for c in GQA_BWD])
def test_gqa_backward(cfg):
    B, H, H_kv, N, d, dtype, mask = cfg
    say(f"gqa bwd {cfg}")
    scale = 1.0 / np.sqrt(d)
    inp = draw_grouped(B, H, H_kv, N, d, dtype, seed=200 + N, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, mask=mask, scale=scale)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, mask=mask, scale=scale)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    name, wl, wr = oracle_mask(mask)
    Q, K, V, dO = (to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    ref = oracle.backward_gqa(Q, K, V, dO, scale, name, wl, wr)
    errs = [rel_fro(to_f64(g.cpu()), r) for g, r in zip((dq, dk, dv), ref)]
    say(f"  rel fro dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e}")
    assert max(errs) <= GRAD_REL_FRO


def test_gqa_backward_is_deterministic():
    inp = draw_grouped(1, 8, 2, 333, 128, "bf16", seed=7, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, mask="causal")
    a = ea.attn_bwd(q, k, v, o, lse, do, mask="causal")
    b = ea.attn_bwd(q, k, v, o, lse, do, mask="causal")
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


PACKED = [
    # (lengths, H, H_kv, d, dtype, mask)
    ([5, 0, 1, 63, 64, 65, 129, 300], 4, 2, 128, "bf16", "causal"),
    ([300, 17, 0, 256], 4, 4, 64, "f16", None),
    ([1, 1, 2, 40, 700], 6, 2, 128, "f16", (33, 4)),
    ([128, 128, 128], 8, 1, 64, "bf16", None),
    ([257], 2, 1, 128, "bf16", "causal"),
    ([0, 0, 90, 0], 2, 2, 64, "f16", "causal"),
]


def packed_case(lengths, H, H_kv, d, dtype, seed, with_do=False, pad=0):
    cu = packed_offsets(lengths)
    T = int(cu[-1]) + pad
    inp = draw_packed(H, H_kv, T, d, dtype, seed, with_do=with_do)
    return cu, T, inp


def covered_rows(cu, T):
    m = np.zeros(T, dtype=bool)
    m[int(cu[0]):int(cu[-1])] = True
    return m


@pytest.mark.parametrize("cfg", PACKED, ids=[str(c) for c in PACKED])
def test_varlen_forward(cfg):
    lengths, H, H_kv, d, dtype, mask = cfg
    say(f"varlen fwd {cfg}")
    scale = 1.0 / np.sqrt(d)
    # 7 rows past the last sequence belong to none: they must stay untouched
    cu, T, inp = packed_case(lengths, H, H_kv, d, dtype, seed=300 + sum(lengths), pad=7)
    q, k, v = (gpu(inp[x]) for x in ("q", "k", "v"))
    cu_t = torch.from_numpy(cu).to("cuda")
    out = torch.full_like(q, 3.0)
    lse = torch.full((H, T), 5.0, dtype=torch.float32, device="cuda")
    ea.attn_fwd_varlen(q, k, v, cu_t, max(max(lengths), 1), mask=mask, scale=scale, out=out,
                       lse=lse)
    torch.cuda.synchronize()
    name, wl, wr = oracle_mask(mask)
    Q, K, V = (to_f64(inp[x]) for x in ("q", "k", "v"))
    O_ref, L_ref = oracle.forward_varlen(Q, K, V, cu, scale, name, wl, wr)
    rows = covered_rows(cu, T)
    og, lg = to_f64(out.cpu()), lse.cpu().double().numpy()
    if rows.any():
        check_fwd(og[:, rows], lg[:, rows], O_ref[:, rows], L_ref[:, rows], label=str(cfg))
    assert np.all(og[:, ~rows] == 3.0) and np.all(lg[:, ~rows] == 5.0)


def seq_tolerance(Q, K, V, dO, scale, dtype, mask, group):
    """The gradient bar of one sequence's rows ([heads, n, d] slices): 1e-2, or
    1.5x the error the backward's 16-bit roundings give in fp64 where larger."""
    name, wl, wr = oracle_mask(mask)
    return heads_bar(Q, K, V, dO, scale, name, wl, wr, dtype, group)


@pytest.mark.parametrize("cfg", PACKED, ids=[str(c) for c in PACKED])
def test_varlen_backward(cfg):
    lengths, H, H_kv, d, dtype, mask = cfg
    say(f"varlen bwd {cfg}")
    scale = 1.0 / np.sqrt(d)
    cu, T, inp = packed_case(lengths, H, H_kv, d, dtype, seed=400 + sum(lengths), with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    cu_t = torch.from_numpy(cu).to("cuda")
    mx = max(max(lengths), 1)
    o, lse = ea.attn_fwd_varlen(q, k, v, cu_t, mx, mask=mask, scale=scale)
    dq, dk, dv = ea.attn_bwd_varlen(q, k, v, o, lse, do, cu_t, mx, mask=mask, scale=scale)
    torch.cuda.synchronize()
    name, wl, wr = oracle_mask(mask)
    Q, K, V, dO = (to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    ref = oracle.backward_varlen(Q, K, V, dO, cu, scale, name, wl, wr)
    got = [to_f64(t.cpu()) for t in (dq, dk, dv)]
    worst = 0.0
    for lo, hi in zip(cu[:-1], cu[1:]):
        lo, hi = int(lo), int(hi)
        if hi == lo:
            continue
        for i in range(3):
            g, r = got[i][:, lo:hi], ref[i][:, lo:hi]
            assert np.all(np.isfinite(g))
            if hi - lo == 1 and i < 2:
                # one allowed key per row: the exact dQ and dK are zero
                assert np.linalg.norm(g) <= 1e-4 * np.linalg.norm(dO[:, lo:hi]) + 1e-30
                continue
            e = rel_fro(g, r)
            worst = max(worst, e)
            bar = seq_tolerance(Q[:, lo:hi], K[:, lo:hi], V[:, lo:hi], dO[:, lo:hi], scale, dtype,
                                mask, H // H_kv)
            assert e <= bar, (lo, hi, "dQ dK dV".split()[i], e, bar)
    say(f"  worst rel fro {worst:.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_varlen_single_sequence_equals_fixed_length_gqa(dtype):
    """One sequence filling T rows gives bit-identical results to the fixed-length call."""
    H, H_kv, T, d = 8, 2, 1000, 128
    inp = draw_packed(H, H_kv, T, d, dtype, seed=9, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    o1, l1 = ea.attn_fwd_varlen(q, k, v, cu, T, mask="causal")
    o2, l2 = ea.attn_fwd(q[None], k[None], v[None], mask="causal")
    g1 = ea.attn_bwd_varlen(q, k, v, o1, l1, do, cu, T, mask="causal")
    g2 = ea.attn_bwd(q[None], k[None], v[None], o2, l2, do[None], mask="causal")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[0]) and torch.equal(l1, l2[0])
    for a, b in zip(g1, g2):
        assert torch.equal(a, b[0])


def test_llama3_shape_gqa_causal_full_size_sampled_heads():
    """B2 H32 H_kv8 N4096 d128 bf16 causal forward + backward; two query heads of one group
    and their key/value head checked against the oracle."""
    B, H, H_kv, N, d = 2, 32, 8, 4096, 128
    say("gqa full size B2 H32 Hkv8 N4096")
    scale = 1.0 / np.sqrt(d)
    inp = draw_grouped(B, H, H_kv, N, d, "bf16", seed=31, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, mask="causal", scale=scale)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, mask="causal", scale=scale)
    torch.cuda.synchronize()
    b, kvh = 1, 5
    Q, K, V, dO = (to_f64(inp[x][b:b + 1]) for x in ("q", "k", "v", "do"))
    # forward of two query heads of the group, rows in blocks
    heads = [(0, kvh * 4), (0, kvh * 4 + 3)]
    O_ref, L_ref = oracle.forward_gqa(Q, K, V, scale, "causal", heads=heads, row_block=1024)
    for _, h in heads:
        check_fwd(to_f64(o[b, h].cpu()), lse[b, h].cpu().double().numpy(), O_ref[0, h],
                  L_ref[0, h], label=f"head {h}")
    # dK, dV of the key/value head: the sum over its four query heads
    dk_ref = np.zeros((N, d))
    dv_ref = np.zeros((N, d))
    for g in range(4):
        h = kvh * 4 + g
        dqh, dkh, dvh = oracle.backward_head(Q[0, h], K[0, kvh], V[0, kvh], dO[0, h], scale,
                                             "causal")
        dk_ref += dkh
        dv_ref += dvh
        e = rel_fro(to_f64(dq[b, h].cpu()), dqh)
        assert e <= GRAD_REL_FRO, ("dQ", h, e)
    ek = rel_fro(to_f64(dk[b, kvh].cpu()), dk_ref)
    ev = rel_fro(to_f64(dv[b, kvh].cpu()), dv_ref)
    say(f"  dK {ek:.3e} dV {ev:.3e}")
    assert ek <= GRAD_REL_FRO and ev <= GRAD_REL_FRO


def test_packed_mixed_lengths_full_size_sampled_sequences():
    """H32 H_kv8 d128 bf16 causal over 32768 packed rows of log-uniform lengths in
    [128, 8192]: forward on three sequences of two heads, backward on the shortest."""
    H, H_kv, d = 32, 8, 128
    lengths = length_mix(32768, 128, 8192, seed=6)
    cu = packed_offsets(lengths)
    T = int(cu[-1])
    say(f"packed full size: {len(lengths)} sequences, T = {T}, max {max(lengths)}")
    scale = 1.0 / np.sqrt(d)
    inp = draw_packed(H, H_kv, T, d, "bf16", seed=61, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    cu_t = torch.from_numpy(cu).to("cuda")
    o, lse = ea.attn_fwd_varlen(q, k, v, cu_t, max(lengths), mask="causal", scale=scale)
    dq, dk, dv = ea.attn_bwd_varlen(q, k, v, o, lse, do, cu_t, max(lengths), mask="causal",
                                    scale=scale)
    torch.cuda.synchronize()
    order = np.argsort(lengths)
    for s in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        lo, hi = int(cu[s]), int(cu[s + 1])
        for h in (0, 13):
            kv = h // 4
            qh, kh, vh = (to_f64(inp[x][i, lo:hi]) for x, i in (("q", h), ("k", kv), ("v", kv)))
            rb = 1024
            for r0 in range(0, hi - lo, rb):
                rows = np.arange(r0, min(hi - lo, r0 + rb))
                O_ref, L_ref = oracle.forward_rows(rows, qh, kh, vh, scale, "causal")
                check_fwd(to_f64(o[h, lo + rows].cpu()), lse[h, lo + rows].cpu().double().numpy(),
                          O_ref, L_ref, label=f"seq {s} ({hi - lo} rows) head {h}")
    s = int(order[0])
    lo, hi = int(cu[s]), int(cu[s + 1])
    kv = 2
    dk_ref = np.zeros((hi - lo, d))
    for g in range(4):
        h = kv * 4 + g
        args = [to_f64(inp[x][i, lo:hi]) for x, i in (("q", h), ("k", kv), ("v", kv), ("do", h))]
        dqh, dkh, _ = oracle.backward_head(*args, scale, "causal")
        dk_ref += dkh
        assert rel_fro(to_f64(dq[h, lo:hi].cpu()), dqh) <= GRAD_REL_FRO
    e = rel_fro(to_f64(dk[kv, lo:hi].cpu()), dk_ref)
    say(f"  shortest sequence ({hi - lo} rows) dK rel fro {e:.3e}")
    assert e <= GRAD_REL_FRO
