"""GPU parity at the full sizes of the grouped-query, multi-query and packed
workloads, in the launch configuration the benchmark times, on every head.

Forward: every query head's O and lse against the fp64 oracle (max and mean
abs over all elements, lse max abs).  Backward: every query head's dQ, and
every key/value head's dK and dV, the sums over the query heads that read it
(summed here from the oracle's per-query-head gradients).  Each query head is
one worker-thread job on the host.
"""
import numpy as np
import pytest
import torch

import exact_attention_14_amd as ea
import oracle
from bwd_rounding import grad_bar
from parity_util import (GRAD_REL_FRO, LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, gpu, map_heads,
                         rel_fro, say)
from workloads import (GQA_CAUSAL_FWDBWD, MQA_CAUSAL_FWDBWD, PACKED_CAUSAL_FWDBWD, make_inputs,
                       packed_offsets, to_f64)

pytestmark = pytest.mark.gpu


def check_all(units, label, n_elems):
    """units: per query-head results (O max abs, O abs sum, lse max abs, dQ rel error)."""
    omax = max(u[0] for u in units)
    omean = sum(u[1] for u in units) / n_elems
    lmax = max(u[2] for u in units)
    dqmax = max(u[3] for u in units)
    say(f"  {label}: O max abs {omax:.3e} mean abs {omean:.3e}; lse max abs {lmax:.3e}; "
        f"worst dQ rel fro {dqmax:.3e}")
    assert omax <= O_MAX_ABS and omean <= O_MEAN_ABS and lmax <= LSE_MAX_ABS
    return dqmax


@pytest.mark.parametrize("w", [GQA_CAUSAL_FWDBWD, MQA_CAUSAL_FWDBWD], ids=lambda w: w.name)
def test_grouped_workload_all_heads(w):
    say(f"workload {w.name}: drawing inputs")
    inp = make_inputs(w)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, mask="causal", scale=w.scale)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, mask="causal", scale=w.scale)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("lse", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), name
    g = [t.cpu() for t in (o, lse, dq, dk, dv)]
    B, H, N, d, G = w.B, w.H, w.N, w.d, w.H // w.kv_heads
    say(f"workload {w.name}: oracle over all {B * H} query heads")

    def one(bh):
        b, h = bh
        qh, kh, vh, doh = (to_f64(inp[x][b, i]) for x, i in
                           (("q", h), ("k", h // G), ("v", h // G), ("do", h)))
        o_ref, l_ref = oracle.forward_rows(np.arange(N), qh, kh, vh, w.scale, "causal")
        e = np.abs(to_f64(g[0][b, h]) - o_ref)
        el = float(np.abs(g[1][b, h].double().numpy() - l_ref).max())
        dqr, dkr, dvr = oracle.backward_head(qh, kh, vh, doh, w.scale, "causal")
        return float(e.max()), float(e.sum()), el, rel_fro(to_f64(g[2][b, h]), dqr), dkr, dvr

    heads = [(b, h) for b in range(B) for h in range(H)]
    res = map_heads(one, heads)
    dqmax = check_all(res, w.name, B * H * N * d)
    assert dqmax <= GRAD_REL_FRO
    worst = [0.0, 0.0]
    for b in range(B):
        for kvh in range(w.kv_heads):
            parts = [res[b * H + h] for h in range(kvh * G, (kvh + 1) * G)]
            dk_ref = sum(p[4] for p in parts)
            dv_ref = sum(p[5] for p in parts)
            worst[0] = max(worst[0], rel_fro(to_f64(g[3][b, kvh]), dk_ref))
            worst[1] = max(worst[1], rel_fro(to_f64(g[4][b, kvh]), dv_ref))
    say(f"  {w.name}: worst dK rel fro {worst[0]:.3e} dV {worst[1]:.3e} over {B * w.kv_heads} "
        f"key/value heads")
    assert max(worst) <= GRAD_REL_FRO


def test_packed_workload_all_heads_and_sequences():
    w = PACKED_CAUSAL_FWDBWD
    say(f"workload {w.name}: drawing inputs")
    inp = make_inputs(w)
    cu = packed_offsets(w.lengths)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    cu_t = torch.from_numpy(cu).to("cuda")
    mx = max(w.lengths)
    o, lse = ea.attn_fwd_varlen(q, k, v, cu_t, mx, mask="causal", scale=w.scale)
    dq, dk, dv = ea.attn_bwd_varlen(q, k, v, o, lse, do, cu_t, mx, mask="causal", scale=w.scale)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("lse", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), name
    g = [t.cpu() for t in (o, lse, dq, dk, dv)]
    H, d, G = w.H, w.d, w.H // w.kv_heads
    seqs = [(int(a), int(b_)) for a, b_ in zip(cu[:-1], cu[1:])]
    say(f"workload {w.name}: oracle over {len(seqs)} sequences x {H} heads")

    def one(item):
        (lo, hi), h = item
        qh, kh, vh, doh = (to_f64(inp[x][i, lo:hi]) for x, i in
                           (("q", h), ("k", h // G), ("v", h // G), ("do", h)))
        rb = 2048
        emax = esum = lmax = 0.0
        for r0 in range(0, hi - lo, rb):
            rows = np.arange(r0, min(hi - lo, r0 + rb))
            o_ref, l_ref = oracle.forward_rows(rows, qh, kh, vh, w.scale, "causal")
            e = np.abs(to_f64(g[0][h, lo + rows]) - o_ref)
            emax, esum = max(emax, float(e.max())), esum + float(e.sum())
            lmax = max(lmax, float(np.abs(g[1][h, lo + rows].double().numpy() - l_ref).max()))
        dqr, dkr, dvr = oracle.backward_head(qh, kh, vh, doh, w.scale, "causal")
        bar = grad_bar(qh, kh, vh, doh, w.scale, "causal", 0, 0, w.dtype)
        return emax, esum, lmax, rel_fro(to_f64(g[2][h, lo:hi]), dqr), dkr, dvr, bar

    items = [(s, h) for s in seqs for h in range(H)]
    res = map_heads(one, items)
    check_all(res, w.name, H * int(cu[-1]) * d)
    worst = [0.0, 0.0, 0.0]
    for si, (lo, hi) in enumerate(seqs):
        # the bar of the sequence: the worst of its query heads' (a shared key/value
        # head's gradient sums its query heads' contributions)
        bar = max(res[si * H + h][6] for h in range(H))
        for h in range(H):
            assert res[si * H + h][3] <= bar, ("dQ", (lo, hi), h, res[si * H + h][3], bar)
            worst[0] = max(worst[0], res[si * H + h][3])
        for kvh in range(w.kv_heads):
            parts = [res[si * H + h] for h in range(kvh * G, (kvh + 1) * G)]
            ek = rel_fro(to_f64(g[3][kvh, lo:hi]), sum(p[4] for p in parts))
            ev = rel_fro(to_f64(g[4][kvh, lo:hi]), sum(p[5] for p in parts))
            assert ek <= bar and ev <= bar, ((lo, hi), kvh, ek, ev, bar)
            worst[1], worst[2] = max(worst[1], ek), max(worst[2], ev)
    say(f"  {w.name}: worst rel fro dQ {worst[0]:.3e} dK {worst[1]:.3e} dV {worst[2]:.3e}")
