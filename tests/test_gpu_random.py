"""Seeded random sweep of batch, heads, length, head size, dtype, mask, window and
scale: GPU forward and backward against the fp64 oracle.

The hand-written cases elsewhere pin the edges one by one; this sweep draws
combinations nobody listed (odd lengths with odd windows, negative scales with
sliding masks, ...) from a fixed seed, so a failure reproduces by its id.
"""
import os

import numpy as np
import pytest

from parity_util import bwd_case, fwd_case, say

pytestmark = pytest.mark.gpu


def draw_configs(n, seed, *, min_n=1, min_window=0):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        N = int(rng.integers(min_n, 70)) if rng.random() < 0.4 else int(rng.integers(70, 700))
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["f16", "bf16"]))
        kind = int(rng.integers(0, 3))
        if kind == 0:
            mask = None
        elif kind == 1:
            mask = "causal"
        else:
            hi = 21 if rng.random() < 0.5 else N + 8  # narrow windows half of the time
            mask = (int(rng.integers(min_window, hi)), int(rng.integers(min_window, hi)))
        scale = float(1.0 / np.sqrt(d)) if rng.random() < 0.5 else float(rng.uniform(-0.5, 0.5))
        out.append((B, H, N, d, dtype, mask, round(scale, 6), 1000 * seed + i))
    return out


def cfg_id(c):
    B, H, N, d, dtype, mask, scale, seed = c
    return f"B{B}H{H}N{N}d{d}-{dtype}-{mask}-s{scale}".replace(" ", "")


# ATTN_SWEEP_SCALE multiplies the number of cases (default 1: 48 forward, 24 backward).
SCALE = max(1, int(os.environ.get("ATTN_SWEEP_SCALE", "1")))
FWD = draw_configs(48 * SCALE, 7)
BWD = draw_configs(24 * SCALE, 8, min_n=16, min_window=1)


@pytest.mark.parametrize("cfg", FWD, ids=[cfg_id(c) for c in FWD])
def test_random_forward(cfg):
    B, H, N, d, dtype, mask, scale, seed = cfg
    say(f"random fwd {cfg_id(cfg)}")
    fwd_case(B, H, N, d, dtype, mask, seed=seed, scale=scale)


@pytest.mark.parametrize("cfg", BWD, ids=[cfg_id(c) for c in BWD])
def test_random_backward(cfg):
    B, H, N, d, dtype, mask, scale, seed = cfg
    # Few allowed keys per row: dP - D nearly cancels and the rounding of the
    # stored O (from which D is formed) dominates dS in bf16; each head's bar
    # comes from the rounding model (1e-2 unless the roundings exceed it).
    say(f"random bwd {cfg_id(cfg)}")
    bwd_case(B, H, N, d, dtype, mask, seed=seed, scale=scale)


# --- grouped-query, packed and paged-decode paths -------------------------

def draw_grouped_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H_kv = int(rng.choice([1, 2, 3, 4]))
        H = H_kv * int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 3))
        N = int(rng.integers(16, 600))
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["f16", "bf16"]))
        kind = int(rng.integers(0, 3))
        mask = None if kind == 0 else ("causal" if kind == 1 else
                                       (int(rng.integers(1, N + 8)), int(rng.integers(0, 40))))
        out.append((B, H, H_kv, N, d, dtype, mask, 5000 + 100 * seed + i))
    return out


def draw_packed_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H_kv = int(rng.choice([1, 2, 4]))
        H = H_kv * int(rng.choice([1, 2, 4]))
        lens = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 400, rng.integers(1, 6))]
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["f16", "bf16"]))
        kind = int(rng.integers(0, 3))
        mask = None if kind == 0 else ("causal" if kind == 1 else
                                       (int(rng.integers(1, 200)), int(rng.integers(0, 30))))
        out.append((lens, H, H_kv, d, dtype, mask, 7000 + 100 * seed + i))
    return out


def draw_decode_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H_kv = int(rng.choice([1, 2, 4, 8]))
        H = H_kv * int(rng.choice([1, 2, 4, 8]))
        n_q = int(rng.choice([1, 1, 2, 5]))
        lens = [int(x) for x in rng.integers(n_q, 3000, rng.integers(1, 5))]
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["f16", "bf16"]))
        page = int(rng.choice([64, 128, 256, 320]))
        kind = int(rng.integers(0, 3))
        mask = None if kind == 0 else ("causal" if kind == 1 else
                                       (int(rng.integers(0, 500)), int(rng.integers(0, 4))))
        out.append((lens, H, H_kv, n_q, d, dtype, page, mask, 9000 + 100 * seed + i))
    return out


GQA = draw_grouped_configs(16 * SCALE, 11)
PACKED = draw_packed_configs(12 * SCALE, 12)
DECODE = draw_decode_configs(16 * SCALE, 13)


@pytest.mark.parametrize("cfg", GQA, ids=[str(c[:7]).replace(" ", "") for c in GQA])
def test_random_grouped_forward_backward(cfg):
    import torch
    import oracle
    import exact_attention_14_amd as ea
    from parity_util import check_fwd, gpu, oracle_mask, rel_fro
    from workloads import draw_grouped, to_f64
    B, H, H_kv, N, d, dtype, mask, seed = cfg
    say(f"random grouped {cfg}")
    scale = float(1.0 / np.sqrt(d))
    inp = draw_grouped(B, H, H_kv, N, d, dtype, seed, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, mask=mask, scale=scale)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, mask=mask, scale=scale)
    torch.cuda.synchronize()
    name, wl, wr = oracle_mask(mask)
    Q, K, V, dO = (to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    O_ref, L_ref = oracle.forward_gqa(Q, K, V, scale, name, wl, wr)
    check_fwd(to_f64(o.cpu()), lse.cpu().double().numpy(), O_ref, L_ref, label="grouped")
    ref = oracle.backward_gqa(Q, K, V, dO, scale, name, wl, wr)
    from bwd_rounding import heads_bar
    tol = max(heads_bar(Q[b], K[b], V[b], dO[b], scale, name, wl, wr, dtype, H // H_kv)
              for b in range(B))
    for g, r in zip((dq, dk, dv), ref):
        assert rel_fro(to_f64(g.cpu()), r) <= tol


@pytest.mark.parametrize("cfg", PACKED, ids=[str(c[:6]).replace(" ", "") for c in PACKED])
def test_random_packed_forward_backward(cfg):
    import torch
    import oracle
    import exact_attention_14_amd as ea
    from parity_util import check_fwd, gpu, oracle_mask, rel_fro
    from workloads import draw_packed, packed_offsets, to_f64
    lens, H, H_kv, d, dtype, mask, seed = cfg
    say(f"random packed {cfg}")
    if sum(lens) == 0:
        lens = lens + [5]
    cu = packed_offsets(lens)
    T = int(cu[-1])
    scale = float(1.0 / np.sqrt(d))
    inp = draw_packed(H, H_kv, T, d, dtype, seed, with_do=True)
    q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
    cu_t = torch.from_numpy(cu).to("cuda")
    o, lse = ea.attn_fwd_varlen(q, k, v, cu_t, max(lens), mask=mask, scale=scale)
    dq, dk, dv = ea.attn_bwd_varlen(q, k, v, o, lse, do, cu_t, max(lens), mask=mask, scale=scale)
    torch.cuda.synchronize()
    name, wl, wr = oracle_mask(mask)
    Q, K, V, dO = (to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    O_ref, L_ref = oracle.forward_varlen(Q, K, V, cu, scale, name, wl, wr)
    check_fwd(to_f64(o.cpu()), lse.cpu().double().numpy(), O_ref, L_ref, label="packed")
    ref = oracle.backward_varlen(Q, K, V, dO, cu, scale, name, wl, wr)
    got = [to_f64(t.cpu()) for t in (dq, dk, dv)]
    from bwd_rounding import heads_bar
    for lo, hi in zip(cu[:-1], cu[1:]):
        lo, hi = int(lo), int(hi)
        if hi - lo < 2:
            continue  # one row: exact dQ, dK are zero (covered in test_gpu_grouped)
        tol = heads_bar(Q[:, lo:hi], K[:, lo:hi], V[:, lo:hi], dO[:, lo:hi], scale, name, wl, wr,
                        dtype, H // H_kv)
        for i in range(3):
            assert rel_fro(got[i][:, lo:hi], ref[i][:, lo:hi]) <= tol, (lo, hi, i)


@pytest.mark.parametrize("cfg", DECODE, ids=[str(c[:8]).replace(" ", "") for c in DECODE])
def test_random_decode(cfg):
    import torch
    import oracle
    import exact_attention_14_amd as ea
    from parity_util import check_fwd, gpu, oracle_mask
    from workloads import draw_paged, to_f64
    lens, H, H_kv, n_q, d, dtype, page, mask, seed = cfg
    say(f"random decode {cfg}")
    scale = float(1.0 / np.sqrt(d))
    inp = draw_paged(lens, H, H_kv, n_q, d, dtype, page, seed)
    q, k, v, bt, sl = (gpu(inp[x]) for x in ("q", "k", "v", "block_table", "seq_lens"))
    o, lse = ea.attn_decode(q, k, v, bt, sl, max(lens), mask=mask, scale=scale)
    torch.cuda.synchronize()
    name, wl, wr = oracle_mask(mask)
    O_ref, L_ref = oracle.forward_decode(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]),
                                         inp["block_table"].numpy(), inp["seq_lens"].numpy(),
                                         scale, name, wl, wr)
    check_fwd(to_f64(o.cpu()), lse.cpu().double().numpy(), O_ref, L_ref, label="decode")
