"""GPU parity of split-KV decoding over a paged cache (attn_decode) against the
fp64 oracle (oracle/decode.py), element by element, with the forward's
tolerances.  Pools are shuffled and every row no sequence owns is NaN, so a
stale read shows; cases cover one and many splits, grouped and multi-query
heads, several query tokens and two query-row tiles, all masks, page sizes
64-256 and ragged last pages."""
import numpy as np
import pytest
import torch

import oracle
import exact_attention_14_amd as ea
from parity_util import check_fwd, gpu, oracle_mask, say
from workloads import draw_paged, to_f64

pytestmark = pytest.mark.gpu

CASES = [
    # (lens, H, H_kv, n_q, d, dtype, page_size, mask)
    ([1000, 64, 5000], 8, 2, 1, 128, "bf16", 64, None),
    ([300, 8192], 32, 1, 1, 128, "f16", 128, "causal"),
    ([17, 256, 1023, 64], 8, 8, 4, 64, "bf16", 256, "causal"),
    ([4096, 777], 16, 2, 3, 128, "f16", 64, (100, 0)),
    ([500, 130], 32, 1, 2, 128, "bf16", 64, "causal"),
    ([65, 129, 200], 4, 4, 1, 64, "f16", 192, (30, 7)),
    ([1, 2, 63], 8, 4, 1, 128, "bf16", 64, "causal"),
]


def run_case(lens, H, H_kv, n_q, d, dtype, page_size, mask, seed):
    scale = 1.0 / np.sqrt(d)
    inp = draw_paged(lens, H, H_kv, n_q, d, dtype, page_size, seed)
    q, k, v, bt, sl = (gpu(inp[x]) for x in ("q", "k", "v", "block_table", "seq_lens"))
    o, lse = ea.attn_decode(q, k, v, bt, sl, max(lens), mask=mask, scale=scale)
    torch.cuda.synchronize()
    name, wl, wr = oracle_mask(mask)
    O_ref, L_ref = oracle.forward_decode(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]),
                                         inp["block_table"].numpy(), inp["seq_lens"].numpy(),
                                         scale, name, wl, wr)
    return check_fwd(to_f64(o.cpu()), lse.cpu().double().numpy(), O_ref, L_ref,
                     label=f"{lens} H{H}/{H_kv} nq{n_q} d{d} {dtype} page{page_size} {mask}")


@pytest.mark.parametrize("cfg", CASES, ids=[str(c) for c in CASES])
def test_decode(cfg):
    lens, H, H_kv, n_q, d, dtype, page_size, mask = cfg
    n_splits_ws = ea.attn_decode_workspace_bytes(torch.bfloat16, len(lens), H, H_kv, n_q, d,
                                                 max(lens))
    say(f"decode {cfg} workspace {n_splits_ws}")
    run_case(lens, H, H_kv, n_q, d, dtype, page_size, mask, seed=sum(lens) + n_q)


def test_decode_many_sequences_one_split():
    """600 sequences x 8 key/value heads fill the chip: no split, no workspace."""
    rng = np.random.default_rng(3)
    lens = [int(x) for x in rng.integers(1, 400, size=600)]
    assert ea.attn_decode_workspace_bytes(torch.bfloat16, 600, 8, 8, 1, 128, max(lens)) == 0
    say("decode 600 sequences")
    run_case(lens, 8, 8, 1, 128, "bf16", 64, None, seed=5)


def test_decode_matches_the_forward_on_the_last_rows():
    """Decode of the last 3 tokens equals rows N-3.. of the causal forward on the same data."""
    N, H, d = 700, 4, 128
    inp = draw_paged([N], H, H, 3, d, "bf16", 64, seed=8, spare_pages=0)
    bt = inp["block_table"][0].long()
    k_dense = torch.cat([inp["k"][bt[i]] for i in range(len(bt))], dim=1)[:, :N]  # [H, N, d]
    v_dense = torch.cat([inp["v"][bt[i]] for i in range(len(bt))], dim=1)[:, :N]
    q_dense = torch.randn(1, H, N, d, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    q_dense[0, :, N - 3:] = inp["q"][0]
    o_f, l_f = ea.attn_fwd(gpu(q_dense), gpu(k_dense[None].contiguous()),
                           gpu(v_dense[None].contiguous()), mask="causal")
    o_d, l_d = ea.attn_decode(*(gpu(inp[x]) for x in ("q", "k", "v", "block_table", "seq_lens")),
                              N, mask="causal")
    torch.cuda.synchronize()
    diff = (o_f[0, :, N - 3:].float() - o_d[0].float()).abs().max().item()
    say(f"  decode vs forward rows: max abs {diff:.3e}")
    assert diff <= 2e-2
    assert (l_f[0, :, N - 3:] - l_d[0]).abs().max().item() <= 1e-3


def test_decode_binding_rejects_misplaced_buffers():
    """The binding checks a caller's workspace and output buffers like the other
    entry points do: on the query's device and contiguous, else ValueError
    before the library is called."""
    lens = [300, 8192]
    inp = draw_paged(lens, 32, 1, 1, 128, "f16", 128, seed=3)
    args = [gpu(inp[x]) for x in ("q", "k", "v", "block_table", "seq_lens")]
    need = ea.attn_decode_workspace_bytes(torch.float16, 2, 32, 1, 1, 128, max(lens))
    assert need > 0
    with pytest.raises(ValueError):
        ea.attn_decode(*args, max(lens), workspace=torch.empty(need, dtype=torch.uint8))
    strided = torch.empty(2 * need, dtype=torch.uint8, device="cuda")[::2]
    with pytest.raises(ValueError):
        ea.attn_decode(*args, max(lens), workspace=strided)
    with pytest.raises(ValueError):
        ea.attn_decode(*args, max(lens), out=torch.empty_like(inp["q"]))
    ok = torch.empty(need, dtype=torch.uint8, device="cuda")
    o, lse = ea.attn_decode(*args, max(lens), workspace=ok)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())


@pytest.mark.parametrize("wname", ["decode_s64h32kv8q1ctx8192d128_bf16_page64",
                                   "decode_s4h32kv8q1ctx131072d128_bf16_page256"])
def test_decode_workload_full_size(wname):
    """The benchmark's decoding workloads at full size, every sequence and head
    against the oracle (each sequence's own pages gathered from the pool)."""
    from parity_util import map_heads
    from workloads import BY_NAME, make_inputs
    w = BY_NAME[wname]
    say(f"workload {w.name}: drawing inputs")
    inp = make_inputs(w)
    q, k, v, bt, sl = (gpu(inp[x]) for x in ("q", "k", "v", "block_table", "seq_lens"))
    o, lse = ea.attn_decode(q, k, v, bt, sl, w.N, scale=w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    table, lens = inp["block_table"].numpy(), inp["seq_lens"].numpy()
    say(f"workload {w.name}: oracle over {w.B} sequences")

    def one(s):
        n_pages = -(-int(lens[s]) // w.page_size)
        own = torch.from_numpy(table[s, :n_pages].astype(np.int64))
        return oracle.forward_decode(to_f64(inp["q"][s:s + 1]), to_f64(inp["k"][own]),
                                     to_f64(inp["v"][own]),
                                     np.arange(n_pages, dtype=np.int32)[None],
                                     lens[s:s + 1], w.scale)

    res = map_heads(one, list(range(w.B)))
    check_fwd(to_f64(o.cpu()), lse.cpu().double().numpy(), np.concatenate([r[0] for r in res]),
              np.concatenate([r[1] for r in res]), label=w.name)
