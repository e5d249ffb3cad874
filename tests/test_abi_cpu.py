"""The C-ABI library on the CPU: it loads, exports every symbol attn.h
declares, and its host logic (validation, tile ranges, workgroup order)
behaves as documented.  Only host-only entry points are called, plus the
launching entry points with invalid arguments, which must return their status
before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import exact_attention_14_amd as ea
from exact_attention_14_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(attn_[a-z_0-9]+)\s*\(",
                                 src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 20, names
    lib = ea.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.EXPORTS)


def test_status_strings():
    for s in range(11):
        assert ea.attn_status_str(s)
    assert "scratch" in ea.attn_status_str(10)


def test_launching_entry_points_reject_bad_arguments_before_any_hip_call():
    lib = ea.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    Q, K, V, O, L = base, base + 4096, base + 8192, base + 12288, base + 16384
    # NULL input
    assert lib.attn_fwd(1, None, K, V, O, L, 1, 1, 8, 64, 0.1, 0, 0, 0, None) == 1
    # unsupported d
    assert lib.attn_fwd(1, Q, K, V, O, L, 1, 1, 8, 80, 0.1, 0, 0, 0, None) == 3
    # negative window
    assert lib.attn_fwd(0, Q, K, V, O, L, 1, 1, 8, 64, 0.1, 2, -1, 0, None) == 4
    # output overlapping an input
    assert lib.attn_fwd(0, Q, K, V, Q + 16, L, 1, 1, 8, 64, 0.1, 0, 0, 0, None) == 7
    # workspace too small
    ws = ea.attn_bwd_workspace_bytes(__import__("torch").float16, 1, 1, 8, 64)
    assert ws == 512
    args = [0, Q, K, V, O, L, O, base + 20480, base + 24576, base + 28672, base + 32768, ws - 16,
            1, 1, 8, 64, 0.1, 1, 0, 0, None]
    assert lib.attn_bwd(*args) == 8
    # nothing was written: the buffer is still zero
    assert bytes(buf) == b"\0" * len(buf)


@pytest.mark.parametrize("d", [64, 128])
def test_longest_head_accepted_is_just_under_2_31_bytes(d):
    """One head of one tensor may hold at most 2^31 - 1 bytes (the kernels' byte
    offsets within a head are 32-bit): N = 2^31 / (2 d) - 1 rows pass the host
    checks, one more row is ATTN_E_SHAPE.  No memory is touched (host-only check)."""
    lib = ea.lib()
    G = 1 << 36  # far-apart addresses, so that no overlap is reported
    Q, K, V, O, L = (G * (i + 1) for i in range(5))
    n_max = (1 << 31) // (2 * d) - 1
    assert lib.attn_fwd_check(1, Q, K, V, O, L, 1, 1, n_max, d, 0.1, 2, 64, 0) == 0
    assert lib.attn_fwd_check(1, Q, K, V, O, L, 1, 1, n_max + 1, d, 0.1, 2, 64, 0) == 2


def test_grouped_and_packed_entry_points_reject_bad_arguments_before_any_hip_call():
    lib = ea.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    Q, K, V, O, L = base, base + 4096, base + 8192, base + 12288, base + 16384
    cu = base + 20480
    # H not a multiple of H_kv, H_kv larger than H, H_kv zero
    assert lib.attn_fwd_gqa(1, Q, K, V, O, L, 1, 6, 4, 8, 64, 0.1, 0, 0, 0, None) == 2
    assert lib.attn_fwd_gqa(1, Q, K, V, O, L, 1, 2, 4, 8, 64, 0.1, 0, 0, 0, None) == 2
    assert lib.attn_fwd_gqa(1, Q, K, V, O, L, 1, 2, 0, 8, 64, 0.1, 0, 0, 0, None) == 2
    # O overlapping V, which has H_kv = 1 head (1 KiB at N = 8, d = 64)
    assert lib.attn_fwd_gqa(1, Q, K, V, V + 512, L, 1, 4, 1, 8, 64, 0.1, 0, 0, 0, None) == 7
    # packed: NULL offsets, misaligned offsets, max_seqlen > T, no sequences,
    # offsets overlapping an output, unsupported d
    vargs = lambda cu_, n, mx, T, d=64: [0, Q, K, V, O, L, cu_, n, mx, T, 2, 1, d, 0.1, 1, 0, 0,
                                         None]
    assert lib.attn_fwd_varlen(*vargs(None, 2, 4, 8)) == 1
    assert lib.attn_fwd_varlen(*vargs(cu + 2, 2, 4, 8)) == 6
    assert lib.attn_fwd_varlen(*vargs(cu, 2, 9, 8)) == 2
    assert lib.attn_fwd_varlen(*vargs(cu, 0, 4, 8)) == 2
    assert lib.attn_fwd_varlen(*vargs(L, 2, 4, 8)) == 7
    assert lib.attn_fwd_varlen(*vargs(cu, 2, 4, 8, 96)) == 3
    # backward: workspace below attn_bwd_varlen_workspace_bytes
    ws = ea.attn_bwd_varlen_workspace_bytes(__import__("torch").float16, 2, 4, 8, 2, 1, 64)
    b = [0, Q, K, V, O, L, O, base + 24576, base + 28672, base + 32768, base + 36864, ws - 4,
         cu, 2, 4, 8, 2, 1, 64, 0.1, 1, 0, 0, None]
    assert lib.attn_bwd_varlen(*b) == 8
    g = [0, Q, K, V, O, L, O, base + 24576, base + 28672, base + 32768, base + 36864, ws,
         1, 6, 4, 8, 64, 0.1, 1, 0, 0, None]
    assert lib.attn_bwd_gqa(*g) == 2
    assert bytes(buf) == b"\0" * len(buf)


def test_grouped_workspace_sizes():
    """Per-row arrays as for attn_bwd; split groups (few key/value heads) add fp32 partials."""
    import torch
    f16 = torch.float16
    rows = lambda n: 2 * ((n * 4 + 255) // 256 * 256)
    # 512 key blocks with H_kv = 8 at B4 N4096: no split, same as standard attention
    assert ea.attn_bwd_workspace_bytes(f16, 4, 32, 4096, 128, 8) == rows(4 * 32 * 4096)
    assert ea.attn_bwd_workspace_bytes(f16, 4, 32, 4096, 128, 8) == \
        ea.attn_bwd_workspace_bytes(f16, 4, 32, 4096, 128)
    # multi-query at B4 N4096: 64 key blocks, split into 8 slices of 4 query heads
    assert ea.attn_bwd_workspace_bytes(f16, 4, 32, 4096, 128, 1) == \
        rows(4 * 32 * 4096) + 2 * 8 * (4 * 1 * 4096) * 128 * 4
    # a group of 3 with 1 block: split 3 (the only divisor reaching the target)
    assert ea.attn_bwd_workspace_bytes(f16, 1, 3, 100, 64, 1) == rows(300) + 2 * 3 * 100 * 64 * 4
    # packed: T = 32768 rows, H_kv = 8 -> 1024 blocks, no split
    assert ea.attn_bwd_varlen_workspace_bytes(f16, 15, 8192, 32768, 32, 8, 128) == rows(32 * 32768)
    assert ea.attn_bwd_varlen_workspace_bytes(f16, 2, 9, 8, 2, 1, 64) == 0  # max_seqlen > T


def test_decode_rejects_bad_arguments_before_any_hip_call():
    import torch
    lib = ea.lib()
    buf = ctypes.create_string_buffer(1 << 20)
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    K1 = 1 << 16
    Q, K, V, O, L = base, base + K1, base + 3 * K1, base + 5 * K1, base + 6 * K1
    bt, sl, ws = base + 7 * K1, base + 8 * K1, base + 9 * K1
    # n_seqs 2, H 4, H_kv 2, n_q 1, d 64, page 64, 4 pages, 2 pages per sequence, max_seqlen 128
    good = [0, Q, K, V, bt, sl, O, L, ws, 1 << 14, 2, 4, 2, 1, 64, 64, 4, 2, 128, 0.1, 0, 0, 0, None]

    def call(**kw):
        a = list(good)
        names = ["dt", "Q", "K", "V", "bt", "sl", "O", "L", "ws", "wsb", "n_seqs", "H", "H_kv",
                 "n_q", "d", "page", "n_pages", "max_pages", "max_seqlen", "scale", "mode", "wl",
                 "wr", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return lib.attn_decode(*a)

    assert call(page=32) == 3            # pages hold whole 64-key tiles
    assert call(page=96) == 3
    assert call(d=96) == 3
    assert call(max_seqlen=129) == 2     # beyond 2 pages of 64
    assert call(H=6, H_kv=4) == 2
    assert call(n_q=0) == 2
    assert call(bt=None) == 1
    assert call(sl=sl + 2) == 6          # int32 arrays need 4-byte alignment
    assert call(O=Q + 16) == 7           # output overlapping an input
    assert call(mode=2, wl=-1) == 4
    assert call(scale=float("inf")) == 5
    # few sequences and a long cache: the keys are split, which needs the workspace
    need = ea.attn_decode_workspace_bytes(torch.float16, 1, 8, 1, 1, 128, 65536)
    assert need > 0
    wbuf = ctypes.create_string_buffer(need + 256)
    wsp = (ctypes.addressof(wbuf) + 255) // 256 * 256
    assert lib.attn_decode(0, Q, K, V, bt, sl, O, L, None, 0, 1, 8, 1, 1, 128, 64, 4, 1024,
                           65536, 0.1, 0, 0, 0, None) == 1
    assert lib.attn_decode(0, Q, K, V, bt, sl, O, L, wsp, need - 4, 1, 8, 1, 1, 128, 64, 4, 1024,
                           65536, 0.1, 0, 0, 0, None) == 8
    assert bytes(wbuf) == b"\0" * len(wbuf)
    assert bytes(buf) == b"\0" * len(buf)


def test_decode_workspace_sizes():
    """No split (and no workspace) once sequences x key/value heads fill 512 workgroups."""
    import torch
    f = torch.bfloat16
    assert ea.attn_decode_workspace_bytes(f, 64, 32, 8, 1, 128, 8192) == 0
    # 1 sequence, 1 key/value head, 32 query rows: 128 tiles of 64 keys -> 128 splits of one tile
    parts = 128
    o_bytes = (parts * 32 * 128 * 4 + 255) // 256 * 256
    assert ea.attn_decode_workspace_bytes(f, 1, 32, 1, 1, 128, 8192) == o_bytes + parts * 32 * 4
    assert ea.attn_decode_workspace_bytes(f, 1, 6, 4, 1, 128, 100) == 0  # invalid group -> 0


def test_binding_rejects_mismatched_grouped_and_packed_shapes():
    """Shape checks of the wrappers (CPU tensors: they raise before any GPU use)."""
    import torch
    q = torch.zeros(1, 4, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        ea.attn_fwd(q, torch.zeros(1, 2, 9, 64, dtype=torch.float16),
                    torch.zeros(1, 2, 9, 64, dtype=torch.float16))
    with pytest.raises(ValueError):
        ea.attn_fwd(q, torch.zeros(1, 2, 8, 64, dtype=torch.float16),
                    torch.zeros(1, 1, 8, 64, dtype=torch.float16))
    qp = torch.zeros(4, 8, 64, dtype=torch.float16)
    kp = torch.zeros(2, 8, 64, dtype=torch.float16)
    cu = torch.tensor([0, 3, 8], dtype=torch.int32)
    with pytest.raises(ValueError):
        ea.attn_fwd_varlen(qp, torch.zeros(2, 7, 64, dtype=torch.float16), kp, cu, 5)
    with pytest.raises(ValueError):
        ea.attn_fwd_varlen(qp, kp, kp, cu, 5)  # inputs on the CPU


def test_fwd_tiles():
    for d in (64, 128):
        assert ea.attn_fwd_tiles(d, 0) == (256, 64)
        assert ea.attn_fwd_tiles(d, 1) == (128, 64)
        assert ea.attn_fwd_tiles(d, 2) == (128, 64)
    with pytest.raises(ea.AttnError):
        ea.attn_fwd_tiles(96)
    with pytest.raises(ea.AttnError):
        ea.attn_fwd_tiles(128, 3)


@pytest.mark.parametrize("N", [1, 17, 128, 333, 1000])
@pytest.mark.parametrize("mask", [None, "causal", (0, 0), (5, 0), (64, 3), (200, 200), (4096, 0)])
def test_kv_tile_range_matches_the_oracle_mask(N, mask):
    """Every visited tile holds an allowed pair and every allowed pair is in a visited tile."""
    mode, wl, wr = ea.mask_args(mask)
    name = ["none", "causal", "sliding"][mode]
    bq, bk = ea.attn_fwd_tiles(128, mode)
    keys = np.arange(N)
    for q0 in range(0, N, bq):
        lo, hi = ea.attn_kv_tile_range(N, q0, bq, bk, mode, wl, wr)
        rows = np.arange(q0, min(N, q0 + bq))
        A = oracle.allowed_matrix(rows, keys, N, name, wl, wr)
        tiles = np.unique(keys[A.any(axis=0)] // bk)
        assert lo == tiles.min() and hi == tiles.max() + 1
        assert len(tiles) == hi - lo


@pytest.mark.parametrize("n_heads,n_qblk", [(1, 1), (3, 5), (128, 32), (40, 256), (7, 3)])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_workgroup_order_is_a_bijection(n_heads, n_qblk, mode):
    seen = set()
    n = n_heads * n_qblk
    for wg in range(n):
        h, qb = ea.attn_fwd_workgroup(wg, n_heads, n_qblk, mode)
        assert 0 <= h < n_heads and 0 <= qb < n_qblk
        seen.add((h, qb))
    assert len(seen) == n
    with pytest.raises(ea.AttnError):
        ea.attn_fwd_workgroup(n, n_heads, n_qblk, mode)


def test_workgroup_order_keeps_a_head_on_one_die():
    """Ids are dealt round-robin to 8 dies; each die sees whole heads (128 heads x 32 blocks)."""
    n_heads, n_qblk = 128, 32
    die_heads = {}
    for wg in range(n_heads * n_qblk):
        h, _ = ea.attn_fwd_workgroup(wg, n_heads, n_qblk, 0)
        die_heads.setdefault(h, set()).add(wg % 8)
    assert all(len(d) == 1 for d in die_heads.values())


@pytest.mark.parametrize("n_heads,n_kblk", [(1, 1), (3, 5), (320, 16), (7, 3)])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_kv_workgroup_order_is_a_bijection(n_heads, n_kblk, mode):
    seen = set()
    n = n_heads * n_kblk
    for wg in range(n):
        h, kb = ea.attn_bwd_kv_workgroup(wg, n_heads, n_kblk, mode)
        assert 0 <= h < n_heads and 0 <= kb < n_kblk
        seen.add((h, kb))
    assert len(seen) == n
    with pytest.raises(ea.AttnError):
        ea.attn_bwd_kv_workgroup(n, n_heads, n_kblk, mode)
    with pytest.raises(ea.AttnError):
        ea.attn_bwd_kv_workgroup(0, n_heads, n_kblk, 3)


def test_causal_kv_order_is_heavy_first_and_keeps_heads_on_one_die():
    """Causal: ids are dealt round-robin to 8 dies; with 320 heads die x runs the
    heads h = x (mod 8), four at a time, key block 0 (every query tile) of the
    four first, then block 1, ...; with 7 heads (no grouping) block-major over all."""
    n_heads, n_kblk = 320, 16
    die_heads = {}
    per_die = {}
    for wg in range(n_heads * n_kblk):
        h, kb = ea.attn_bwd_kv_workgroup(wg, n_heads, n_kblk, 1)
        assert h % 8 == wg % 8
        die_heads.setdefault(h, set()).add(wg % 8)
        per_die.setdefault(wg % 8, []).append((h, kb))
    assert all(len(d) == 1 for d in die_heads.values())
    for seq in per_die.values():
        for g in range(0, len(seq), 4 * n_kblk):
            grp = seq[g:g + 4 * n_kblk]
            assert len({h for h, _ in grp}) == 4          # one group of four heads ...
            assert [kb for _, kb in grp] == sorted(kb for _, kb in grp)  # ... heaviest first
    prev = -1
    for wg in range(7 * 5):
        h, kb = ea.attn_bwd_kv_workgroup(wg, 7, 5, 1)
        assert kb >= prev and h == wg % 7
        prev = kb
    # other masks: the forward's head-major order
    for wg in (0, 17, 5119):
        assert ea.attn_bwd_kv_workgroup(wg, n_heads, n_kblk, 0) == ea.attn_fwd_workgroup(
            wg, n_heads, n_kblk, 0)


def test_causal_runs_longest_query_blocks_first():
    h0, qb0 = ea.attn_fwd_workgroup(0, 4, 16, 1)
    assert qb0 == 15
    h0, qb0 = ea.attn_fwd_workgroup(0, 4, 16, 0)
    assert qb0 == 0


@pytest.mark.parametrize("n_heads", [128, 320, 6])
def test_causal_order_runs_four_heads_at_a_time(n_heads):
    """Causal: ids are dealt round-robin to 8 dies and die x runs a contiguous run of
    the item sequence, so die 0's items, then die 1's, ... give that sequence.  It
    takes four consecutive heads at a time (a short last chunk alike): the last
    query block of each of the four, then the second-to-last of each, ..."""
    n_qblk = 32
    per_die = {}
    for wg in range(n_heads * n_qblk):
        per_die.setdefault(wg % 8, []).append(ea.attn_fwd_workgroup(wg, n_heads, n_qblk, 1))
    seq = [hq for x in range(8) for hq in per_die.get(x, [])]
    assert sorted(seq) == sorted((h, qb) for h in range(n_heads) for qb in range(n_qblk))
    pos = 0
    for c in range(0, n_heads, 4):
        nh = min(4, n_heads - c)
        grp = seq[pos:pos + nh * n_qblk]
        pos += nh * n_qblk
        assert [h for h, _ in grp] == [c + r % nh for r in range(nh * n_qblk)]
        assert [qb for _, qb in grp] == [n_qblk - 1 - r // nh for r in range(nh * n_qblk)]
    if n_heads % 8 == 0:  # whole heads per die
        dies = {}
        for wg in range(n_heads * n_qblk):
            dies.setdefault(ea.attn_fwd_workgroup(wg, n_heads, n_qblk, 1)[0], set()).add(wg % 8)
        assert all(len(d) == 1 for d in dies.values())


def test_binding_rejects_host_tensors_before_any_library_call():
    """CPU tensors never reach the kernels: the binding raises first."""
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        ea.attn_fwd(q, q, q)
    lse = torch.zeros(1, 1, 8, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        ea.attn_bwd(q, q, q, q, lse, q)
    with pytest.raises(ValueError, match="shape"):
        ea.attn_bwd(q, q[:, :, :4], q, q, lse, q)


def test_noalloc_backward_validates_before_any_hip_call():
    """attn_bwd_noalloc checks every argument like attn_bwd, and sizes whose
    workspace exceeds its fixed scratch fail with ATTN_E_SCRATCH, all before
    any HIP call and without touching the buffers."""
    lib = ea.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    Q, K, V, O, L, dO = (base + 4096 * i for i in range(6))
    dQ, dK, dV = (base + 4096 * i for i in range(6, 9))
    ok = [0, Q, K, V, O, L, dO, dQ, dK, dV, 1, 1, 8, 64, 0.1, 1, 0, 0, None]
    bad = list(ok)
    bad[1] = None
    assert lib.attn_bwd_noalloc(*bad) == 1            # NULL input
    bad = list(ok)
    bad[7] = Q + 16
    assert lib.attn_bwd_noalloc(*bad) == 7            # dQ overlaps Q
    bad = list(ok)
    bad[13] = 96
    assert lib.attn_bwd_noalloc(*bad) == 3            # unsupported d
    assert bytes(buf) == b"\0" * len(buf)
    # Sizes beyond the scratch: addresses far apart so nothing overlaps (never dereferenced).
    big = [0] + [(i + 1) << 40 for i in range(9)] + [1, 1, 5_000_000, 64, 0.1, 0, 0, 0, None]
    need = ea.attn_bwd_workspace_bytes(__import__("torch").float16, 1, 1, 5_000_000, 64)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    assert lib.attn_bwd_noalloc(*big) == 10
    # the largest row count that fits: two 256-byte-padded float32 arrays
    rows = binding.NOALLOC_SCRATCH_BYTES // 8 // 64 * 64
    assert ea.attn_bwd_workspace_bytes(__import__("torch").float16, 1, 1, rows, 64) <= \
        binding.NOALLOC_SCRATCH_BYTES
