"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to the storage type.
It holds none of the attention arithmetic, so both the fp64 oracle (``oracle/``)
and the HIP path (``exact_attention_14_amd``) may take their inputs from it
without sharing any of the method's code.

Recipe (the same for every workload):
  * generator: numpy ``default_rng(seed)`` (PCG64);
  * Q, K, V and then (for the backward workload) the upstream gradient dO are
    drawn, in that order, as float32 standard normals of shape [B, H, N, d]
    in C order;
  * each float32 tensor is rounded once, to nearest-even, to fp16 or bf16;
  * the causal outlier workload then picks round(0.01 * N) distinct key rows per
    (b, h), b-major then h, uniformly without replacement from the same
    generator, and multiplies those K rows by 8 (a power of two, so exact).

Inputs too large to draw on the host (the longest head the boundary accepts)
are drawn on the GPU by torch's seeded Philox generator instead
(``draw_on_device``), with the same order and rounding.

Grouped-query inputs draw K and V with H_kv heads; packed variable-length inputs
are [H, T, d] (K, V [H_kv, T, d]) with row offsets from ``packed_offsets`` and
lengths, for the mixed-length workloads, from ``length_mix`` (log-uniform,
seeded).

The pages measure on model-shaped random activations (LLaMA-7B / LLaMA-13B
attention shapes, and a long-sequence window case); i.i.d. N(0, 1) inputs of the
same shapes stand in for them.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f16" or "bf16": storage type of Q, K, V, O (and dO)
    mask: str           # "none", "causal" or "sliding"
    window_left: int    # read only for "sliding"
    window_right: int   # read only for "sliding"
    seed: int
    backward: bool = False       # also draw dO (forward + backward workload)
    outlier_frac: float = 0.0    # fraction of K rows per head scaled by outlier_mul
    outlier_mul: float = 1.0
    H_kv: int = 0                # key/value heads (grouped-query); 0 means H
    # Packed variable-length batch: N is then the total row count T (B = 1),
    # split into sequences by length_mix(N, packed_lo, packed_hi, packed_seed).
    packed_lo: int = 0
    packed_hi: int = 0
    packed_seed: int = 0
    # Decoding over a paged cache: B sequences of N cached keys each, with
    # decode_q new query tokens per sequence and pages of page_size keys.
    decode_q: int = 0
    page_size: int = 0

    @property
    def kv_heads(self) -> int:
        return self.H_kv if self.H_kv > 0 else self.H

    @property
    def packed(self) -> bool:
        return self.packed_hi > 0

    @property
    def lengths(self) -> list:
        """Sequence lengths of a packed workload; [N] * B otherwise."""
        if not self.packed:
            return [self.N] * self.B
        return length_mix(self.N, self.packed_lo, self.packed_hi, self.packed_seed)

    @property
    def scale(self) -> float:
        """Score scale 1/sqrt(d), as the float32 value handed to the kernels."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[self.dtype]


# The five workloads, named by what they are.
SINGLE_HEAD_N256 = Workload("b1h1n256d64_f16_full", 1, 1, 256, 64, "f16", "none", 0, 0, seed=1)
FULL_N4096 = Workload("b4h32n4096d128_bf16_full", 4, 32, 4096, 128, "bf16", "none", 0, 0, seed=2)
CAUSAL_OUTLIERS_N4096 = Workload("b4h32n4096d128_bf16_causal_outlierkeys", 4, 32, 4096, 128, "bf16",
                                 "causal", 0, 0, seed=3, outlier_frac=0.01, outlier_mul=8.0)
LLAMA13B_CAUSAL_FWDBWD = Workload("b8h40n4096d128_f16_causal_fwdbwd", 8, 40, 4096, 128, "f16",
                                  "causal", 0, 0, seed=4, backward=True)
SLIDING_N32768 = Workload("b1h40n32768d128_bf16_sliding4096", 1, 40, 32768, 128, "bf16",
                          "sliding", 4096, 0, seed=5)

# Grouped-query and packed variable-length workloads (P1 §5's extensions):
# LLaMA-3-8B's attention shape (32 query heads, 8 key/value heads, d = 128),
# fixed-length and as a packed batch of mixed-length sequences, and the same
# query shape with one shared key/value head (multi-query attention).
GQA_CAUSAL_FWDBWD = Workload("b4h32kv8n4096d128_bf16_causal_gqa_fwdbwd", 4, 32, 4096, 128, "bf16",
                             "causal", 0, 0, seed=7, backward=True, H_kv=8)
MQA_CAUSAL_FWDBWD = Workload("b4h32kv1n4096d128_bf16_causal_mqa_fwdbwd", 4, 32, 4096, 128, "bf16",
                             "causal", 0, 0, seed=9, backward=True, H_kv=1)
PACKED_CAUSAL_FWDBWD = Workload("h32kv8t32768d128_bf16_causal_packed128to8192_fwdbwd", 1, 32,
                                32768, 128, "bf16", "causal", 0, 0, seed=8, backward=True, H_kv=8,
                                packed_lo=128, packed_hi=8192, packed_seed=6)

# Decoding: 64 sequences with 8192 cached tokens each, one new token, the
# LLaMA-3-8B attention shape, 64-key pages.
DECODE_CTX8192 = Workload("decode_s64h32kv8q1ctx8192d128_bf16_page64", 64, 32, 8192, 128, "bf16",
                          "none", 0, 0, seed=10, H_kv=8, decode_q=1, page_size=64)

# Long-context decoding: 4 sequences of 131072 cached tokens; 4 x 8 (sequence,
# key/value head) items, so the keys are split over workgroups.
DECODE_CTX131072 = Workload("decode_s4h32kv8q1ctx131072d128_bf16_page256", 4, 32, 131072, 128,
                            "bf16", "none", 0, 0, seed=11, H_kv=8, decode_q=1, page_size=256)

ALL = (SINGLE_HEAD_N256, FULL_N4096, CAUSAL_OUTLIERS_N4096, LLAMA13B_CAUSAL_FWDBWD, SLIDING_N32768,
       GQA_CAUSAL_FWDBWD, MQA_CAUSAL_FWDBWD, PACKED_CAUSAL_FWDBWD, DECODE_CTX8192,
       DECODE_CTX131072)
BY_NAME = {w.name: w for w in ALL}


def _round(x32: np.ndarray, dtype: str) -> torch.Tensor:
    """Round a float32 array once, to nearest-even, to the storage type."""
    return torch.from_numpy(x32).to(_TORCH_DTYPES[dtype])


def draw(B: int, H: int, N: int, d: int, dtype: str, seed: int, *, with_do: bool = False,
         outlier_frac: float = 0.0, outlier_mul: float = 1.0) -> dict:
    """Draw Q, K, V (and dO) on the host, rounded to ``dtype``.

    Returns a dict of CPU torch tensors of shape [B, H, N, d]; with outliers it
    also holds ``outlier_rows`` (an int64 array [B, H, n_out]) for reference.
    """
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    out = {}
    for key in ("q", "k", "v") + (("do",) if with_do else ()):
        out[key] = _round(rng.standard_normal(shape, dtype=np.float32), dtype)
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * N))
        rows = np.empty((B, H, n_out), dtype=np.int64)
        for b in range(B):
            for h in range(H):
                rows[b, h] = rng.choice(N, size=n_out, replace=False)
        kk = out["k"]
        mul = torch.tensor(outlier_mul, dtype=kk.dtype)
        for b in range(B):
            for h in range(H):
                idx = torch.from_numpy(rows[b, h])
                kk[b, h, idx] = kk[b, h, idx] * mul
        out["outlier_rows"] = rows
    return out


def draw_on_device(B: int, H: int, N: int, d: int, dtype: str, seed: int, *,
                   with_do: bool = False, device: str = "cuda") -> dict:
    """Q, K, V (and dO) drawn on the GPU, for inputs too large to draw on the host.

    torch's seeded device generator (Philox) draws float32 standard normals of
    shape [B, H, N, d], Q, K, V, dO in that order, each rounded once
    (nearest-even) to ``dtype``.  Returns device tensors; slices copied to the
    host feed the oracle, so both sides see the same values.
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = {}
    for key in ("q", "k", "v") + (("do",) if with_do else ()):
        x = torch.randn((B, H, N, d), generator=g, device=device, dtype=torch.float32)
        out[key] = x.to(_TORCH_DTYPES[dtype])
        del x
    return out


def draw_grouped(B: int, H: int, H_kv: int, N: int, d: int, dtype: str, seed: int, *,
                 with_do: bool = False) -> dict:
    """Q [B, H, N, d], K and V [B, H_kv, N, d] (and dO [B, H, N, d]), in that order."""
    rng = np.random.default_rng(seed)
    out = {}
    for key, heads in (("q", H), ("k", H_kv), ("v", H_kv)) + ((("do", H),) if with_do else ()):
        out[key] = _round(rng.standard_normal((B, heads, N, d), dtype=np.float32), dtype)
    return out


def draw_packed(H: int, H_kv: int, T: int, d: int, dtype: str, seed: int, *,
                with_do: bool = False) -> dict:
    """Packed batch: Q [H, T, d], K and V [H_kv, T, d] (and dO [H, T, d]), in that order."""
    rng = np.random.default_rng(seed)
    out = {}
    for key, heads in (("q", H), ("k", H_kv), ("v", H_kv)) + ((("do", H),) if with_do else ()):
        out[key] = _round(rng.standard_normal((heads, T, d), dtype=np.float32), dtype)
    return out


def packed_offsets(lengths) -> np.ndarray:
    """Row offsets (int32, n + 1 entries, starting at 0) of sequences packed in order."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def length_mix(total: int, lo: int, hi: int, seed: int) -> list:
    """Sequence lengths drawn log-uniformly from [lo, hi] until they fill ``total`` rows
    (the last one is cut to fit): a mixed-length packed batch of exactly ``total`` rows."""
    rng = np.random.default_rng(seed)
    out, used = [], 0
    while used < total:
        n = int(round(float(np.exp(rng.uniform(np.log(lo), np.log(hi))))))
        n = min(max(n, 1), total - used)
        out.append(n)
        used += n
    return out


def draw_paged(lens, H: int, H_kv: int, n_q: int, d: int, dtype: str, page_size: int, seed: int,
               spare_pages: int = 2) -> dict:
    """Decode inputs over a paged cache: Q [n_seqs, H, n_q, d] and page pools K, V
    [n_pages, H_kv, page_size, d] drawn in that order (sequence by sequence,
    K then V of each); the pages of all sequences are dealt to a random
    permutation of the pool, and every pool row no sequence owns (the tails of
    last pages and the spare pages) is NaN, so reading one shows.  Also returns
    block_table (int32 [n_seqs, max_pages]) and seq_lens (int32 [n_seqs])."""
    rng = np.random.default_rng(seed)
    n_seqs = len(lens)
    q = rng.standard_normal((n_seqs, H, n_q, d), dtype=np.float32)
    per = [max(1, -(-int(L) // page_size)) for L in lens]
    n_pages = sum(per) + spare_pages
    perm = rng.permutation(n_pages)
    K = np.full((n_pages, H_kv, page_size, d), np.nan, dtype=np.float32)
    V = np.full((n_pages, H_kv, page_size, d), np.nan, dtype=np.float32)
    table = np.zeros((n_seqs, max(per)), dtype=np.int32)
    used = 0
    for s, L in enumerate(lens):
        ks = rng.standard_normal((H_kv, int(L), d), dtype=np.float32)
        vs = rng.standard_normal((H_kv, int(L), d), dtype=np.float32)
        for pg in range(per[s]):
            phys = int(perm[used])
            used += 1
            table[s, pg] = phys
            lo, hi = pg * page_size, min(int(L), (pg + 1) * page_size)
            K[phys, :, :hi - lo] = ks[:, lo:hi]
            V[phys, :, :hi - lo] = vs[:, lo:hi]
    return {"q": _round(q, dtype), "k": _round(K, dtype), "v": _round(V, dtype),
            "block_table": torch.from_numpy(table),
            "seq_lens": torch.from_numpy(np.asarray(lens, dtype=np.int32))}


def make_inputs(w: Workload) -> dict:
    """The seeded inputs of a named workload (CPU tensors); packed workloads also
    hold ``cu_seqlens`` (int32 row offsets)."""
    if w.decode_q > 0:
        return draw_paged([w.N] * w.B, w.H, w.kv_heads, w.decode_q, w.d, w.dtype, w.page_size,
                          w.seed, spare_pages=0)
    if w.packed:
        out = draw_packed(w.H, w.kv_heads, w.N, w.d, w.dtype, w.seed, with_do=w.backward)
        out["cu_seqlens"] = torch.from_numpy(packed_offsets(w.lengths))
        return out
    if w.kv_heads != w.H:
        return draw_grouped(w.B, w.H, w.kv_heads, w.N, w.d, w.dtype, w.seed, with_do=w.backward)
    return draw(w.B, w.H, w.N, w.d, w.dtype, w.seed, with_do=w.backward,
                outlier_frac=w.outlier_frac, outlier_mul=w.outlier_mul)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of an fp16/bf16 CPU tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
