"""Thin ctypes binding over libattn.so: argument marshalling only.

The names match the C ABI in ``include/attn.h``.  Every step of the forward and
backward runs in the library's HIP kernels; this module only checks torch
tensors, allocates outputs with torch on the tensors' device, and passes raw
pointers plus torch's current HIP stream.  There is no fallback of any kind:
if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

# The in-tree library; EXACT_ATTN_LIB may name another build of it (a tile-shape
# variant from ``build --out``) for sweeps.
_LIB_PATH = os.environ.get("EXACT_ATTN_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libattn.so")
_lib = None

ATTN_F16, ATTN_BF16 = 0, 1
ATTN_MASK_NONE, ATTN_MASK_CAUSAL, ATTN_MASK_SLIDING = 0, 1, 2
STATUS = {0: "ATTN_OK", 1: "ATTN_E_NULLPTR", 2: "ATTN_E_SHAPE", 3: "ATTN_E_UNSUPPORTED",
          4: "ATTN_E_MASK", 5: "ATTN_E_SCALE", 6: "ATTN_E_ALIGN", 7: "ATTN_E_ALIAS",
          8: "ATTN_E_WORKSPACE", 9: "ATTN_E_HIP", 10: "ATTN_E_SCRATCH"}

# Fixed device scratch of attn_bwd_noalloc per GPU (ATTN_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol include/attn.h declares.
EXPORTS = ("attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_status_str",
           "attn_fwd_check", "attn_bwd_check", "attn_fwd_tiles", "attn_kv_tile_range",
           "attn_fwd_workgroup", "attn_bwd_kv_workgroup", "attn_fwd_gqa", "attn_bwd_gqa",
           "attn_fwd_varlen", "attn_bwd_varlen", "attn_bwd_gqa_workspace_bytes",
           "attn_bwd_varlen_workspace_bytes", "attn_decode", "attn_decode_workspace_bytes",
           "attn_bwd_noalloc", "attn_fwd_persistent")


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({message})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libattn.so (built by ``exact_attention_14_amd.build``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m exact_attention_14_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64, f32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    p64 = ctypes.POINTER(ctypes.c_int64)
    L.attn_fwd.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i64, i64, vp]
    L.attn_fwd.restype = i32
    L.attn_fwd_check.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i64, i64]
    L.attn_fwd_check.restype = i32
    L.attn_bwd.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64,
                           f32, i32, i64, i64, vp]
    L.attn_bwd.restype = i32
    L.attn_bwd_check.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64,
                                 i64, f32, i32, i64, i64]
    L.attn_bwd_noalloc.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                   f32, i32, i64, i64, vp]
    L.attn_bwd_noalloc.restype = i32
    L.attn_bwd_check.restype = i32
    L.attn_fwd_gqa.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i64, i64,
                               vp]
    L.attn_fwd_gqa.restype = i32
    L.attn_fwd_persistent.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32,
                                      i64, i64, vp]
    L.attn_fwd_persistent.restype = i32
    L.attn_bwd_gqa.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64,
                               i64, f32, i32, i64, i64, vp]
    L.attn_bwd_gqa.restype = i32
    L.attn_fwd_varlen.argtypes = [i32, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32,
                                  i32, i64, i64, vp]
    L.attn_fwd_varlen.restype = i32
    L.attn_bwd_varlen.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i64, i64,
                                  i64, i64, i64, i64, f32, i32, i64, i64, vp]
    L.attn_bwd_varlen.restype = i32
    L.attn_bwd_gqa_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i64]
    L.attn_bwd_gqa_workspace_bytes.restype = sz
    L.attn_bwd_varlen_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i64, i64]
    L.attn_bwd_varlen_workspace_bytes.restype = sz
    L.attn_decode.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64, i64,
                              i64, i64, i64, i64, f32, i32, i64, i64, vp]
    L.attn_decode.restype = i32
    L.attn_decode_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i64, i64]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_bwd_workspace_bytes.argtypes = [i32, i64, i64, i64, i64]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_status_str.argtypes = [i32]
    L.attn_status_str.restype = ctypes.c_char_p
    L.attn_fwd_tiles.argtypes = [i64, i32, p64, p64]
    L.attn_fwd_tiles.restype = i32
    L.attn_kv_tile_range.argtypes = [i64, i64, i64, i64, i32, i64, i64, p64, p64]
    L.attn_kv_tile_range.restype = i32
    L.attn_fwd_workgroup.argtypes = [i64, i64, i64, i32, p64, p64]
    L.attn_fwd_workgroup.restype = i32
    L.attn_bwd_kv_workgroup.argtypes = [i64, i64, i64, i32, p64, p64]
    L.attn_bwd_kv_workgroup.restype = i32
    _lib = L
    return L


def attn_status_str(status: int) -> str:
    return lib().attn_status_str(status).decode()


def _raise(fn: str, status: int):
    if status != 0:
        raise AttnError(fn, status, attn_status_str(status))


def mask_args(mask) -> tuple:
    """None -> none; "causal" -> causal; (window_left, window_right) -> sliding.

    Mirrors the mask argument of the pages' Python interface (P4 "usage"),
    with an explicit string for causal instead of inferring it from a tensor.
    """
    if mask is None or mask == "none":
        return ATTN_MASK_NONE, 0, 0
    if mask == "causal":
        return ATTN_MASK_CAUSAL, 0, 0
    if isinstance(mask, (tuple, list)) and len(mask) == 2:
        return ATTN_MASK_SLIDING, int(mask[0]), int(mask[1])
    raise ValueError(f"mask must be None, 'causal' or (window_left, window_right), got {mask!r}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16")


def _check4(name: str, t: torch.Tensor, ref: torch.Tensor):
    if t.dim() != 4 or tuple(t.shape) != tuple(ref.shape):
        raise ValueError(f"{name} must have shape {tuple(ref.shape)}, got {tuple(t.shape)}")
    if t.dtype != ref.dtype or t.device != ref.device:
        raise ValueError(f"{name} must be {ref.dtype} on {ref.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, N, d]")


def _check_kv(name: str, t: torch.Tensor, q: torch.Tensor, ref: torch.Tensor):
    """K, V (and dK, dV) have q's shape except for the head count, that of ``ref``."""
    want = (q.shape[0], ref.shape[1]) + tuple(q.shape[2:])
    if t.dim() != 4 or tuple(t.shape) != want:
        raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
    if t.dtype != q.dtype or t.device != q.device:
        raise ValueError(f"{name} must be {q.dtype} on {q.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_gpu(q: torch.Tensor):
    if not q.is_cuda:
        raise ValueError("inputs must be on a GPU")


def _check_lse(lse: torch.Tensor, q: torch.Tensor):
    B, H, N, _ = q.shape
    if (tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError(f"lse must be contiguous float32 [B, H, N] on {q.device}")


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, mask=None, scale=None,
             out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
             persistent: bool = False):
    """Forward pass; returns (O, lse).  Inputs: contiguous q [B, H, N, d] and k, v
    [B, H_kv, N, d] on a GPU (H_kv < H: grouped-query attention, query head h
    reads key/value head h // (H // H_kv)).

    ``scale`` defaults to 1/sqrt(d) (P1 §1).  ``out``/``lse`` may be given to
    write into preallocated buffers.  ``persistent`` selects the library's
    persistent-scheduling entry point (attn_fwd_persistent; same results).
    """
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, N, d] and k [B, H_kv, N, d]")
    _check4("q", q, q)
    _check_kv("k", k, q, k)
    _check_kv("v", v, q, k)
    _check_gpu(q)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mode, wl, wr = mask_args(mask)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check4("out", out, q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_lse(lse, q)
    # The library launches on the calling thread's current device.
    with torch.cuda.device(q.device):
        if persistent:
            fn = "attn_fwd_persistent"
            st = lib().attn_fwd_persistent(dt, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           out.data_ptr(), lse.data_ptr(), B, H, H_kv, N, d,
                                           float(scale), mode, wl, wr, _stream_ptr(q.device))
        elif H_kv == H:
            fn = "attn_fwd"
            st = lib().attn_fwd(dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, H, N, d, float(scale), mode, wl, wr,
                                _stream_ptr(q.device))
        else:
            fn = "attn_fwd_gqa"
            st = lib().attn_fwd_gqa(dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, H, H_kv, N, d, float(scale), mode, wl, wr,
                                    _stream_ptr(q.device))
    _raise(fn, st)
    return out, lse


def _code(dtype: torch.dtype) -> int:
    return ATTN_BF16 if dtype == torch.bfloat16 else ATTN_F16


def attn_bwd_workspace_bytes(dtype: torch.dtype, B: int, H: int, N: int, d: int,
                             H_kv: int | None = None) -> int:
    """Workspace bytes of attn_bwd (or, with H_kv < H, of its grouped-query form)."""
    if H_kv is None or H_kv == H:
        return int(lib().attn_bwd_workspace_bytes(_code(dtype), B, H, N, d))
    return int(lib().attn_bwd_gqa_workspace_bytes(_code(dtype), B, H, H_kv, N, d))


def attn_bwd_varlen_workspace_bytes(dtype: torch.dtype, n_seqs: int, max_seqlen: int, total: int,
                                    H: int, H_kv: int, d: int) -> int:
    return int(lib().attn_bwd_varlen_workspace_bytes(_code(dtype), n_seqs, max_seqlen, total, H,
                                                     H_kv, d))


def attn_bwd(q, k, v, o, lse, do, *, mask=None, scale=None, workspace=None):
    """Recomputation backward; returns (dQ, dK, dV) for upstream gradient ``do``.

    k, v (and the returned dK, dV) may have fewer heads than q (grouped-query
    attention); dK, dV then sum over each key/value head's query heads.
    """
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, N, d] and k [B, H_kv, N, d]")
    _check4("q", q, q)
    for name, t in (("o", o), ("do", do)):
        _check4(name, t, q)
    _check_kv("k", k, q, k)
    _check_kv("v", v, q, k)
    _check_gpu(q)
    _check_lse(lse, q)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mode, wl, wr = mask_args(mask)
    dt = _dtype_code(q)
    need = attn_bwd_workspace_bytes(q.dtype, B, H, N, d, H_kv)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {q.device}")
    ws_bytes = workspace.numel() * workspace.element_size()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    with torch.cuda.device(q.device):
        if H_kv == H:
            fn = "attn_bwd"
            st = lib().attn_bwd(dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), workspace.data_ptr(), ws_bytes, B, H, N, d,
                                float(scale), mode, wl, wr, _stream_ptr(q.device))
        else:
            fn = "attn_bwd_gqa"
            st = lib().attn_bwd_gqa(dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                    dv.data_ptr(), workspace.data_ptr(), ws_bytes, B, H, H_kv, N,
                                    d, float(scale), mode, wl, wr, _stream_ptr(q.device))
    _raise(fn, st)
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, do, *, out=None, mask=None, scale=None):
    """attn_bwd through the library's allocation-free entry point (fixed per-GPU
    scratch; standard multi-head attention, H_kv = H).  ``out`` may hold
    caller-allocated (dQ, dK, dV) tensors, so that a call allocates nothing."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check4(name, t, q)
    _check_gpu(q)
    _check_lse(lse, q)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mode, wl, wr = mask_args(mask)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    for name, t in zip(("dq", "dk", "dv"), out):
        _check4(name, t, q)
    dq, dk, dv = out
    with torch.cuda.device(q.device):
        st = lib().attn_bwd_noalloc(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                                    dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale), mode,
                                    wl, wr, _stream_ptr(q.device))
    _raise("attn_bwd_noalloc", st)
    return dq, dk, dv


def _check_packed(q, k, v):
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed q must be [H, T, d] and k, v [H_kv, T, d]")
    H, T, d = q.shape
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (k.shape[0], T, d) or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must be {q.dtype} [H_kv, {T}, {d}] on {q.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    return H, k.shape[0], T, d


def _check_offsets(cu_seqlens, q):
    if (cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2 or cu_seqlens.dtype != torch.int32
            or cu_seqlens.device != q.device or not cu_seqlens.is_contiguous()):
        raise ValueError(f"cu_seqlens must be a contiguous int32 vector of n_seqs + 1 row offsets "
                         f"on {q.device}")
    return cu_seqlens.numel() - 1


def attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, *, mask=None, scale=None, out=None,
                    lse=None):
    """Forward over a packed variable-length batch; returns (O [H, T, d], lse [H, T]).

    q: [H, T, d]; k, v: [H_kv, T, d]; sequence s is rows cu_seqlens[s] ..
    cu_seqlens[s+1] - 1 and attends only to itself (masks count positions from
    its first row).  ``max_seqlen`` must be at least every sequence's length.
    Rows outside every sequence are left as they are in ``out`` / ``lse``.
    """
    H, H_kv, T, d = _check_packed(q, k, v)
    _check_gpu(q)
    n_seqs = _check_offsets(cu_seqlens, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mode, wl, wr = mask_args(mask)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError(f"out must be contiguous {q.dtype} {tuple(q.shape)}")
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (H, T) or lse.dtype != torch.float32 or not lse.is_contiguous()
          or lse.device != q.device):
        raise ValueError(f"lse must be contiguous float32 [H, T] on {q.device}")
    with torch.cuda.device(q.device):
        st = lib().attn_fwd_varlen(dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), cu_seqlens.data_ptr(), n_seqs, int(max_seqlen),
                                   T, H, H_kv, d, float(scale), mode, wl, wr,
                                   _stream_ptr(q.device))
    _raise("attn_fwd_varlen", st)
    return out, lse


def attn_bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen: int, *, mask=None, scale=None,
                    workspace=None):
    """Backward over a packed variable-length batch; returns (dQ, dK, dV).

    Shapes as for attn_fwd_varlen; o and do are [H, T, d], lse [H, T].  Rows
    outside every sequence of the returned tensors are unspecified.
    """
    H, H_kv, T, d = _check_packed(q, k, v)
    _check_gpu(q)
    for name, t in (("o", o), ("do", do)):
        if tuple(t.shape) != tuple(q.shape) or t.dtype != q.dtype or not t.is_contiguous() \
                or t.device != q.device:
            raise ValueError(f"{name} must be contiguous {q.dtype} {tuple(q.shape)} on {q.device}")
    if (tuple(lse.shape) != (H, T) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError(f"lse must be contiguous float32 [H, T] on {q.device}")
    n_seqs = _check_offsets(cu_seqlens, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mode, wl, wr = mask_args(mask)
    dt = _dtype_code(q)
    need = attn_bwd_varlen_workspace_bytes(q.dtype, n_seqs, int(max_seqlen), T, H, H_kv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {q.device}")
    ws_bytes = workspace.numel() * workspace.element_size()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    with torch.cuda.device(q.device):
        st = lib().attn_bwd_varlen(dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), workspace.data_ptr(), ws_bytes,
                                   cu_seqlens.data_ptr(), n_seqs, int(max_seqlen), T, H, H_kv, d,
                                   float(scale), mode, wl, wr, _stream_ptr(q.device))
    _raise("attn_bwd_varlen", st)
    return dq, dk, dv


def attn_kv_tile_range(N, q0, block_q, block_k, mode, wl=0, wr=0):
    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    st = lib().attn_kv_tile_range(N, q0, block_q, block_k, mode, wl, wr, ctypes.byref(lo),
                                  ctypes.byref(hi))
    _raise("attn_kv_tile_range", st)
    return lo.value, hi.value


def attn_fwd_tiles(d, mode=ATTN_MASK_NONE):
    bq, bk = ctypes.c_int64(), ctypes.c_int64()
    _raise("attn_fwd_tiles", lib().attn_fwd_tiles(d, mode, ctypes.byref(bq), ctypes.byref(bk)))
    return bq.value, bk.value


def attn_fwd_workgroup(wg, n_heads, n_qblk, mode):
    h, qb = ctypes.c_int64(), ctypes.c_int64()
    st = lib().attn_fwd_workgroup(wg, n_heads, n_qblk, mode, ctypes.byref(h), ctypes.byref(qb))
    _raise("attn_fwd_workgroup", st)
    return h.value, qb.value


def attn_bwd_kv_workgroup(wg, n_heads, n_kblk, mode):
    h, kb = ctypes.c_int64(), ctypes.c_int64()
    st = lib().attn_bwd_kv_workgroup(wg, n_heads, n_kblk, mode, ctypes.byref(h), ctypes.byref(kb))
    _raise("attn_bwd_kv_workgroup", st)
    return h.value, kb.value


def attn_decode_workspace_bytes(dtype: torch.dtype, n_seqs: int, H: int, H_kv: int, n_q: int,
                                d: int, max_seqlen: int) -> int:
    return int(lib().attn_decode_workspace_bytes(_code(dtype), n_seqs, H, H_kv, n_q, d, max_seqlen))


def attn_decode(q, k_cache, v_cache, block_table, seq_lens, max_seqlen: int, *, mask=None,
                scale=None, out=None, lse=None, workspace=None):
    """Split-KV decoding over a paged cache; returns (O [n_seqs, H, n_q, d], lse [n_seqs, H, n_q]).

    q: [n_seqs, H, n_q, d]; k_cache, v_cache: [n_pages, H_kv, page_size, d] page pools;
    block_table: int32 [n_seqs, max_pages]; seq_lens: int32 [n_seqs] (cache lengths, each at
    least n_q and at most ``max_seqlen``).  The n_q query tokens of a sequence sit at its last
    n_q cache positions; masks count cache positions.
    """
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q must be [n_seqs, H, n_q, d] and the caches [n_pages, H_kv, page_size, d]")
    n_seqs, H, n_q, d = q.shape
    n_pages, H_kv, page_size, dk = k_cache.shape
    _check_gpu(q)
    for name, t, shape in (("q", q, tuple(q.shape)), ("k_cache", k_cache, tuple(k_cache.shape)),
                           ("v_cache", v_cache, tuple(k_cache.shape))):
        if tuple(t.shape) != shape or t.dtype != q.dtype or t.device != q.device \
                or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous {q.dtype} {shape} on {q.device}")
    if dk != d:
        raise ValueError("q and the caches must have the same head size")
    if (block_table.dim() != 2 or block_table.shape[0] != n_seqs or block_table.dtype != torch.int32
            or block_table.device != q.device or not block_table.is_contiguous()):
        raise ValueError(f"block_table must be a contiguous int32 [n_seqs, max_pages] on {q.device}")
    if (tuple(seq_lens.shape) != (n_seqs,) or seq_lens.dtype != torch.int32
            or seq_lens.device != q.device or not seq_lens.is_contiguous()):
        raise ValueError(f"seq_lens must be a contiguous int32 [n_seqs] on {q.device}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mode, wl, wr = mask_args(mask)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    elif (tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError(f"out must be contiguous {q.dtype} {tuple(q.shape)} on {q.device}")
    if lse is None:
        lse = torch.empty((n_seqs, H, n_q), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (n_seqs, H, n_q) or lse.dtype != torch.float32
          or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError(f"lse must be contiguous float32 [n_seqs, H, n_q] on {q.device}")
    need = attn_decode_workspace_bytes(q.dtype, n_seqs, H, H_kv, n_q, d, int(max_seqlen))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace is not None and (workspace.device != q.device or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous tensor on {q.device}")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(q.device):
        st = lib().attn_decode(dt, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                               block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), ws_ptr, ws_bytes, n_seqs, H, H_kv, n_q, d,
                               page_size, n_pages, block_table.shape[1], int(max_seqlen),
                               float(scale), mode, wl, wr, _stream_ptr(q.device))
    _raise("attn_decode", st)
    return out, lse
