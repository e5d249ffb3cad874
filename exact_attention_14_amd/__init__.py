"""MI355X-native exact attention: a C-ABI library of hand-written gfx950 kernels.

``attn_fwd`` / ``attn_bwd`` (with grouped-query K/V when K has fewer heads than
Q), ``attn_bwd_noalloc`` (the backward with a fixed per-GPU scratch, for
callers that cannot allocate) and ``attn_fwd_varlen`` / ``attn_bwd_varlen`` (packed variable-length
batches) and ``attn_decode`` (split-KV decoding over a paged cache) are thin ctypes wrappers over the C ABI declared in
``include/attn.h`` (library: ``libattn.so``, built by
``python -m exact_attention_14_amd.build``).
"""
from .binding import (AttnError, attn_bwd, attn_bwd_kv_workgroup, attn_bwd_noalloc, attn_bwd_varlen,
                      attn_decode, attn_decode_workspace_bytes,
                      attn_bwd_varlen_workspace_bytes, attn_bwd_workspace_bytes, attn_fwd,
                      attn_fwd_tiles, attn_fwd_varlen, attn_fwd_workgroup, attn_kv_tile_range,
                      attn_status_str, lib, mask_args)

__all__ = ["AttnError", "attn_fwd", "attn_bwd", "attn_bwd_noalloc", "attn_fwd_varlen", "attn_bwd_varlen",
           "attn_decode", "attn_decode_workspace_bytes",
           "attn_bwd_workspace_bytes", "attn_bwd_varlen_workspace_bytes", "attn_status_str", "attn_bwd_kv_workgroup",
           "attn_fwd_tiles", "attn_fwd_workgroup", "attn_kv_tile_range", "lib", "mask_args"]
