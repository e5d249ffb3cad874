"""The allocation-free backward (attn_bwd_noalloc) against attn_bwd.

Both run the same kernels, so the gradients must agree bit for bit; the
no-alloc call writes into caller-allocated outputs and its only workspace is
the library's fixed per-GPU scratch.  Two calls in a row, the second with a
smaller input, show that the scratch holds no state a later call depends on.
"""
import ctypes

import pytest
import torch

import exact_attention_14_amd as ea
from parity_util import gpu, say
from workloads import draw

pytestmark = pytest.mark.gpu

CASES = [  # (B, H, N, d, dtype, mask, seed): the second is smaller than the first
    (2, 4, 1000, 128, "bf16", "causal", 41),
    (1, 2, 300, 64, "f16", (40, 3), 42),
    (1, 1, 1, 128, "bf16", None, 43),
]


def c_abi_noalloc(q, k, v, o, lse, do, dq, dk, dv, mask, scale):
    """One call of attn_bwd_noalloc straight through the C ABI (ctypes)."""
    mode, wl, wr = ea.mask_args(mask)
    B, H, N, d = q.shape
    dt = 1 if q.dtype == torch.bfloat16 else 0
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ea.lib().attn_bwd_noalloc(dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                     dv.data_ptr(), B, H, N, d, float(scale), mode, wl, wr, stream)


def test_noalloc_backward_equals_attn_bwd_twice():
    for B, H, N, d, dtype, mask, seed in CASES:
        say(f"noalloc bwd B{B} H{H} N{N} d{d} {dtype} {mask}")
        scale = 1.0 / d ** 0.5
        inp = draw(B, H, N, d, dtype, seed, with_do=True)
        q, k, v, do = (gpu(inp[x]) for x in ("q", "k", "v", "do"))
        o, lse = ea.attn_fwd(q, k, v, mask=mask, scale=scale)
        ref = ea.attn_bwd(q, k, v, o, lse, do, mask=mask, scale=scale)
        # outputs pre-filled with garbage: every element must be written
        got = [torch.full_like(t, 7.0) for t in ref]
        torch.cuda.synchronize()
        st = c_abi_noalloc(q, k, v, o, lse, do, *got, mask, scale)
        assert st == 0, ea.attn_status_str(st)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, b), f"{name} differs from attn_bwd"


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """A call whose workspace would exceed the scratch fails before any launch
    and leaves its outputs untouched."""
    B, H, N, d = 1, 1, 4_200_000, 64
    need = ea.attn_bwd_workspace_bytes(torch.bfloat16, B, H, N, d)
    assert need > ea.binding.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(B, H, N, dtype=torch.float32, device="cuda")
    outs = [torch.full_like(t, 3.0) for _ in range(3)]
    ins = [torch.zeros_like(t) for _ in range(4)]
    st = c_abi_noalloc(ins[0], ins[1], ins[2], ins[3], lse, t, *outs, None, 0.125)
    torch.cuda.synchronize()
    assert st == 10, ea.attn_status_str(st)
    assert all(bool((x == 3.0).all()) for x in outs)
