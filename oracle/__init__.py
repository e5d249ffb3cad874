"""Plain, slow fp64 CPU oracle for exact attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything from this package.  The GPU path never calls
it and shares no code with it; the two meet only in the seeded input module
``workloads``.

Sources (cited as P1..P4 with their sections throughout this package):
  P1  ai6s.net/6af30f4d40858c2d8819b6d5.html -- FlashAttention's generic ideas
      (tiling, online softmax, recomputation, a CUDA teaching kernel) and its
      Ascend NPU implementation.
  P2  aicoding.csdn.net/6a69d3ff10ee7a33f2941f44.html -- FlashAttention in the
      Ascend ops-transformer library (memory table, block loop, pitfalls).
  P3  jsqmd.com/news/1148352 -- porting FlashAttention into a custom inference
      engine (online softmax state m, l, O_acc; porting constraints).
  P4  ai6s.net/6a0ed07b662f9a54cb761aa2.html -- FlashAttention under the catlass
      templates (epilogue mask variants: none / causal / sliding window).

Grouped-query heads and packed variable-length batches (P1 §5's
extensions) are in ``grouped.py``; decoding over a paged K/V cache in
``decode.py``.

Every public function here is pinned by ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force on tiny inputs and an independent
library routine (torch's CPU float64 scaled-dot-product attention and
autograd): the definitions (forward_head / forward_rows / forward,
backward_head, the grouped, packed and paged forms), the mask helpers
(allowed_matrix against brute-force loops and torch's tril/triu masks,
allowed_count against its per-mask closed forms) and the pages' online update.
"""
from .attention import (MASK_MODES, allowed_matrix, allowed_count, forward_head, forward_rows,
                        forward, backward_head)
from .decode import forward_decode, gather
from .grouped import (backward_gqa, backward_varlen, forward_gqa, forward_varlen, group_size)
from .online import online_forward_head

__all__ = ["MASK_MODES", "allowed_matrix", "allowed_count", "forward_head", "forward_rows",
           "forward", "backward_head", "online_forward_head", "group_size",
           "forward_gqa", "backward_gqa", "forward_varlen", "backward_varlen", "forward_decode",
           "gather"]
