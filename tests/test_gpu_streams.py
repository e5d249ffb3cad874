"""Calls on two streams at once share no state: the forward and backward of two
different problems, enqueued alternately on two streams (default priority) so
that their kernels may overlap on the GPU, give bitwise the results of the same
calls made one after the other on one stream.  (attn_fwd_persistent is not
among them: its work queues are per device, and two of its launches must not
overlap.)"""
import pytest
import torch

import exact_attention_14_amd as ea
from parity_util import gpu, say
from workloads import draw, draw_grouped

pytestmark = pytest.mark.gpu


def problems():
    a = draw(2, 8, 1500, 128, "bf16", 91, with_do=True)
    b = draw_grouped(1, 16, 4, 2300, 64, "f16", 92, with_do=True)
    return [({k: gpu(v) for k, v in a.items()}, "causal"),
            ({k: gpu(v) for k, v in b.items()}, (300, 20))]


def run(inp, mask):
    q, k, v, do = (inp[x] for x in ("q", "k", "v", "do"))
    o, lse = ea.attn_fwd(q, k, v, mask=mask)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, mask=mask)
    return o, lse, dq, dk, dv


def test_two_streams_match_serial_calls():
    probs = problems()
    serial = [run(inp, mask) for inp, mask in probs]
    torch.cuda.synchronize()
    say("two streams: 3 rounds of interleaved calls")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rnd in range(3):
        outs = [None, None]
        for rep in range(2):  # alternate enqueues so both streams hold work at once
            for i, st in enumerate((s1, s2)):
                with torch.cuda.stream(st):
                    outs[i] = run(*probs[i])
        torch.cuda.synchronize()
        for i in range(2):
            for name, a, b in zip(("O", "lse", "dQ", "dK", "dV"), outs[i], serial[i]):
                assert torch.equal(a, b), (rnd, i, name)
