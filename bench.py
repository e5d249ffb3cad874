"""Benchmark of the exact-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one attn_fwd call (attn_fwd_varlen for a packed workload) over the
whole batch of the workload (host plan,
Q load, K/V streaming, score products, masking, online softmax, output
products, epilogue: the whole forward path), with inputs already resident in
device memory.  The default workload is B=4, H=32, N=4096, d=128, bf16, no
mask.  Prints one JSON line with the throughput in TFLOP/s of algorithmic work
(4*d FLOP per allowed (query, key) pair), the roofline position of the forward
kernel (HIP events on the launch stream), and the fp64 CPU oracle timed on a
bounded sample of the same workload.  For the workload with an upstream
gradient (the fp16 causal forward + backward), the recomputation backward is
timed as well and reported in a "backward" object of the same line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import BY_NAME, FULL_N4096, make_inputs  # noqa: E402

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}  # MI355X dense matrix-core peak
HBM_PEAK_GBS = 8000.0


def allowed_pairs(N: int, mode: str, wl: int, wr: int) -> int:
    """Number of allowed (query, key) pairs of one head (closed form)."""
    if mode == "none":
        return N * N
    if mode == "causal":
        return N * (N + 1) // 2
    wl, wr = min(wl, N), min(wr, N)
    total = 0
    # row i: min(i, wl) + 1 + min(N - 1 - i, wr)
    for i in range(N):
        total += min(i, wl) + 1 + min(N - 1 - i, wr)
    return total


def pairs_per_head(w) -> int:
    """Allowed (query, key) pairs of one query head over all its sequences."""
    return sum(allowed_pairs(n, w.mask, w.window_left, w.window_right) for n in w.lengths)


def fwd_flops(w) -> int:
    return 4 * w.d * w.H * pairs_per_head(w)


def mask_arg(w):
    if w.mask == "none":
        return None
    if w.mask == "causal":
        return "causal"
    return (w.window_left, w.window_right)


def oracle_units(w, inp):
    """(label, q, k, v) float64 arrays of one query head of one sequence each, in order:
    the head's own Q rows and its key/value head's K, V rows."""
    from workloads import to_f64
    g = w.H // w.kv_heads
    if w.packed:
        cu = inp["cu_seqlens"].numpy()
        for s_ in range(len(cu) - 1):
            lo, hi = int(cu[s_]), int(cu[s_ + 1])
            for h in range(w.H):
                yield ((s_, h),) + tuple(to_f64(inp[x][i, lo:hi])
                                         for x, i in (("q", h), ("k", h // g), ("v", h // g)))
    else:
        for b in range(w.B):
            for h in range(w.H):
                yield ((b, h),) + tuple(to_f64(inp[x][b, i])
                                        for x, i in (("q", h), ("k", h // g), ("v", h // g)))


def cpu_baseline(w, inp, budget_s: float = 12.0, max_units: int = 128):
    """The fp64 oracle as it stands, on whole heads (whole sequences of one head for a
    packed batch) of the workload, until ~budget_s."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    done, pairs = 0, 0
    t0 = time.perf_counter()
    for _, q, k, v in oracle_units(w, inp):
        n = q.shape[0]
        rb = 1024 if n > 8192 else n
        for r0 in range(0, n, rb):
            rows = np.arange(r0, min(n, r0 + rb))
            oracle.forward_rows(rows, q, k, v, w.scale, w.mask, w.window_left, w.window_right)
        pairs += allowed_pairs(n, w.mask, w.window_left, w.window_right)
        done += 1
        if done >= max_units or time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4 * w.d * pairs
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    unit = "sequence-heads" if w.packed else "heads"
    total = w.H * len(w.lengths)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {total} {unit}, all their rows (fp64 numpy, S and P "
                      f"materialised per head), {dt:.1f} s"}


def decode_bytes(w) -> int:
    """Algorithmic HBM bytes of one decode call: every cached K and V row of every
    key/value head once, Q and O once, lse once."""
    rows = sum(w.lengths)
    kv = 2 * rows * w.kv_heads * w.d * 2
    q_o = 2 * w.B * w.H * w.decode_q * w.d * 2
    return kv + q_o + w.B * w.H * w.decode_q * 4


def bench_decode(w, args, inp):
    """Timed attn_decode calls; one JSON line with GB/s against the HBM peak."""
    import numpy as np
    import torch

    import exact_attention_14_amd as ea

    q, k, v, bt, sl = (inp[x].to("cuda") for x in ("q", "k", "v", "block_table", "seq_lens"))
    o = torch.empty_like(q)
    lse = torch.empty(tuple(q.shape[:-1]), dtype=torch.float32, device="cuda")
    need = ea.attn_decode_workspace_bytes(q.dtype, w.B, w.H, w.kv_heads, w.decode_q, w.d, w.N)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    mask = mask_arg(w)

    def step():
        ea.attn_decode(q, k, v, bt, sl, w.N, mask=mask, scale=w.scale, out=o, lse=lse,
                       workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ta = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_wall = (time.perf_counter() - ta) * 1e3 / args.steps
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_kernel = evs[0].elapsed_time(evs[-1]) / args.steps
    nbytes = decode_bytes(w)
    value = nbytes / (ms_wall * 1e-3) / 1e9
    achieved = nbytes / (ms_kernel * 1e-3) / 1e9
    rec = {
        "metric": f"attention decode GB/s of K/V cache read ({w.name})",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_wall, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded i.i.d. N(0,1) queries and cache, pages dealt to a random "
                "permutation of the pool)",
        "config": {"workload": w.name, "n_seqs": w.B, "H": w.H, "H_kv": w.kv_heads,
                   "n_q": w.decode_q, "cache_len": w.N, "d": w.d, "page_size": w.page_size,
                   "mask": w.mask, "global_batch": w.B, "seq_len": w.N, "parallelism": "none"},
        "tokens_per_s": round(w.B * w.decode_q / (ms_wall * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_kernel" + (" + decode_combine_kernel" if need > 0 else ""),
                     "kernel_ms": round(ms_kernel, 5),
                     "kernel_ms_per_call": {f"p{p}": round(per[min(len(per) - 1,
                                                                   len(per) * p // 100)], 5)
                                            for p in (10, 50, 90)},
                     "bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        import oracle
        from workloads import to_f64
        budget, done, t0 = 12.0, 0, time.perf_counter()
        table, lens = inp["block_table"], inp["seq_lens"].numpy()
        while done < w.B and time.perf_counter() - t0 < budget:
            # the sequence's own pages, renumbered 0.., widened to fp64
            pages = table[done].long()
            sub = np.arange(len(pages), dtype=np.int64)[None]
            oracle.forward_decode(to_f64(inp["q"][done:done + 1]), to_f64(inp["k"][pages]),
                                  to_f64(inp["v"][pages]), sub, lens[done:done + 1], w.scale,
                                  w.mask)
            done += 1
        dt = time.perf_counter() - t0
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        rec["cpu_baseline"] = {"value": round(nbytes * done / w.B / dt / 1e9, 4), "unit": "GB/s",
                               "cores": int(threads), "kind": "oracle",
                               "sample": f"{done} of {w.B} sequences, all heads (fp64 numpy), "
                                         f"{dt:.1f} s"}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The chip takes tens of milliseconds to settle at its power-limited clock
    # after idling; 100 warm-up calls (~0.1 s at the headline shape) get there.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=FULL_N4096.name, choices=sorted(BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--persistent", action="store_true",
                    help="time attn_fwd_persistent (fixed-length workloads) instead of attn_fwd")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the forward shards by head with no exchange, "
              "so the one-GPU figure is the per-GPU figure", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_14_amd as ea

    w = BY_NAME[args.workload]
    inp = make_inputs(w)
    if w.decode_q > 0:
        bench_decode(w, args, inp)
        return
    q, k, v = (inp[x].to("cuda") for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(tuple(q.shape[:-1]), dtype=torch.float32, device="cuda")
    mask = mask_arg(w)
    if w.packed:
        cu = inp["cu_seqlens"].to("cuda")
        max_len = max(w.lengths)

    def step():
        if w.packed:
            ea.attn_fwd_varlen(q, k, v, cu, max_len, mask=mask, scale=w.scale, out=o, lse=lse)
        else:
            ea.attn_fwd(q, k, v, mask=mask, scale=w.scale, out=o, lse=lse,
                        persistent=args.persistent)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def timed(fn):
        """Wall time of args.steps calls (host clock, synchronised on both sides)
        and the calls' GPU times from events recorded between them on the
        launch stream: (wall ms per call, mean GPU ms per call, percentiles)."""
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        ta = time.perf_counter()
        evs[0].record(stream)
        for i in range(args.steps):
            fn()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        tb = time.perf_counter()
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
        pct = {f"p{q}": round(per[min(len(per) - 1, (len(per) * q) // 100)], 5)
               for q in (10, 50, 90)}
        return (tb - ta) * 1e3 / args.steps, evs[0].elapsed_time(evs[-1]) / args.steps, pct

    ms_wall, ms_kernel, per_call = timed(step)
    flops = fwd_flops(w)
    value = flops / (ms_wall * 1e-3) / 1e12
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]

    # The recomputation backward, for workloads that carry an upstream
    # gradient: timed the same way, from the O and lse of the forward above.
    backward = None
    if w.backward:
        do = inp["do"].to("cuda")
        if w.packed:
            need = ea.attn_bwd_varlen_workspace_bytes(q.dtype, len(w.lengths), max_len, w.N, w.H,
                                                      w.kv_heads, w.d)
        else:
            need = ea.attn_bwd_workspace_bytes(q.dtype, w.B, w.H, w.N, w.d, w.kv_heads)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

        def bstep():
            if w.packed:
                ea.attn_bwd_varlen(q, k, v, o, lse, do, cu, max_len, mask=mask, scale=w.scale,
                                   workspace=ws)
            else:
                ea.attn_bwd(q, k, v, o, lse, do, mask=mask, scale=w.scale, workspace=ws)

        for _ in range(args.warmup):
            bstep()
        b_wall, b_ms, b_pct = timed(bstep)
        bflops = 10 * w.d * w.H * pairs_per_head(w)
        backward = {"ms_per_call": round(b_wall, 5),
                    "kernel_ms": round(b_ms, 5),
                    "kernel_ms_per_call": b_pct,
                    "tflops": round(bflops / (b_ms * 1e-3) / 1e12, 3),
                    "frac_of_peak": round(bflops / (b_ms * 1e-3) / 1e12 / PEAK_TFLOPS[w.dtype], 4),
                    "flop_per_call": bflops,
                    "flop_model": "10*d per allowed pair (S, dP, dV, dK, dQ products)"}
        del do, ws

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # HBM bytes per launch from the committed counter runs, while the kernel
    # they measured is unchanged (see exact_attention_14_amd/profiles.py).
    from exact_attention_14_amd.profiles import kernel_source_sha

    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha") == kernel_source_sha():
            traffic = round(tr.get("bytes_per_launch"))

    if w is FULL_N4096:
        metric = "attention fwd TFLOP/s (and % of bf16 MFMA peak) at B4 H32 N4096 d128"
    else:
        metric = f"attention fwd TFLOP/s ({w.name})"
    config = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "mask": w.mask,
              "window_left": w.window_left, "window_right": w.window_right,
              "scale": w.scale, "global_batch": w.B, "seq_len": w.N, "parallelism": "none"}
    if w.kv_heads != w.H:
        config["H_kv"] = w.kv_heads
    if w.packed:
        config.update({"packed_rows": w.N, "n_seqs": len(w.lengths), "max_seqlen": max(w.lengths),
                       "lengths": f"log-uniform in [{w.packed_lo}, {w.packed_hi}], "
                                  f"seed {w.packed_seed}"})
    rec = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded i.i.d. N(0,1) inputs of the workload's shape)",
        "config": config,
        "tokens_per_s": round(w.B * w.N / (ms_wall * 1e-3), 1),
        "frac_of_peak": round(value / peak, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": "fwd_kernel", "kernel_ms": round(ms_kernel, 5),
                     "kernel_ms_per_call": per_call,
                     "flop_per_launch": flops},
    }
    if backward is not None:
        rec["backward"] = backward
    if args.persistent:
        rec["entry_point"] = "attn_fwd_persistent"
    if os.environ.get("EXACT_ATTN_LIB"):
        rec["library"] = os.environ["EXACT_ATTN_LIB"]
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
