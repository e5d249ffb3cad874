"""Summaries of rocprofv3 output for the committed profiles/ folder.

    python -m exact_attention_14_amd.profiles stats  <kernel_stats.csv> <out.md> <command...>
    python -m exact_attention_14_amd.profiles traffic <fetch_dir> <write_dir> <workload> <copy_mib> <out.json> <out.md> <commands...>
    python -m exact_attention_14_amd.profiles counters [--clock-ghz=F] <counter_dir> <kernel_stats.csv> <out.md> <command...>
    python -m exact_attention_14_amd.profiles sweep [--rows=NAME] <out.md> <title> <commands> <label:flop:dir[:kernel]>...

``stats`` turns the ``*_kernel_stats.csv`` of ``rocprofv3 --kernel-trace --stats
--output-format csv`` into a short markdown table.  ``traffic`` reads two
``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of ``bench.py
--copy-calibration-mib M`` and scales the forward kernel's per-dispatch
counters by what the same counters read for the calibration copy of M MiB
(a device-to-device copy reads and writes exactly M MiB), giving HBM bytes
per launch.  The JSON records a hash of the forward kernel's sources so that
bench.py reports the traffic only while the kernel is unchanged.  ``counters``
summarises one ``--pmc`` pass (per-dispatch means of every attention kernel
in it): matrix-core busy cycles per SIMD and, given the shader clock read
with amd-smi under the same load, the busy fraction.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FWD_SOURCES = ("fwd_kernel.hip", "device_common.hpp", "plan.hpp")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for name in FWD_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_14_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_BOOL_NAMES = {"fwd_kernel": ("pair", "persistent"), "bwd_dq_kernel": ("pair",)}
_MASK_NAMES = ("none", "causal", "sliding")


def _demangle_short(name: str) -> str:
    """kernel<type,d,mask,flags> from an Itanium-mangled kernel name."""
    import re
    for key in ("fwd_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_kv_reduce_kernel",
                "decode_combine_kernel", "decode_kernel"):
        if key in name:
            tail = name.split(key, 1)[1]
            args = []
            ints = 0
            bools = []
            for m in re.finditer(r"DF16b|DF16_|Li(\d+)E|Lb([01])E", tail.split("EEvNS")[0]):
                t = m.group(0)
                if t == "DF16b":
                    args.append("bf16")
                elif t == "DF16_":
                    args.append("f16")
                elif m.group(1) is not None:
                    ints += 1
                    v = int(m.group(1))
                    # the second integer of the attention kernels is the mask mode
                    args.append(_MASK_NAMES[v] if ints == 2 and key != "decode_combine_kernel"
                                and v < 3 else str(v))
                else:
                    bools.append(m.group(2) == "1")
            names = _BOOL_NAMES.get(key, ())
            args += [n for n, b in zip(names, bools) if b]
            return f"{key}<{','.join(args)}>"
    return name[:60]


def stats(csv_path: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    lines = ["# rocprofv3 kernel statistics", "", f"Command: `{command}`", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {_demangle_short(r['Name'])} | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))


def _counter(dirname: str, counter: str):
    """(attn forward values, copy values) per dispatch, in the counter's unit (KiB)."""
    fwd, copy = [], []
    for path in glob.glob(os.path.join(dirname, "*counter_collection.csv")):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if "fwd_kernel" in r["Kernel_Name"]:
                fwd.append(v)
            elif "copybuffer" in r["Kernel_Name"].lower():
                copy.append((v, r["Kernel_Name"]))
    return fwd, copy


def traffic(fetch_dir: str, write_dir: str, workload: str, copy_mib: int, out_json: str,
            out_md: str, commands: str = "") -> None:
    copy_bytes = copy_mib * (1 << 20)
    out = {"workload": workload, "kernel_source_sha": kernel_source_sha(), "copy_mib": copy_mib}
    lines = ["# HBM traffic of the forward kernel (rocprofv3 PMC)", "",
             f"Workload: `{workload}`.  Counters in KiB per dispatch, scaled by the same counter",
             f"read for a device copy of {copy_mib} MiB (reads and writes exactly that).", ""]
    if commands:
        lines += [f"Commands: {commands}", ""]
    total = 0.0
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        fwd, copy = _counter(d, counter)
        if not fwd or not copy:
            raise SystemExit(f"missing {counter} values in {d}")
        copy_val = max(v for v, _ in copy)
        factor = copy_bytes / (copy_val * 1024.0)
        per_launch = sum(fwd) / len(fwd) * 1024.0 * factor
        out[counter] = {"fwd_kib_mean": sum(fwd) / len(fwd), "copy_kib": copy_val,
                        "scale": factor, "bytes_per_launch": per_launch}
        total += per_launch
        lines.append(f"- {counter}: forward {sum(fwd) / len(fwd):.0f} KiB/dispatch (mean of "
                     f"{len(fwd)}), copy {copy_val:.0f} KiB -> scale {factor:.4f} -> "
                     f"{per_launch / 1e6:.1f} MB per launch")
    out["bytes_per_launch"] = total
    lines += ["", f"Total HBM traffic per launch: {total / 1e6:.1f} MB.", ""]
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    with open(out_md, "w") as f:
        f.write("\n".join(lines))


def counters(counter_dir: str, kernel_stats: str, out_md: str, command: str,
             clock_ghz: float = 0.0) -> None:
    keys = ("fwd_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel")
    per = {}  # kernel -> counter -> dispatch -> value
    for path in glob.glob(os.path.join(counter_dir, "*counter_collection.csv")):
        for r in csv.DictReader(open(path)):
            key = next((k for k in keys if k in r["Kernel_Name"]), None)
            if key is None:
                continue
            d = per.setdefault(key, {}).setdefault(r["Counter_Name"], {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    durations = {}
    for r in csv.DictReader(open(kernel_stats)):
        key = next((k for k in keys if k in r["Name"]), None)
        if key is not None:
            durations[key] = float(r["AverageNs"])
    lines = ["# Kernel counters (rocprofv3 PMC)", "", f"Command: `{command}`", "",
             "Means per dispatch; durations are the averages from the kernel trace of the same",
             "workload.  SQ_VALU_MFMA_BUSY_CYCLES is summed over the 1024 SIMDs.  GRBM_GUI_ACTIVE",
             "does not count shader-clock cycles (divided by the duration it gives neither the",
             "clock amd-smi reports nor a constant multiple of it), so no clock is derived from it.",
             ""]
    for key in keys:
        if key not in per:
            continue
        mean = {k: sum(v.values()) / len(v) for k, v in per[key].items()}
        lines += [f"## {key}", ""]
        if key in durations:
            lines += [f"Kernel duration: {durations[key] / 1e3:.1f} us", ""]
        lines += ["| counter | mean per dispatch |", "|---|---|"]
        lines += [f"| {k} | {v:.4g} |" for k, v in sorted(mean.items())]
        if mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) > 0 and key in durations:
            busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024
            lines += ["", f"- matrix-core busy cycles per SIMD: {busy:.4g}"]
            if mean.get("SQ_INSTS_MFMA", 0) > 0:
                lines.append(f"- matrix instructions per SIMD: {mean['SQ_INSTS_MFMA'] / 1024:.4g} "
                             f"({busy / (mean['SQ_INSTS_MFMA'] / 1024):.1f} busy cycles each)")
            if clock_ghz:
                lines.append(f"- busy fraction at the {clock_ghz:.2f} GHz shader clock amd-smi "
                             f"reports under this load: {busy / (durations[key] * clock_ghz):.1%}")
        lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))


def _pmc_means(dirname: str, key: str = "fwd_kernel"):
    """Counter -> mean per dispatch of kernel `key` over every pass CSV under dirname."""
    per = {}
    for path in glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if key not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Counter_Name"], {})
            d[(path, r["Dispatch_Id"])] = d.get((path, r["Dispatch_Id"]), 0.0) + float(
                r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def _trace_us(dirname: str, key: str = "fwd_kernel") -> float:
    for path in glob.glob(os.path.join(dirname, "**", "*kernel_stats.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if key in r["Name"]:
                return float(r["AverageNs"]) / 1e3
    raise SystemExit(f"no {key} in the kernel statistics under {dirname}")


def sweep(out_md: str, title: str, commands: str, entries, first: str = "variant") -> None:
    """One table row per `label:flop_per_launch:dir[:kernel]`, where dir holds the
    kernel trace and the counter passes of one bench run and kernel (default
    fwd_kernel) names the kernel of the row."""
    rows = []
    for e in entries:
        label, flop, d, *key = e.split(":")
        key = key[0] if key else "fwd_kernel"
        us = _trace_us(d, key)
        m = _pmc_means(d, key)
        mfma = m.get("SQ_INSTS_MFMA", float("nan"))
        busy = m.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / 1024  # per SIMD
        wave_cyc = m.get("SQ_WAVE_CYCLES", float("nan"))
        hit, miss = m.get("TCC_HIT_sum", float("nan")), m.get("TCC_MISS_sum", float("nan"))
        rows.append([
            label, f"{us:.1f}", f"{float(flop) / (us * 1e-6) / 1e12:.0f}",
            f"{busy / us:.0f}",
            f"{m.get('SQ_INSTS_VALU', float('nan')) / mfma:.2f}",
            f"{m.get('SQ_INSTS_VALU_TRANS_F32', float('nan')) / mfma:.2f}",
            f"{m.get('SQ_INSTS_LDS', float('nan')) / mfma:.2f}",
            f"{m.get('SQ_LDS_BANK_CONFLICT', float('nan')):.3g}",
            f"{m.get('SQ_WAIT_INST_ANY', float('nan')) / wave_cyc:.0%}",
            f"{m.get('SQ_WAIT_ANY', float('nan')) / wave_cyc:.0%}",
            f"{m.get('SQ_ACTIVE_INST_ANY', float('nan')) / wave_cyc:.0%}",
            f"{m.get('SQ_VALU_MFMA_COEXEC_CYCLES', float('nan')) / max(busy * 1024, 1):.0%}",
            f"{hit / (hit + miss):.1%}",
        ])
    hdr = [first, "kernel us", "TFLOP/s", "MFMA busy cycles per SIMD per us",
           "VALU / MFMA instr", "exp2 / MFMA", "LDS / MFMA instr", "LDS bank conflict cycles",
           "ready, not issued (of wave cycles)", "waiting", "issuing", "VALU co-issued "
           "beside busy MFMA (of MFMA busy)", "L2 hit rate"]
    lines = [f"# {title}", "", "Commands:", "", commands, "",
             "Kernel time: average of the rocprofv3 kernel trace; counters: means per dispatch of "
             "separate `--pmc` passes of the same workload.  MFMA busy cycles per SIMD per us is the "
             "busy fraction times the shader clock in MHz (no clock counter is read; at the "
             "~2.0 GHz this load settles at, 1000 = 50%).  The wave-cycle fractions divide "
             "SQ_WAIT_INST_ANY (ready but not issued), SQ_WAIT_ANY (waiting on a dependency, "
             "s_waitcnt or a barrier) and SQ_ACTIVE_INST_ANY (issuing) by SQ_WAVE_CYCLES, all in "
             "the same units.",
             "", "| " + " | ".join(hdr) + " |", "|" + "---|" * len(hdr)]
    lines += ["| " + " | ".join(r) + " |" for r in rows]
    lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif sys.argv[1] == "counters":
        args = sys.argv[2:]
        clk = 0.0
        if args and args[0].startswith("--clock-ghz="):
            clk = float(args[0].split("=", 1)[1])
            args = args[1:]
        counters(args[0], args[1], args[2], " ".join(args[3:]), clk)
    elif sys.argv[1] == "sweep":
        args = sys.argv[2:]
        first = "variant"
        if args and args[0].startswith("--rows="):
            first = args[0].split("=", 1)[1]
            args = args[1:]
        sweep(args[0], args[1], args[2], args[3:], first)
    elif sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]), sys.argv[6], sys.argv[7],
                " ".join(sys.argv[8:]))
    else:
        raise SystemExit(__doc__)
