"""Turn rocprofv3 CSV output of bench.py into the short text summaries kept
under profiles/.

    # kernel-time table from a --kernel-trace --stats run
    python -m invariant_bi_rmsnorm_amd.profile_summary stats DIR OUT.md --cmd "..." --title "..."

    # HBM traffic per launch from a FETCH_SIZE run and a WRITE_SIZE run
    python -m invariant_bi_rmsnorm_amd.profile_summary traffic FETCH_DIR WRITE_DIR OUT.md OUT.json \
        --cmd-fetch "..." --cmd-write "..."

    # MFMA utilisation (MfmaUtil, MfmaFlopsBF16) next to kernel durations
    python -m invariant_bi_rmsnorm_amd.profile_summary mfma DIR TRACE_DIR OUT.md --cmd "..."

    # any other counters (per kernel, per dispatch averages)
    python -m invariant_bi_rmsnorm_amd.profile_summary counters DIR OUT.md --cmd "..." --title "..."

FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.  What they count per
byte moved is calibrated on the copy probe (bi_probe_copy), which bench.py
runs once on COPY_PROBE_BYTES of source: the probe reads and writes exactly
that many bytes, so bytes = counter * (probe bytes / probe counter).
"""
from __future__ import annotations

import argparse
import csv
import re
import glob
import hashlib
import json
import os
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "invariant_bi_rmsnorm_amd", "csrc")
COPY_PROBE_BYTES = 512 << 20
GEMM_SOURCES = ("gemm.hip", "gemm_tiles.hpp", "gemm_kernel.hpp", "bi_common.hpp")
HIDDEN = 4096
GEMM_N = (4096, 14336)
M_SWEEP = list(range(1, 65)) + [128, 256, 512, 1024, 2048]

KERNELS = ("gemm_kernel", "rmsnorm_kernel", "decode_split_kernel", "decode_combine_kernel",
           "decode_ticket_reset", "prefill_kernel", "kv_append_kernel", "copy_kernel", "log_softmax_kernel",
           "nb_splitk_reduce", "read_kernel", "lds_fill_kernel")


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one(pattern, d):
    found = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not found:
        raise SystemExit(f"no {pattern} under {d}")
    return found[0]


def short(name: str) -> str:
    # the GEMM template: libbi.so's tiles (tag 0) vs the baseline library's tiles (tag 1)
    if "gemm_kernel<" in name:
        m = re.search(r"GemmTile<\d+, \d+, \d+, \d+, \d+, \d+, (\d+)(?:, \d+)?>", name)
        return "gemm_kernel" if m and m.group(1) == "0" else "gemm_kernel (baseline lib)"
    # the prefill template: splits from position 0 (libbi.so) or from each
    # chunk's start (the baseline library)
    if "prefill_kernel<true>" in name:
        return "prefill_kernel (baseline lib)"
    for k in KERNELS:
        if re.search(rf"(^|[ :]){k}($|[<( ])", name):
            return k
    return name if len(name) <= 60 else name[:57] + "..."


def trace_durations(d):
    """{kernel: [duration in microseconds per dispatch]} from the per-dispatch
    kernel trace of a --kernel-trace run, kernels named by short()."""
    out = defaultdict(list)
    for r in csv.DictReader(open(_one("*kernel_trace.csv", d))):
        out[short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return out


def stats_md(d, out, cmd, title):
    dur = trace_durations(d)
    total = sum(sum(v) for v in dur.values())
    lines = [f"# {title}", "", "Command (from the repository root, one MI355X):", "", "```", cmd, "```", "",
             "Kernel durations from rocprofv3's per-dispatch kernel trace (microseconds), per kernel "
             "instantiation: `gemm_kernel` is libbi.so's GEMM tiles, `gemm_kernel (baseline lib)` the "
             "non-invariant library's tiles.", "",
             "| kernel | calls | total us | avg us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for k, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {k} | {len(v)} | {sum(v):.1f} | {sum(v) / len(v):.2f} | {min(v):.2f} | "
                     f"{max(v):.2f} | {100 * sum(v) / total:.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_counters(d):
    """{kernel: {counter: [value per dispatch, in dispatch order]}}"""
    per = defaultdict(lambda: defaultdict(float))          # (dispatch, kernel) -> counter -> value
    for r in csv.DictReader(open(_one("*counter_collection.csv", d))):
        key = (int(r["Dispatch_Id"]), short(r["Kernel_Name"]))
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
    out = defaultdict(lambda: defaultdict(list))
    for (disp, k), cs in sorted(per.items()):
        for c, v in cs.items():
            out[k][c].append(v)
    return out


def avg_durations_us(trace_dir):
    """{kernel: average duration in microseconds} from a --kernel-trace run"""
    return {k: sum(v) / len(v) for k, v in trace_durations(trace_dir).items() if k in KERNELS}


def traffic(fetch_dir, write_dir, out_md, out_json, cmd_fetch, cmd_write, trace_dir=None):
    fe = read_counters(fetch_dir)
    wr = read_counters(write_dir)
    cf = fe["copy_kernel"]["FETCH_SIZE"]
    cw = wr["copy_kernel"]["WRITE_SIZE"]
    if not cf or not cw:
        raise SystemExit("no copy_kernel dispatch in the counter runs: cannot calibrate")
    # the first probe launch, before the timed repeats
    f_fetch = COPY_PROBE_BYTES / (cf[0] * 1024.0)
    f_write = COPY_PROBE_BYTES / (cw[0] * 1024.0)
    lines = [f"# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE), bench.py phases", "",
             "Commands (from the repository root, one MI355X; one counter per run):", "", "```",
             cmd_fetch, cmd_write, "```", "",
             f"Calibration on the copy probe ({COPY_PROBE_BYTES >> 20} MiB read + written): "
             f"FETCH_SIZE read {cf[0]:.0f} KiB, WRITE_SIZE {cw[0]:.0f} KiB; "
             f"bytes = KiB x 1024 x {f_fetch:.4f} (fetch), x {f_write:.4f} (write).", "",
             "| kernel | dispatches | fetch MB/launch | write MB/launch | traffic MB/launch | avg us | HBM GB/s |",
             "|---|---|---|---|---|---|---|"]
    dur = avg_durations_us(trace_dir) if trace_dir else {}
    summary = {}
    for k in KERNELS:
        a, b = fe.get(k, {}).get("FETCH_SIZE", []), wr.get(k, {}).get("WRITE_SIZE", [])
        if not a or not b:
            continue
        fm = sum(a) / len(a) * 1024 * f_fetch
        wm = sum(b) / len(b) * 1024 * f_write
        summary[k] = {"dispatches": len(a), "fetch_bytes": fm, "write_bytes": wm, "traffic_bytes": fm + wm}
        us = dur.get(k)
        rate = f"{(fm + wm) / (us * 1e-6) / 1e9:.0f}" if us else ""
        lines.append(f"| {k} | {len(a)} | {fm / 1e6:.2f} | {wm / 1e6:.2f} | {(fm + wm) / 1e6:.2f} | "
                     f"{us if us is None else round(us, 2)} | {rate} |")
    g = summary.get("gemm_kernel")
    doc = {"source_hash": src_hash(*GEMM_SOURCES), "kernels": summary,
           "calibration": {"fetch_factor": f_fetch, "write_factor": f_write}}
    if g:
        # the sweep repeats in a fixed order: (M, N) of dispatch i is order[i % len(order)]
        order = [(M, N) for M in M_SWEEP for N in GEMM_N]
        alg = sum(2 * (M * HIDDEN + N * HIDDEN + M * N) for (M, N) in order) / len(order)
        doc["traffic_bytes_per_launch"] = g["traffic_bytes"]
        doc["algorithmic_bytes_per_launch"] = alg
        lines += ["", f"bi_matmul over the projection sweep: {g['traffic_bytes'] / 1e6:.2f} MB per launch "
                      f"measured vs {alg / 1e6:.2f} MB algorithmic (A + W + C once), "
                      f"ratio {g['traffic_bytes'] / alg:.3f}.", ""]
        fa = fe["gemm_kernel"]["FETCH_SIZE"]
        wa = wr["gemm_kernel"]["WRITE_SIZE"]
        if len(fa) % len(order) == 0 and len(wa) == len(fa):
            lines += ["Per shape (mean over sweeps):", "",
                      "| M | N | measured MB | algorithmic MB | ratio |", "|---|---|---|---|---|"]
            reps = len(fa) // len(order)
            for i, (M, N) in enumerate(order):
                if M not in (1, 8, 16, 32, 64, 128, 256, 512, 1024, 2048):
                    continue
                meas = sum(fa[i + r * len(order)] * f_fetch + wa[i + r * len(order)] * f_write
                           for r in range(reps)) * 1024 / reps
                a_ = 2 * (M * HIDDEN + N * HIDDEN + M * N)
                lines.append(f"| {M} | {N} | {meas / 1e6:.2f} | {a_ / 1e6:.2f} | {meas / a_:.3f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(out_json, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


def mfma_md(d, trace_dir, out, cmd):
    cs = read_counters(d)
    dur = avg_durations_us(trace_dir)
    lines = ["# MFMA utilisation per kernel (rocprofv3 MfmaUtil, MfmaFlopsBF16), bench.py phases", "",
             "Command (from the repository root, one MI355X):", "", "```", cmd, "```", "",
             "MfmaUtil = busy cycles of the MFMA units / (GPU active cycles x SIMDs), in percent, "
             "mean over dispatches.  MFMA TFLOP/s = counted bf16 MFMA flops per dispatch / the kernel's "
             "average duration from the kernel trace of the same workload.", "",
             "| kernel | dispatches | MfmaUtil % | MFMA GFLOP/dispatch | avg us | MFMA TFLOP/s |",
             "|---|---|---|---|---|---|"]
    for k in KERNELS:
        if k not in cs or "MfmaUtil" not in cs[k]:
            continue
        u = cs[k]["MfmaUtil"]
        f = cs[k].get("MfmaFlopsBF16", [])
        fl = sum(f) / len(f) if f else 0.0
        us = dur.get(k)
        tf = f"{fl / (us * 1e-6) / 1e12:.1f}" if us and fl else ""
        lines.append(f"| {k} | {len(u)} | {sum(u) / len(u):.1f} | {fl / 1e9:.3f} | "
                     f"{'' if us is None else round(us, 2)} | {tf} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def counters_md(d, out, cmd, title):
    cs = read_counters(d)
    names = sorted({c for k in cs for c in cs[k]})
    lines = [f"# {title}", "", "Command (from the repository root, one MI355X):", "", "```", cmd, "```", "",
             "Mean per dispatch:", "", "| kernel | dispatches | " + " | ".join(names) + " |",
             "|---|---|" + "---|" * len(names)]
    for k in sorted(cs):
        n = max(len(v) for v in cs[k].values())
        vals = [f"{sum(cs[k][c]) / len(cs[k][c]):.4g}" if cs[k].get(c) else "" for c in names]
        lines.append(f"| {k} | {n} | " + " | ".join(vals) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir"), s.add_argument("out"), s.add_argument("--cmd", required=True)
    s.add_argument("--title", required=True)
    t = sub.add_parser("traffic")
    for a in ("fetch_dir", "write_dir", "out_md", "out_json"):
        t.add_argument(a)
    t.add_argument("--cmd-fetch", required=True), t.add_argument("--cmd-write", required=True)
    t.add_argument("--trace-dir")
    mf = sub.add_parser("mfma")
    mf.add_argument("dir"), mf.add_argument("trace_dir"), mf.add_argument("out")
    mf.add_argument("--cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir"), c.add_argument("out"), c.add_argument("--cmd", required=True)
    c.add_argument("--title", required=True)
    a = ap.parse_args()
    if a.what == "stats":
        stats_md(a.dir, a.out, a.cmd, a.title)
    elif a.what == "traffic":
        traffic(a.fetch_dir, a.write_dir, a.out_md, a.out_json, a.cmd_fetch, a.cmd_write, a.trace_dir)
    elif a.what == "mfma":
        mfma_md(a.dir, a.trace_dir, a.out, a.cmd)
    else:
        counters_md(a.dir, a.out, a.cmd, a.title)


if __name__ == "__main__":
    main()
