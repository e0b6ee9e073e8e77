#!/usr/bin/env python3
"""Benchmark of the batch-invariant forward path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  1. projections (Llama-8B shapes): for every M in 1..64,128,256,...,2048:
     RMSNorm [M,4096] -> bi_matmul [M,4096]x[4096,4096] -> bi_matmul
     [M,4096]x[4096,14336]   (each N cycles through its own weight copies,
     more than 512 MB of them per N: 16 x 33.5 MB and 5 x 117 MB, so a copy is
     read again only after more than 256 MB, the last-level cache, of other
     copies of the same shape: weight reads come from HBM, whatever the cache
     policy of the other shape's loads);
  2. paged decode at 256 sequences, KV lengths log-uniform in [1, 32768]
     (32/8 heads, head dim 128): bi_kv_append of the step's token + decode;
  3. causal prefill of one 8192-token prompt.

`value` (the headline) is the invariant GEMM throughput of phase 1: GEMM
flops / wall time of phase 1 (HIP events bracketing the phase on the stream
the kernels run on).  Decode GB/s and prefill TFLOP/s are reported beside it.
The roofline entry is for the dominant kernel (bi_matmul), against the bound
of the whole sweep: its algorithmic intensity (sum of 2MNK over sum of
2(MK + NK + MN)) is below the MFMA/HBM ridge, so `achieved` is algorithmic
bytes per launch over the average launch duration, against HBM; the MFMA view
(flops per launch over the same duration) and the fraction of each shape's own
min(MFMA, HBM) roofline are reported beside it.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "invariant GEMM TFLOP/s + decode-attn HBM GB/s (% roofline), M=1..2048"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
COLD_BYTES = 512 * 10**6        # copies of one weight shape exceed this (twice the last-level cache)
PER_SHAPE_LAUNCHES = 5          # launches per shape in the per-shape timing graphs (the rotation goes on)


def weight_copies(nbytes: int) -> int:
    """How many copies of a weight of nbytes the sweep rotates through: at least
    3, and more than COLD_BYTES in all."""
    return max(3, COLD_BYTES // nbytes + 1)


class WeightRotation:
    """Which copy of an N x K weight each GEMM launch reads: one counter per N,
    so every N cycles through all of its copies whatever the launch order.
    copies maps N to its number of copies."""

    def __init__(self, copies: dict):
        self.copies = dict(copies)
        self.count = {}

    def next(self, N: int) -> int:
        k = self.count.get(N, 0)
        self.count[N] = k + 1
        return k % self.copies[N]


def sweep_schedule(m_sweep, ns, rot: WeightRotation):
    """(M, N, copy) of every GEMM of one projection sweep, in launch order."""
    return [(M, N, rot.next(N)) for M in m_sweep for N in ns]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--skip", default="", help="comma list of phases to skip: decode,prefill")
    ap.add_argument("--no-toy", action="store_true",
                    help="skip the toy-decoder experiment through both libraries")
    ap.add_argument("--toy-runs", type=int, default=100)
    ap.add_argument("--no-table", action="store_true",
                    help="skip the per-shape GEMM timing graphs (counter runs: every library GEMM dispatch is "
                         "then a launch of the sweep, in sweep order)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the supplementary points (RMSNorm 1 GiB, log_softmax, decode S sweep, prefill P sweep)")
    return ap.parse_args()


def gpu_sclk_mhz():
    """Current shader clock (MHz) of the first amdgpu device, from the DPM level
    sysfs marks with '*' (a file read: no child process), or a note."""
    import glob
    import re
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*Mhz", line, re.IGNORECASE)
                        if m:
                            return int(m.group(1))
        except OSError:
            continue
    return "unavailable (no pp_dpm_sclk)"


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "invariant_bi_rmsnorm_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


GEMM_SOURCES = ("gemm.hip", "gemm_tiles.hpp", "gemm_kernel.hpp", "bi_common.hpp")
COPY_PROBE_BYTES = 512 << 20


def traffic_from_profile():
    """HBM bytes per bi_matmul launch of the sweep, from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE scaled by the copy probe), if it
    was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "gemm_llama_sweep_counters.json")
    try:
        with open(p) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != src_hash(*GEMM_SOURCES):
        return None
    return d.get("traffic_bytes_per_launch")


def invariance_cost(result: dict) -> dict:
    """Time of the invariant build over the time of the same work through the
    non-invariant baseline library (libbi_nb.so), per phase, from the rows the
    run measured (above 1: invariance costs time).  The pages price it at
    about 20% for the matmul alone and 42 s against 26 s end to end."""
    out = {}
    nb = result.get("baseline_nb_gemm_sweep", {})
    if "nb_TFLOP/s" in nb:
        out["gemm_sweep"] = round(nb["nb_TFLOP/s"] / nb["invariant_TFLOP/s"], 3)
    sup = result.get("supplementary", {})
    for r in sup.get("decode_S_sweep", {}).get("rows", []):
        if r["S"] == 256 and r.get("nb_us"):
            out["decode_S256"] = round(r["us"] / r["nb_us"], 3)
    for r in sup.get("prefill_P_sweep", {}).get("rows", []):
        if r.get("nb_us"):
            key = f"prefill_P{r['P']}" + (f"_chunks{r['chunks']}" if "chunks" in r else "")
            out[key] = round(r["us"] / r["nb_us"], 3)
    toy = result.get("toy_experiment", {})
    if "invariant_over_nb_time" in toy:
        out["toy_100_runs"] = toy["invariant_over_nb_time"]
        out["toy_unique_completions"] = {"invariant": toy["invariant"]["unique_completions"],
                                         "nb": toy["nb"]["unique_completions"]}
    out["note"] = ("invariant time / libbi_nb.so time for the same work, from the rows above; the pages: "
                   "about 20% for the matmul alone, 26 s (default) against 55 s and then 42 s (invariant) end "
                   "to end")
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from invariant_bi_rmsnorm_amd import inputs as I
    from invariant_bi_rmsnorm_amd import ops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ops.lib()
    dev = "cuda"
    stream = torch.cuda.current_stream()
    skip = set(s for s in args.skip.split(",") if s)

    def d16(bits):
        return torch.from_numpy(np.array(bits, dtype=np.uint16, copy=True).view(np.int16)).to(dev).view(torch.bfloat16)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    # ------------------------------------------------------------ phase 1 data
    log("setup: projection weights")
    H = I.LLAMA_H
    Ns = I.LLAMA_N
    wn = d16(I.llama_norm_weight())
    W = {N: [d16(I.llama_weight(N))] for N in Ns}
    for N in Ns:
        for _ in range(weight_copies(N * H * 2) - 1):
            W[N].append(W[N][0].clone())
    x = d16(I.llama_x(2048))
    Mmax = max(I.M_SWEEP)
    y = torch.empty((Mmax, H), dtype=torch.bfloat16, device=dev)
    C = {N: torch.empty((Mmax, N), dtype=torch.bfloat16, device=dev) for N in Ns}
    gemm_flops_step = sum(2 * M * N * H for M in I.M_SWEEP for N in Ns)

    # ------------------------------------------------------------ phase 2 data
    S_DEC = 256
    if "decode" not in skip:
        log("setup: paged decode cache")
        g = np.random.default_rng([I.TAG_DECODE, 0, 0])
        lens = I.loguniform_lengths(g, S_DEC)
        table, nblk = I.block_tables(g, lens)
        gen = torch.Generator(device=dev)
        gen.manual_seed(3000)
        kc = torch.randn((nblk, I.ATT_HKV, 16, I.ATT_D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        vc = torch.randn((nblk, I.ATT_HKV, I.ATT_D, 16), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        qd = d16(I.queries(I.TAG_DECODE, 0, S_DEC))
        knew = d16(I.normal_bf16(g, (S_DEC, I.ATT_HKV, I.ATT_D)))
        vnew = d16(I.normal_bf16(g, (S_DEC, I.ATT_HKV, I.ATT_D)))
        slots = torch.from_numpy(np.array([I.slots_for(table[s], [lens[s] - 1])[0] for s in range(S_DEC)],
                                          np.int32)).to(dev)
        tbl = torch.from_numpy(table).to(dev)
        lens_d = torch.from_numpy(lens).to(dev)
        max_len = int(lens.max())
        ws = torch.empty(ops.bi_attention_workspace_bytes(S_DEC, I.ATT_HQ, I.ATT_D, max_len) // 4 + 4,
                         dtype=torch.float32, device=dev)
        dec_out = torch.empty((S_DEC, I.ATT_HQ, I.ATT_D), dtype=torch.bfloat16, device=dev)
        dec_bytes = (int(lens.sum()) * I.ATT_HKV * I.ATT_D * 2 * 2 + S_DEC * I.ATT_HQ * I.ATT_D * 2 * 2
                     + 4 * int(sum(-(-int(L) // 16) for L in lens)))
    # ------------------------------------------------------------ phase 3 data
    P_PRE = 8192
    if "prefill" not in skip:
        log("setup: prefill prompt")
        gp = np.random.default_rng([I.TAG_PREFILL, 0, 0])
        ptable, pnblk = I.block_tables(gp, [P_PRE])
        genp = torch.Generator(device=dev)
        genp.manual_seed(4000)
        pk = torch.randn((pnblk, I.ATT_HKV, 16, I.ATT_D), generator=genp, device=dev).to(torch.bfloat16)
        pv = torch.randn((pnblk, I.ATT_HKV, I.ATT_D, 16), generator=genp, device=dev).to(torch.bfloat16)
        pq = torch.randn((P_PRE, I.ATT_HQ, I.ATT_D), generator=genp, device=dev).to(torch.bfloat16)
        ptbl = torch.from_numpy(ptable).to(dev)
        pqs = torch.tensor([0, P_PRE], dtype=torch.int32, device=dev)
        plens = torch.tensor([P_PRE], dtype=torch.int32, device=dev)
        pout = torch.empty_like(pq)
        pre_flops = 4 * I.ATT_HQ * I.ATT_D * (P_PRE * (P_PRE + 1) // 2)
    scale = 1.0 / math.sqrt(I.ATT_D)

    # ------------------------------------------------------------ one step
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    rec = {"phase1": [], "decode": [], "prefill": []}
    rot = WeightRotation({N: len(W[N]) for N in Ns})

    def phase1(record: bool = False):
        for M in I.M_SWEEP:
            ops.bi_rmsnorm(x[:M], wn, I.LLAMA_EPS, y=y[:M], want_rstd=False)
            for N in Ns:
                ops.bi_matmul(y[:M], W[N][rot.next(N)], c=C[N][:M])

    def phase2():
        ops.bi_kv_append(knew, vnew, slots, kc, vc)
        ops.bi_attention_decode(qd, kc, vc, tbl, lens_d, max_len, scale, ws=ws, out=dec_out)

    def phase3():
        ops.bi_attention_prefill(pq, pqs, plens, pk, pv, ptbl, P_PRE, scale, out=pout)

    phases = [("phase1", lambda: phase1(False))]
    if "decode" not in skip:
        phases.append(("decode", phase2))
    if "prefill" not in skip:
        phases.append(("prefill", phase3))

    # Eager reference outputs, then one HIP graph per phase (the sweep is
    # ~200 launches of a few microseconds each: replaying them as a graph
    # removes the host launch gaps, as a serving loop would).
    for _, fn in phases:
        fn()
    torch.cuda.synchronize()
    ref_c = C[14336][:64].clone()
    graphs = {}
    for name, fn in phases:
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            fn()
        graphs[name] = gph
    torch.cuda.synchronize()

    def total_ms(pairs):
        return sum(a.elapsed_time(b) for a, b, *_ in pairs)

    def step(record: bool):
        for name, _ in phases:
            if record:
                a, b = E(), E()
                a.record(stream)
            graphs[name].replay()
            if record:
                b.record(stream)
                rec[name].append((a, b))

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"timed {args.steps}")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    sclk_after = gpu_sclk_mhz()
    # the replayed sweep ends with M=2048: its first rows must equal the eager run bit for bit
    graph_matches_eager = bool(torch.equal(C[14336][:64].view(torch.int16), ref_c.view(torch.int16)))
    # Per-launch durations without host launch gaps: the sweep's 138 GEMM
    # launches captured as one HIP graph (the RMSNorms left out), each shape as
    # a graph of 4 launches over its 4 weight copies, and the 69 RMSNorms as one
    # graph; HIP events on the stream the graphs are replayed on bracket the
    # replays (median of several).
    def capture(fn):
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            fn()
        return gph

    def replay_ms(gph, reps):
        gph.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a_, b_ = E(), E()
            a_.record(stream)
            gph.replay()
            b_.record(stream)
            torch.cuda.synchronize()
            ts.append(a_.elapsed_time(b_))
        return float(np.median(ts))

    def gemm_sweep_only():
        for M in I.M_SWEEP:
            for N in Ns:
                ops.bi_matmul(y[:M], W[N][rot.next(N)], c=C[N][:M])

    def rms_sweep_only():
        for M in I.M_SWEEP:
            ops.bi_rmsnorm(x[:M], wn, I.LLAMA_EPS, y=y[:M], want_rstd=False)

    reps = max(5, args.steps)
    g_gemm = capture(gemm_sweep_only)
    gemm_ms = replay_ms(g_gemm, reps)                     # one sweep of 138 launches
    del g_gemm
    g_rms = capture(rms_sweep_only)
    rms_ms = replay_ms(g_rms, reps)
    del g_rms
    order = [(M, N) for M in I.M_SWEEP for N in Ns]
    n_launch = len(order)
    gemm_flops = sum(2 * M * N * H for (M, N) in order)
    gemm_bytes = sum(2 * (M * H + N * H + M * N) for (M, N) in order)
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
    traffic = traffic_from_profile()
    phase1_ms = total_ms(rec["phase1"]) / args.steps
    value = gemm_flops_step / (phase1_ms * 1e-3) / 1e12

    # per-shape table: a graph of PER_SHAPE_LAUNCHES launches of the shape, each
    # on the next copy of its weight (the same number for every shape, so the
    # kernel trace's average over all launches keeps the sweep's mix)
    per_us = {}
    per_nb_us = {}
    if not args.no_table:
        for (M, N) in order:
            gph = capture(lambda: [ops.bi_matmul(y[:M], W[N][rot.next(N)], c=C[N][:M])
                                   for _ in range(PER_SHAPE_LAUNCHES)])
            per_us[(M, N)] = replay_ms(gph, 3) * 1e3 / PER_SHAPE_LAUNCHES
            del gph
        # the same table through the non-invariant build (its split-K at small M)
        prev_lib = ops.use_library(ops.NB_LIB_PATH)
        try:
            for (M, N) in order:
                gph = capture(lambda: [ops.bi_matmul(y[:M], W[N][rot.next(N)], c=C[N][:M])
                                       for _ in range(PER_SHAPE_LAUNCHES)])
                per_nb_us[(M, N)] = replay_ms(gph, 3) * 1e3 / PER_SHAPE_LAUNCHES
                del gph
        except Exception as e:  # context only
            log(f"per-shape nb table skipped: {type(e).__name__}: {e}")
            per_nb_us = {}
        finally:
            ops.use_library(prev_lib)
    sweep = []
    for (M, N) in sorted(per_us):
        t = per_us[(M, N)] * 1e-6
        fl = 2 * M * N * H
        byt = 2 * (M * H + N * H + M * N)
        roof_t = max(fl / (PEAK_BF16_TFLOPS * 1e12), byt / (PEAK_HBM_GBS * 1e9))
        row = {"M": M, "N": N, "us": round(t * 1e6, 2), "tflops": round(fl / t / 1e12, 2),
               "frac_mfma_peak": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4),
               "frac_roofline": round(roof_t / t, 4), "GB/s": round(byt / t / 1e9, 1)}
        if (M, N) in per_nb_us:
            row["nb_us"] = round(per_nb_us[(M, N)], 2)
            row["invariant_over_nb_time"] = round(per_us[(M, N)] / per_nb_us[(M, N)], 3)
        sweep.append(row)

    avg_launch_s = gemm_ms * 1e-3 / n_launch
    achieved_gbs = gemm_bytes / n_launch / avg_launch_s / 1e9
    if gemm_flops / gemm_bytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        bound, achieved_r, peak_r, unit_r = "hbm", achieved_gbs, PEAK_HBM_GBS, "GB/s"
    else:
        bound, achieved_r, peak_r, unit_r = "mfma", achieved, PEAK_BF16_TFLOPS, "TFLOP/s"
    roof_total = sum(max(2 * M * N * H / (PEAK_BF16_TFLOPS * 1e12), 2 * (M * H + N * H + M * N) / (PEAK_HBM_GBS * 1e9))
                     for (M, N) in order)
    meas_total = sum(per_us.values()) * 1e-6
    rms_bytes = sum(4 * M * H + 2 * H for M in I.M_SWEEP)

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama8b-projection sweep (RMSNorm 4096 + bf16 GEMM 4096->4096 and 4096->14336, "
                        "M=1..64,128,256,512,1024,2048) + paged decode S=256 + causal prefill 8192",
            "M_sweep": list(I.M_SWEEP), "hidden": H, "N": list(Ns),
            "gemm_tile": "one per-element chain (fp32 from 0, one v_mfma_f32_16x16x32_bf16 per 32-wide k chunk, ascending) dealt out by nine tiles chosen by shape, all bitwise equal: M<=64 (non-temporal weight loads): 64x64x128 where 64-wide tiles give >= 3/4 of the CUs in workgroups, else 16x16x256 (M<=16), 16x32x256 (M<=32) or 32x32x128 with 6 stages; M>64: the largest of 64x32x128 / 64x64x128 / 128x64x128 / 128x128x64 / 256x128x64 no taller than M rounded up to 64 giving >= 3/4 of the CUs in workgroups; global_load_lds pipelines of 3-6 stages, next k tile read from LDS during the current MFMAs",
            "value_basis": "GEMM flops of the sweep / GPU time of the projection phase (HIP graph replay)",
            "graph_matches_eager": graph_matches_eager,
            "gpu_sclk_mhz_after_timed_steps": sclk_after,
        },
        "roofline": {
            "kernel": "bi_matmul (gemm_kernel)",
            # the sweep's algorithmic intensity (flops / bytes over all its
            # launches) sits below the MFMA/HBM ridge, so HBM is its bound
            "bound": bound, "achieved": round(achieved_r, 3), "peak": peak_r,
            "unit": unit_r, "frac": round(achieved_r / peak_r, 5),
            "traffic": traffic,
            "sweep_intensity_flop_per_byte": round(gemm_flops / gemm_bytes, 1),
            "ridge_flop_per_byte": round(PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9), 1),
            "mfma_view": {"achieved_tflops": round(achieved, 3), "peak_tflops": PEAK_BF16_TFLOPS,
                          "frac": round(achieved / PEAK_BF16_TFLOPS, 5)},
            "launches": n_launch, "avg_launch_us": round(gemm_ms * 1e3 / n_launch, 3),
            "flops_per_launch_avg": gemm_flops / n_launch,
            "algorithmic_bytes_per_launch_avg": gemm_bytes / n_launch,
            "frac_of_min_roofline": round(roof_total / meas_total, 4) if meas_total else None,
            "timing": ("the sweep's 138 GEMM launches as one HIP graph (no RMSNorm), replayed "
                       f"{reps} times, median; HIP events on the replaying stream"),
            "source_hash": src_hash(*GEMM_SOURCES),
        },
        "gemm_sweep": sweep,
        "gemm_sweep_timing": "each shape as a HIP graph of 5 launches, each on the next copy of its weight "
                             "(N=4096: 16 copies, 537 MB; N=14336: 5 copies, 587 MB: every launch reads its "
                             "weights from HBM); GB/s = algorithmic bytes 2(MK+NK+MN) / time; nb_us = the same "
                             "graph through libbi_nb.so",
        "rmsnorm": {"GB/s": round(rms_bytes / (rms_ms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(rms_bytes / (rms_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "note": "the 69 RMSNorms of the sweep (M=1..2048 rows of 4096) as one HIP graph; "
                            "launch-latency bound at this size"},
    }
    if "decode" not in skip:
        dms = total_ms(rec["decode"]) / args.steps
        gbs = dec_bytes / (dms * 1e-3) / 1e9
        result["decode_attn"] = {"S": S_DEC, "kv_tokens": int(lens.sum()), "max_len": max_len,
                                 "us": round(dms * 1e3, 2), "GB/s": round(gbs, 1),
                                 "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "bytes": dec_bytes,
                                 "includes": "bi_kv_append + split kernel + combine kernel"}
    if "prefill" not in skip:
        pms = total_ms(rec["prefill"]) / args.steps
        tf = pre_flops / (pms * 1e-3) / 1e12
        result["prefill"] = {"P": P_PRE, "us": round(pms * 1e3, 1), "TFLOP/s": round(tf, 2),
                             "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4)}

    # ------------------------------------------------------------ supplementary points
    # (outside the step; each timed as a HIP graph of back-to-back launches)
    def graph_us(fn, reps):
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            for _ in range(reps):
                fn()
        gph.replay()
        torch.cuda.synchronize()
        a, b = E(), E()
        a.record(stream)
        gph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    if not args.no_extra:
        extra = {}
        log("supplementary: RMSNorm 65536 x 4096")
        Mbig = 65536
        xb = torch.randn((Mbig, H), device=dev, dtype=torch.float32).to(torch.bfloat16)
        yb = torch.empty_like(xb)
        us = graph_us(lambda: ops.bi_rmsnorm(xb, wn, I.LLAMA_EPS, y=yb, want_rstd=False), 5)
        byt = 4 * Mbig * H + 2 * H
        extra["rmsnorm_65536x4096"] = {"us": round(us, 1), "bytes": byt,
                                       "GB/s": round(byt / (us * 1e-6) / 1e9, 1),
                                       "frac_hbm": round(byt / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        del xb, yb
        log("supplementary: log_softmax")
        for rows_ls in (256, 8192):
            Vls = 32000
            xl = torch.randn((rows_ls, Vls), device=dev, dtype=torch.float32) * 3
            yl = torch.empty_like(xl)
            us = graph_us(lambda: ops.bi_log_softmax(xl, out=yl), 5)
            byt = 8 * rows_ls * Vls
            extra[f"log_softmax_{rows_ls}x{Vls}"] = {"us": round(us, 1), "bytes": byt,
                                                    "GB/s": round(byt / (us * 1e-6) / 1e9, 1),
                                                    "frac_hbm": round(byt / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            del xl, yl
        if "decode" not in skip:
            log("supplementary: decode S sweep")
            rows = []
            for Sd in (1, 2, 4, 8, 16, 32, 64, 128, 256):
                ls = lens[:Sd]
                ml = int(ls.max())
                us = graph_us(lambda: ops.bi_attention_decode(qd[:Sd], kc, vc, tbl[:Sd], lens_d[:Sd], ml, scale,
                                                              ws=ws, out=dec_out[:Sd]), 10)
                byt = (int(ls.sum()) * I.ATT_HKV * I.ATT_D * 4 + Sd * I.ATT_HQ * I.ATT_D * 4
                       + 4 * int(sum(-(-int(L) // 16) for L in ls)))
                rows.append({"S": Sd, "kv_tokens": int(ls.sum()), "us": round(us, 2),
                             "GB/s": round(byt / (us * 1e-6) / 1e9, 1)})
            # the same calls through the non-invariant build (split length chosen
            # from the batch, as a load-tuned kernel would): what fixed splits cost
            prev = ops.use_library(ops.NB_LIB_PATH)
            try:
                ws_nb = torch.empty(ops.bi_attention_workspace_bytes(S_DEC, I.ATT_HQ, I.ATT_D, max_len) // 4 + 4,
                                    dtype=torch.float32, device=dev)
                for r in rows:
                    Sd = r["S"]
                    ls = lens[:Sd]
                    ml = int(ls.max())
                    r["nb_us"] = round(graph_us(lambda: ops.bi_attention_decode(
                        qd[:Sd], kc, vc, tbl[:Sd], lens_d[:Sd], ml, scale, ws=ws_nb, out=dec_out[:Sd]), 10), 2)
            finally:
                ops.use_library(prev)
            del ws_nb
            extra["decode_S_sweep"] = {"rows": rows, "includes": "split + combine (no append)",
                                       "nb_us": "libbi_nb.so: split length from the load (not invariant)",
                                       "note": "aggregate KV below the 256 MB MALL at small S"}
        if "prefill" not in skip:
            log("supplementary: prefill P sweep")
            rows = []
            for P in (512, 2048, 8192):
                qsP = torch.tensor([0, P], dtype=torch.int32, device=dev)
                lP = torch.tensor([P], dtype=torch.int32, device=dev)
                us = graph_us(lambda: ops.bi_attention_prefill(pq[:P], qsP, lP, pk, pv, ptbl, P, scale,
                                                               out=pout[:P]), 3)
                fl = 4 * I.ATT_HQ * I.ATT_D * (P * (P + 1) // 2)
                rows.append({"P": P, "us": round(us, 1), "TFLOP/s": round(fl / (us * 1e-6) / 1e12, 1)})
            # the 8192-token prompt in chunks over the growing cache: 2048-token
            # chunks (every chunk starts on a 256-token split boundary) and
            # 2000-token chunks (they do not)
            def chunk_calls(CH):
                starts = list(range(0, P_PRE, CH))
                args = []
                for st in starts:
                    n = min(CH, P_PRE - st)
                    args.append((st, n, torch.tensor([0, n], dtype=torch.int32, device=dev),
                                 torch.tensor([st + n], dtype=torch.int32, device=dev)))

                def run():
                    for st, n, qs_c, l_c in args:
                        ops.bi_attention_prefill(pq[st:st + n], qs_c, l_c, pk, pv, ptbl, n, scale,
                                                 out=pout[st:st + n])
                return run
            for CH in (2048, 2000):
                us = graph_us(chunk_calls(CH), 2)
                rows.append({"P": P_PRE, "chunks": CH, "us": round(us, 1),
                             "TFLOP/s": round(pre_flops / (us * 1e-6) / 1e12, 1)})
            # the same calls through the non-invariant build, whose splits start
            # at each chunk's first cache block instead of position 0
            prev = ops.use_library(ops.NB_LIB_PATH)
            try:
                for r in rows:
                    P = r["P"]
                    if "chunks" in r:
                        fn = chunk_calls(r["chunks"])
                    else:
                        qsP = torch.tensor([0, P], dtype=torch.int32, device=dev)
                        lP = torch.tensor([P], dtype=torch.int32, device=dev)
                        fn = (lambda P=P, qsP=qsP, lP=lP: ops.bi_attention_prefill(
                            pq[:P], qsP, lP, pk, pv, ptbl, P, scale, out=pout[:P]))
                    r["nb_us"] = round(graph_us(fn, 2 if "chunks" in r else 3), 1)
            finally:
                ops.use_library(prev)
            extra["prefill_P_sweep"] = {"rows": rows,
                                        "nb_us": "libbi_nb.so: splits start at each chunk's first cache "
                                                 "block (not invariant under re-chunking)"}
        result["supplementary"] = extra

    # copy probe: a plain device copy of known size, the reference for what the
    # HBM traffic counters read per byte, and the copy bandwidth this machine reaches
    src = torch.empty(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    ops.bi_probe_copy(src, dst)
    torch.cuda.synchronize()
    cs, ce = E(), E()
    cs.record(stream)
    for _ in range(5):
        ops.bi_probe_copy(src, dst)
    ce.record(stream)
    torch.cuda.synchronize()
    copy_us = cs.elapsed_time(ce) * 1e3 / 5
    result["copy_probe"] = {"bytes_read": COPY_PROBE_BYTES, "bytes_written": COPY_PROBE_BYTES,
                            "us": round(copy_us, 1),
                            "GB/s": round(2 * COPY_PROBE_BYTES / (copy_us * 1e-6) / 1e9, 1)}
    # read probe: the achievable HBM read rate (the buffer is twice the
    # last-level cache), the practical ceiling of decode and of the GEMMs that
    # stream their weights
    sink = torch.zeros(ops.PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
    ops.bi_probe_read(src, sink)
    torch.cuda.synchronize()
    cs, ce = E(), E()
    cs.record(stream)
    for _ in range(5):
        ops.bi_probe_read(src, sink)
    ce.record(stream)
    torch.cuda.synchronize()
    read_us = cs.elapsed_time(ce) * 1e3 / 5
    read_gbs = COPY_PROBE_BYTES / (read_us * 1e-6) / 1e9
    result["read_probe"] = {"bytes": COPY_PROBE_BYTES, "us": round(read_us, 1), "GB/s": round(read_gbs, 1),
                            "frac_hbm": round(read_gbs / PEAK_HBM_GBS, 4)}
    # global -> LDS fill rate of the staging instruction, by where the data
    # comes from (L2 of each XCD, last-level cache, HBM), one and two
    # workgroups of 8 wavefronts per CU: the feed rate that bounds the GEMM
    # tiles, which stage (BM + BN) x BK x 2 bytes per k tile
    fill = []
    for span in (2 << 20, 64 << 20, COPY_PROBE_BYTES):
        for per_cu in (1, 2):
            wgs = 256 * per_cu
            iters = (16 << 20) // (8 * 8192) // per_cu
            ops.bi_probe_lds_fill(src, span, wgs, iters, sink)
            torch.cuda.synchronize()
            cs, ce = E(), E()
            cs.record(stream)
            for _ in range(3):
                ops.bi_probe_lds_fill(src, span, wgs, iters, sink)
            ce.record(stream)
            torch.cuda.synchronize()
            us = cs.elapsed_time(ce) * 1e3 / 3
            fill.append({"span_MB": span >> 20, "workgroups_per_CU": per_cu, "us": round(us, 1),
                         "bytes": wgs * 8 * iters * 8192})
    # per clock at the shader clock read right after the probe (2400 MHz, the
    # nominal peak clock, when the box does not expose it)
    sclk_probe = gpu_sclk_mhz()
    clk_mhz = sclk_probe if isinstance(sclk_probe, int) else 2400
    for r in fill:
        moved = r.pop("bytes")
        r["TB/s"] = round(moved / (r["us"] * 1e-6) / 1e12, 2)
        r["B_per_clk_per_CU"] = round(moved / (r["us"] * 1e-6) / (clk_mhz * 1e6) / 256, 1)
    result["lds_fill_probe"] = {"rows": fill, "clock_MHz": clk_mhz,
                                "clock_source": "sysfs" if isinstance(sclk_probe, int) else "nominal",
                                "note": "global_load_lds_dwordx4, 8 wavefronts per workgroup, 8-16 1 KB "
                                        "loads in flight per wavefront; 256 CUs"}
    result["roofline"]["achievable_read_GB/s"] = round(read_gbs, 1)
    result["roofline"]["frac_of_achievable_read"] = round(result["roofline"]["achieved"] / read_gbs, 4)
    if "decode_attn" in result:
        result["decode_attn"]["frac_of_read_probe"] = round(result["decode_attn"]["GB/s"] / read_gbs, 4)
    del src, dst, sink

    # the same sweep of GEMMs (no RMSNorm) through the invariant library and through
    # libbi_nb.so (batch-size-dependent K order at small M), each as a HIP graph
    def sweep_gemms():
        for M in I.M_SWEEP:
            for N in Ns:
                ops.bi_matmul(y[:M], W[N][rot.next(N)], c=C[N][:M])

    try:
        inv_us = graph_us(sweep_gemms, 1)
        prev = ops.use_library(ops.NB_LIB_PATH)
        try:
            nb_us = graph_us(sweep_gemms, 1)
        finally:
            ops.use_library(prev)
        result["baseline_nb_gemm_sweep"] = {
            "invariant_TFLOP/s": round(gemm_flops_step / (inv_us * 1e-6) / 1e12, 3),
            "nb_TFLOP/s": round(gemm_flops_step / (nb_us * 1e-6) / 1e12, 3),
            "note": "the 138 GEMMs of the sweep as one HIP graph, invariant library vs libbi_nb.so "
                    "(the library's tiles and rule, plus split-K at M <= 64 where the 64x32 tiles fill at most half "
                    "the CUs: N <= 4096)"}
    except Exception as e:  # context only
        result["baseline_nb_gemm_sweep"] = {"error": str(e)[:200]}

    # non-invariant vendor GEMM (hipBLASLt through torch) on the same sweep, context only
    try:
        torch.cuda.synchronize()
        for rep in range(2):
            bs, be = E(), E()
            bs.record(stream)
            for M in I.M_SWEEP:
                for N in Ns:
                    torch.nn.functional.linear(y[:M], W[N][rot.next(N)], out=C[N][:M])
            be.record(stream)
        torch.cuda.synchronize()
        bms = bs.elapsed_time(be)
        result["baseline_hipblaslt"] = {"TFLOP/s": round(gemm_flops_step / (bms * 1e-3) / 1e12, 3),
                                        "note": "torch.nn.functional.linear on the same sweep (not batch-invariant)"}
    except Exception as e:  # context only
        result["baseline_hipblaslt"] = {"error": str(e)[:200]}

    # ------------------------------------------------------------ toy decoder, both libraries
    # The pages' end-to-end experiment (one prompt decoded greedily many times
    # under a varying co-batched load) through the invariant library and the
    # shape-tuned non-invariant one, on the same load schedule (the schedule is
    # drawn from its own seed, not from the tokens): wall time, tokens/s and
    # the number of distinct completions of each.
    toy_w = None
    if not args.no_toy:
        try:
            from invariant_bi_rmsnorm_amd.toy import Request, ToyEngine, run_load_experiment
            log("toy: weights")
            toy_w = I.toy_weights(I.TOY)
            prompt = I.toy_prompt(I.TOY, 64)
            n_new = 256
            eng = {"invariant": ToyEngine(I.TOY, toy_w, 4096, 1024, 64, 1024)}
            prev = ops.use_library(ops.NB_LIB_PATH)
            try:
                eng["nb"] = ToyEngine.sharing(eng["invariant"])
            finally:
                ops.use_library(prev)
            toy = {"runs": args.toy_runs, "tokens_per_run": n_new, "prompt": 64, "load_seed": 5002,
                   "schedule": "continuous batching of 0-63 other requests (1-512-token prompts, 1-256 new "
                               "tokens), prefill chunks of 16-512 tokens, batch order shuffled every step"}
            for name in ("invariant", "nb"):
                e = eng[name]
                # first step alone on the GPU: the 64-token prompt, as the oracle times it below
                r = Request(10 ** 9, prompt, 1, target=True)
                torch.cuda.synchronize()
                t0s = time.perf_counter()
                e.step([(r, len(prompt))])
                torch.cuda.synchronize()
                first_s = time.perf_counter() - t0s
                e.release(r)
                log(f"toy: {args.toy_runs} runs x {n_new} tokens through {name}")
                e.tokens_processed = 0
                torch.cuda.synchronize()
                t0s = time.perf_counter()
                hashes, stats = run_load_experiment(e, prompt, args.toy_runs, n_new, seed=5002)
                torch.cuda.synchronize()
                dt = time.perf_counter() - t0s
                toy[name] = {"s": round(dt, 3), "unique_completions": len(set(hashes)),
                             "target_tokens_per_s": round(args.toy_runs * n_new / dt, 1),
                             "engine_tokens_per_s": round(e.tokens_processed / dt, 1),
                             "engine_tokens": e.tokens_processed, "steps": stats["steps"],
                             "co_load_mean": round(stats["co_load_mean"], 1),
                             "first_step_prompt64_s": round(first_s, 5)}
            toy["invariant_over_nb_time"] = round(toy["invariant"]["s"] / toy["nb"]["s"], 3)
            result["toy_experiment"] = toy
            del eng
        except Exception as e:  # context only: never lose the result line for it
            result["toy_experiment"] = {"error": f"{type(e).__name__}: {e}"[:300]}

    # ------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        import oracle
        oracle.require_built()      # built before the run; never compiled from a GPU process
        # the oracle on the sweep's own GEMMs (every M, both N, in the sweep's
        # order), stopped once it has run 3 x --cpu-seconds
        a = I.llama_x(2048)
        wts = {N: I.llama_weight(N) for N in Ns}
        fl, done, t = 0, 0, time.perf_counter()
        for M in I.M_SWEEP:
            for N in Ns:
                oracle.matmul(a[:M], wts[N])
                fl += 2 * M * N * H
                done += 1
            if time.perf_counter() - t > 3 * args.cpu_seconds:
                break
        dt = time.perf_counter() - t
        cores = oracle.num_threads()
        result["cpu_baseline"] = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
                                  "sample": f"oracle matmul (fp64) of {done} of the sweep's {2 * len(I.M_SWEEP)} "
                                            f"GEMMs ({fl / 1e9:.0f} GFLOP of {gemm_flops_step / 1e9:.0f}), {dt:.1f} s"}
        # the same oracle on one thread, on the sweep's first GEMMs (bounded)
        try:
            oracle.set_num_threads(1)
            fl1, done1, t = 0, 0, time.perf_counter()
            for M in I.M_SWEEP:
                for N in Ns:
                    oracle.matmul(a[:M], wts[N])
                    fl1 += 2 * M * N * H
                    done1 += 1
                if time.perf_counter() - t > args.cpu_seconds / 2:
                    break
            dt1 = time.perf_counter() - t
            result["cpu_baseline"]["single_thread"] = {
                "value": round(fl1 / dt1 / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                "sample": f"the sweep's first {done1} GEMMs ({fl1 / 1e9:.1f} GFLOP), {dt1:.1f} s"}
        except Exception as e:  # context only
            result["cpu_baseline"]["single_thread"] = {"error": f"{type(e).__name__}: {e}"[:200]}
        finally:
            oracle.set_num_threads(cores)
        # the toy decoder's first step (64-token prompt -> logits of its last token)
        if toy_w is not None:
            try:
                t = time.perf_counter()
                oracle.toy_forward(I.TOY, toy_w, I.toy_prompt(I.TOY, 64))
                dtt = time.perf_counter() - t
                gpu_first = result.get("toy_experiment", {}).get("invariant", {}).get("first_step_prompt64_s")
                result["cpu_baseline"]["toy_first_step"] = {
                    "cpu_s": round(dtt, 3), "cores": cores, "gpu_s": gpu_first,
                    "note": "oracle toy_forward over the 64-token prompt (fp64, 8 layers, vocab 32000) vs the "
                            "invariant engine's step on the same prompt (host-timed, includes one host sync)"}
            except Exception as e:  # context only
                result["cpu_baseline"]["toy_first_step"] = {"error": f"{type(e).__name__}: {e}"[:200]}

        # the oracle beside the other rows, on bounded samples of the same work
        # (GPU times from this run: the instrumented sweep and the supplementary points)
        beside = {}
        try:

            def timed(fn):
                t0 = time.perf_counter()
                fn()
                return time.perf_counter() - t0

            g2048 = capture(lambda: ops.bi_rmsnorm(x[:2048], wn, I.LLAMA_EPS, y=y[:2048], want_rstd=False))
            rms_2048_us = replay_ms(g2048, 5) * 1e3
            del g2048
            dt = timed(lambda: oracle.rmsnorm(I.llama_x(2048), I.llama_norm_weight(), I.LLAMA_EPS))
            beside["rmsnorm_2048x4096"] = {"cpu_s": round(dt, 3), "gpu_us": round(rms_2048_us, 2)}
            sup = result.get("supplementary", {})
            if "log_softmax_256x32000" in sup:
                xl = (np.random.default_rng(7).standard_normal((256, 32000)) * 3).astype(np.float32)
                beside["log_softmax_256x32000"] = {"cpu_s": round(timed(lambda: oracle.log_softmax(xl)), 3),
                                                   "gpu_us": sup["log_softmax_256x32000"]["us"]}
            for Sd in (16, 64):
                if "decode_S_sweep" not in sup:
                    break
                qh = I.queries(I.TAG_DECODE, 0, S_DEC)

                def decode_oracle():
                    for s_ in range(Sd):
                        L_ = int(lens[s_])
                        nb_ = -(-L_ // 16)
                        blk = torch.from_numpy(table[s_, :nb_].astype(np.int64)).to(dev)
                        kh = kc[blk].permute(0, 2, 1, 3).reshape(nb_ * 16, I.ATT_HKV, I.ATT_D)[:L_]
                        vh = vc[blk].permute(0, 3, 1, 2).reshape(nb_ * 16, I.ATT_HKV, I.ATT_D)[:L_]
                        oracle.attention(qh[s_][None], [L_ - 1], kh.contiguous().view(torch.int16).cpu().numpy().view(np.uint16),
                                         vh.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), scale)
                gpu_row = [r for r in sup["decode_S_sweep"]["rows"] if r["S"] == Sd][0]
                beside[f"decode_S{Sd}"] = {"cpu_s": round(timed(decode_oracle), 3), "gpu_us": gpu_row["us"],
                                           "kv_tokens": gpu_row["kv_tokens"],
                                           "note": "cpu_s includes copying those sequences' K/V to the host"}
            for P_ in (512, 2048):
                if "prefill_P_sweep" not in sup:
                    break
                kh = pk[torch.from_numpy(ptable[0, :P_ // 16].astype(np.int64)).to(dev)]
                vh = pv[torch.from_numpy(ptable[0, :P_ // 16].astype(np.int64)).to(dev)]
                kh = kh.permute(0, 2, 1, 3).reshape(P_, I.ATT_HKV, I.ATT_D).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                vh = vh.permute(0, 3, 1, 2).reshape(P_, I.ATT_HKV, I.ATT_D).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                qp = pq[:P_].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                gpu_row = [r for r in sup["prefill_P_sweep"]["rows"] if r["P"] == P_ and "chunks" not in r][0]
                beside[f"prefill_P{P_}"] = {"cpu_s": round(timed(lambda: oracle.attention(qp, np.arange(P_), kh, vh,
                                                                                           scale)), 3),
                                            "gpu_us": gpu_row["us"]}
            for v_ in beside.values():
                v_["cpu_over_gpu"] = round(v_["cpu_s"] / (v_["gpu_us"] * 1e-6), 1)
        except Exception as e:  # context only: never lose the result line for it
            beside["error"] = f"{type(e).__name__}: {e}"[:300]
        result["cpu_oracle_beside"] = beside
    result["invariance_cost"] = invariance_cost(result)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
