#!/usr/bin/env python3
"""Benchmark of the batch-invariant forward path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  1. projections (Llama-8B shapes): for every M in 1..64,128,256,...,2048:
     RMSNorm [M,4096] -> bi_matmul [M,4096]x[4096,4096] -> bi_matmul
     [M,4096]x[4096,14336]   (weights rotated over 4 copies, 604 MB: more than
     twice the 256 MB last-level cache, so weight reads come from HBM);
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
N_WEIGHT_COPIES = 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--skip", default="", help="comma list of phases to skip: decode,prefill")
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


GEMM_SOURCES = ("gemm.hip", "gemm_kernel.hpp", "bi_common.hpp")
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
        for _ in range(N_WEIGHT_COPIES - 1):
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
    rec = {"gemm": [], "rms": [], "phase1": [], "decode": [], "prefill": []}
    call = [0]

    def phase1(record: bool):
        for M in I.M_SWEEP:
            if record:
                rs, re_ = E(), E()
                rs.record(stream)
            ops.bi_rmsnorm(x[:M], wn, I.LLAMA_EPS, y=y[:M], want_rstd=False)
            if record:
                re_.record(stream)
                rec["rms"].append((rs, re_, M))
            for N in Ns:
                wt = W[N][call[0] % N_WEIGHT_COPIES]
                call[0] += 1
                if record:
                    gs, ge = E(), E()
                    gs.record(stream)
                ops.bi_matmul(y[:M], wt, c=C[N][:M])
                if record:
                    ge.record(stream)
                    rec["gemm"].append((gs, ge, 2 * M * N * H, M, N))

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
    # per-launch durations of bi_matmul: eager passes of the same sweep, a HIP
    # event pair around every launch.  Each pass is queued behind a few graph
    # replays of the sweep, so the host has queued every launch before the GPU
    # reaches it and an event pair brackets the kernel, not host launch gaps.
    head = 3
    host_enqueue_ms = []
    for _ in range(max(2, args.steps // 2)):
        for _ in range(head):
            graphs["phase1"].replay()
        th = time.perf_counter()
        phase1(True)
        host_enqueue_ms.append((time.perf_counter() - th) * 1e3)
    torch.cuda.synchronize()

    def total_ms(pairs):
        return sum(a.elapsed_time(b) for a, b, *_ in pairs)

    phase1_ms = total_ms(rec["phase1"]) / args.steps
    value = gemm_flops_step / (phase1_ms * 1e-3) / 1e12
    gemm_ms = total_ms(rec["gemm"])
    gemm_flops = sum(r[2] for r in rec["gemm"])
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
    n_launch = len(rec["gemm"])
    traffic = traffic_from_profile()
    gemm_bytes = sum(2 * (M * H + N * H + M * N) for (_, _, _, M, N) in rec["gemm"])

    # per-M table (median over steps)
    per = {}
    for (a, b, fl, M, N) in rec["gemm"]:
        per.setdefault((M, N), []).append(a.elapsed_time(b))
    sweep = []
    for (M, N), ts in sorted(per.items()):
        t = float(np.median(ts)) * 1e-3
        fl = 2 * M * N * H
        byt = 2 * (M * H + N * H + M * N)
        roof_t = max(fl / (PEAK_BF16_TFLOPS * 1e12), byt / (PEAK_HBM_GBS * 1e9))
        sweep.append({"M": M, "N": N, "us": round(t * 1e6, 2), "tflops": round(fl / t / 1e12, 2),
                      "frac_mfma_peak": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "frac_roofline": round(roof_t / t, 4)})

    avg_launch_s = gemm_ms * 1e-3 / n_launch
    achieved_gbs = gemm_bytes / n_launch / avg_launch_s / 1e9
    if gemm_flops / gemm_bytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        bound, achieved_r, peak_r, unit_r = "hbm", achieved_gbs, PEAK_HBM_GBS, "GB/s"
    else:
        bound, achieved_r, peak_r, unit_r = "mfma", achieved, PEAK_BF16_TFLOPS, "TFLOP/s"
    roof_total = sum(max(2 * M * N * H / (PEAK_BF16_TFLOPS * 1e12), 2 * (M * H + N * H + M * N) / (PEAK_HBM_GBS * 1e9))
                     for (M, N) in per)
    meas_total = sum(float(np.median(ts)) * 1e-3 for ts in per.values())
    rms_ms = total_ms(rec["rms"])
    rms_bytes = sum(4 * M * H + 2 * H for (_, _, M) in rec["rms"])

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
            "gemm_tile": "64x32x128 workgroup tile, 8 waves of 16x16, v_mfma_f32_16x16x32_bf16, 3-stage global_load_lds pipeline (2 in flight)",
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
            "frac_of_min_roofline": round(roof_total / meas_total, 4),
            "timing": (f"event pair per launch in eager sweeps queued behind {head} graph replays "
                       f"({head * phase1_ms:.1f} ms of GPU work); host queued each sweep in "
                       f"{max(host_enqueue_ms):.1f} ms at most"),
            "source_hash": src_hash(*GEMM_SOURCES),
        },
        "gemm_sweep": sweep,
        "rmsnorm": {"GB/s": round(rms_bytes / (rms_ms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(rms_bytes / (rms_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "note": "M=1..2048 rows of 4096, launch-latency bound at this size"},
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
            # the 8192-token prompt as four 2048-token chunks over the growing cache
            CH = 2048
            qs_ch = torch.tensor([0, CH], dtype=torch.int32, device=dev)
            l_ch = [torch.tensor([(c + 1) * CH], dtype=torch.int32, device=dev) for c in range(P_PRE // CH)]

            def chunked():
                for c in range(P_PRE // CH):
                    ops.bi_attention_prefill(pq[c * CH:(c + 1) * CH], qs_ch, l_ch[c], pk, pv, ptbl, CH, scale,
                                             out=pout[c * CH:(c + 1) * CH])
            us = graph_us(chunked, 2)
            rows.append({"P": P_PRE, "chunks": CH, "us": round(us, 1),
                         "TFLOP/s": round(pre_flops / (us * 1e-6) / 1e12, 1)})
            extra["prefill_P_sweep"] = rows
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
    del src, dst

    # the same sweep of GEMMs (no RMSNorm) through the invariant library and through
    # libbi_nb.so (batch-size-dependent K order at small M), each as a HIP graph
    def sweep_gemms():
        for M in I.M_SWEEP:
            for N in Ns:
                ops.bi_matmul(y[:M], W[N][call[0] % N_WEIGHT_COPIES], c=C[N][:M])
                call[0] += 1

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
                    "(the same tile with a batch-size-dependent K order at M <= 128)"}
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
                    torch.nn.functional.linear(y[:M], W[N][call[0] % N_WEIGHT_COPIES], out=C[N][:M])
                    call[0] += 1
            be.record(stream)
        torch.cuda.synchronize()
        bms = bs.elapsed_time(be)
        result["baseline_hipblaslt"] = {"TFLOP/s": round(gemm_flops_step / (bms * 1e-3) / 1e12, 3),
                                        "note": "torch.nn.functional.linear on the same sweep (not batch-invariant)"}
    except Exception as e:  # context only
        result["baseline_hipblaslt"] = {"error": str(e)[:200]}

    # ------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
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
        result["cpu_baseline"] = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
                                  "sample": f"oracle matmul (fp64) of {done} of the sweep's {2 * len(I.M_SWEEP)} "
                                            f"GEMMs ({fl / 1e9:.0f} GFLOP of {gemm_flops_step / 1e9:.0f}), {dt:.1f} s"}

        # the oracle beside the other rows, on bounded samples of the same work
        # (GPU times from this run: the instrumented sweep and the supplementary points)
        beside = {}
        try:

            def timed(fn):
                t0 = time.perf_counter()
                fn()
                return time.perf_counter() - t0

            rms_2048 = [a.elapsed_time(b) * 1e3 for (a, b, M) in rec["rms"] if M == 2048]
            dt = timed(lambda: oracle.rmsnorm(I.llama_x(2048), I.llama_norm_weight(), I.LLAMA_EPS))
            beside["rmsnorm_2048x4096"] = {"cpu_s": round(dt, 3), "gpu_us": round(float(np.median(rms_2048)), 2)}
            sup = result.get("supplementary", {})
            if "log_softmax_256x32000" in sup:
                xl = (np.random.default_rng(7).standard_normal((256, 32000)) * 3).astype(np.float32)
                beside["log_softmax_256x32000"] = {"cpu_s": round(timed(lambda: oracle.log_softmax(xl)), 3),
                                                   "gpu_us": sup["log_softmax_256x32000"]["us"]}
            if "decode_S_sweep" in sup:
                Sd = 16
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
                beside["decode_S16"] = {"cpu_s": round(timed(decode_oracle), 3), "gpu_us": gpu_row["us"],
                                        "kv_tokens": gpu_row["kv_tokens"],
                                        "note": "cpu_s includes copying those sequences' K/V to the host"}
            if "prefill_P_sweep" in sup:
                P_ = 512
                kh = pk[torch.from_numpy(ptable[0, :P_ // 16].astype(np.int64)).to(dev)]
                vh = pv[torch.from_numpy(ptable[0, :P_ // 16].astype(np.int64)).to(dev)]
                kh = kh.permute(0, 2, 1, 3).reshape(P_, I.ATT_HKV, I.ATT_D).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                vh = vh.permute(0, 3, 1, 2).reshape(P_, I.ATT_HKV, I.ATT_D).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                qp = pq[:P_].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                gpu_row = [r for r in sup["prefill_P_sweep"] if r["P"] == P_ and "chunks" not in r][0]
                beside["prefill_P512"] = {"cpu_s": round(timed(lambda: oracle.attention(qp, np.arange(P_), kh, vh,
                                                                                         scale)), 3),
                                          "gpu_us": gpu_row["us"]}
            for v_ in beside.values():
                v_["cpu_over_gpu"] = round(v_["cpu_s"] / (v_["gpu_us"] * 1e-6), 1)
        except Exception as e:  # context only: never lose the result line for it
            beside["error"] = f"{type(e).__name__}: {e}"[:300]
        result["cpu_oracle_beside"] = beside
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
