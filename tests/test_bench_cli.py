"""Host-side contract of bench.py and __graft_entry__ (no GPU needed).

bench.py measures one GPU: any other GPU count, asked for on the command line
or through WORLD_SIZE, must end the run with a message and a non-zero status
before anything touches a GPU.  The helpers that record the host context
must degrade to a note where the information is missing (no amdgpu sysfs in
a container without a GPU) instead of raising.
"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    if env_extra:
        env.update(env_extra)
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def _load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_refuses_more_than_one_gpu():
    r = _bench(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no result line


def test_bench_refuses_a_multi_rank_launch():
    r = _bench(["--steps", "1", "--warmup", "0"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "WORLD_SIZE 2" in r.stderr


def test_bench_host_context_helpers_degrade_to_notes():
    b = _load_bench()
    clk = b.gpu_sclk_mhz()
    assert isinstance(clk, int) and clk > 0 or isinstance(clk, str)
    model = b.cpu_model()
    assert isinstance(model, str) and model
    # the counter-file hash covers the GEMM sources it names
    assert len(b.src_hash(*b.GEMM_SOURCES)) >= 16


def test_graft_entry_exposes_build_and_smoke():
    spec = importlib.util.spec_from_file_location("graft_entry_under_test", os.path.join(ROOT, "__graft_entry__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert callable(mod.build) and callable(mod.smoke)


def test_weight_rotation_touches_every_copy_of_each_n_and_defeats_the_llc():
    """One projection sweep (69 M values x 2 N): each N has at least 3 weight
    copies, more than 512 MB of them, reads all of them in turn, and between two
    reads of one copy more than 256 MB (the MI355X last-level cache) of other
    copies of the same N are read -- so the weights are cold whatever the other
    shape's loads do to the cache."""
    b = _load_bench()
    from invariant_bi_rmsnorm_amd import inputs as I
    nbytes = {N: N * I.LLAMA_H * 2 for N in I.LLAMA_N}
    copies = {N: b.weight_copies(nbytes[N]) for N in I.LLAMA_N}
    for N in I.LLAMA_N:
        assert copies[N] >= 3 and copies[N] * nbytes[N] > 512 * 10**6
    assert copies == {4096: 16, 14336: 5}
    sched = b.sweep_schedule(I.M_SWEEP, I.LLAMA_N, b.WeightRotation(copies))
    assert len(sched) == 2 * len(I.M_SWEEP)
    for N in I.LLAMA_N:
        seq = [c for (_, n, c) in sched if n == N]
        assert set(seq) == set(range(copies[N]))
        assert all(seq[i] != seq[i + 1] for i in range(len(seq) - 1))
        last = {}
        min_gap = None
        for pos, c in enumerate(seq):
            if c in last:
                gap = (pos - last[c] - 1) * nbytes[N]      # other copies of the same N read in between
                min_gap = gap if min_gap is None else min(min_gap, gap)
            last[c] = pos
        assert min_gap is not None and min_gap > 256 * 10**6
    # the rotation continues across sweeps (graph capture, eager passes, baselines)
    rot = b.WeightRotation(copies)
    first = b.sweep_schedule(I.M_SWEEP, I.LLAMA_N, rot)
    second = b.sweep_schedule(I.M_SWEEP, I.LLAMA_N, rot)
    assert [c for (_, _, c) in second][:2] == [len(I.M_SWEEP) % copies[N] for N in I.LLAMA_N]
    assert len(first) == len(second)


def test_profile_summary_names_kernels_by_library():
    """rocprofv3 names kernels with their template arguments; the summaries
    group them per kernel and keep the baseline library's instances apart."""
    sys.path.insert(0, ROOT)
    from invariant_bi_rmsnorm_amd.profile_summary import short
    lib = "void (anonymous namespace)::gemm_kernel<(anonymous namespace)::GemmTile<64, 64, 128, 2, 2, 3, 0, 2>, false>(x)"
    base = "void (anonymous namespace)::gemm_kernel<(anonymous namespace)::GemmTile<64, 32, 128, 4, 2, 3, 1, 0>, true>(x)"
    assert short(lib) == "gemm_kernel"
    assert short(base) == "gemm_kernel (baseline lib)"
    assert short("void (anonymous namespace)::prefill_kernel<false>(unsigned short const*, long)") == "prefill_kernel"
    assert short("void (anonymous namespace)::prefill_kernel<true>(unsigned short const*, long)") == \
        "prefill_kernel (baseline lib)"
    assert short("decode_split_kernel(int, float)") == "decode_split_kernel"
    assert short("void (anonymous namespace)::rmsnorm_kernel<0>(unsigned short const*)") == "rmsnorm_kernel"
    assert short("void at::native::vectorized_elementwise_kernel<4>(int)").startswith("void at::native")


def test_invariance_cost_is_invariant_over_baseline_time_per_phase():
    b = _load_bench()
    result = {
        "baseline_nb_gemm_sweep": {"invariant_TFLOP/s": 300.0, "nb_TFLOP/s": 270.0},
        "supplementary": {
            "decode_S_sweep": {"rows": [{"S": 128, "us": 9.0, "nb_us": 8.0}, {"S": 256, "us": 520.0, "nb_us": 500.0}]},
            "prefill_P_sweep": {"rows": [{"P": 8192, "us": 800.0, "nb_us": 800.0},
                                         {"P": 8192, "chunks": 2000, "us": 1100.0, "nb_us": 1210.0}]}},
        "toy_experiment": {"invariant_over_nb_time": 0.98, "invariant": {"unique_completions": 1},
                           "nb": {"unique_completions": 63}},
    }
    c = b.invariance_cost(result)
    assert c["gemm_sweep"] == 0.9                    # time ratio = inverse of the throughput ratio
    assert c["decode_S256"] == 1.04 and "decode_S128" not in c
    assert c["prefill_P8192"] == 1.0 and c["prefill_P8192_chunks2000"] == 0.909
    assert c["toy_100_runs"] == 0.98 and c["toy_unique_completions"] == {"invariant": 1, "nb": 63}
    assert set(b.invariance_cost({})) == {"note"}     # phases not run leave no entry
