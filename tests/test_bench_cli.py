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
