"""Build libbi.so (all HIP kernels + the C ABI) in-tree with hipcc for gfx950.

    python -m invariant_bi_rmsnorm_amd._build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BASELINE = os.path.join(CSRC, "baseline")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbi.so")
# The non-invariant baseline library: the same ABI, with the batch-dependent
# strategies of csrc/baseline/ in place of the invariant GEMM, RMSNorm,
# decode and prefill.  Used only for measurement and to show the invariance tests can fail.
LIB_NB = os.path.join(HERE, "libbi_nb.so")
REPLACED_IN_NB = {"gemm.hip", "rmsnorm.hip", "attn_decode.hip", "attn_prefill.hip"}

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # every + and * rounds on its own; FMAs only where written explicitly
    "-ffp-contract=off", "-fno-fast-math",
    # no packed fp32 ALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def baseline_sources():
    return sorted(os.path.join(BASELINE, f) for f in os.listdir(BASELINE) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    # -Bsymbolic: calls between entry points bind inside their own library, so
    # both libraries can be loaded into one process
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-Bsymbolic", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    nb_srcs = baseline_sources()
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = dict(zip(srcs + nb_srcs, ex.map(_compile, srcs + nb_srcs)))
    _link([objs[s] for s in srcs], LIB)
    _link([objs[s] for s in srcs if os.path.basename(s) not in REPLACED_IN_NB] +
          [objs[s] for s in nb_srcs], LIB_NB)
    return LIB


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 8))
