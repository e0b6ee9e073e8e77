"""The hot path captured as one HIP graph (as bench.py times it) gives the
eager run's bits on every replay.

The captured sequence is RMSNorm -> GEMM -> KV append -> decode -> causal
prefill.  It holds no memset node: every kernel writes its whole output.  The
graph is replayed three times.  Before each replay its outputs are filled
with NaN, and unrelated eager work plus a synchronisation run in between.
Each replay must reproduce the eager outputs bit for bit.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_util import dev_bf16, dev_i32, host_bits, log  # noqa: E402
from invariant_bi_rmsnorm_amd import inputs as I  # noqa: E402

pytestmark = pytest.mark.gpu

HQ, HKV, D, BLK = I.ATT_HQ, I.ATT_HKV, I.ATT_D, I.BLOCK
SCALE = 1.0 / math.sqrt(D)


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from invariant_bi_rmsnorm_amd import ops as o
    o.lib()
    return o


def test_graph_replays_match_eager(ops):
    g = np.random.default_rng(4242)
    M, H, N = 37, 1024, 512
    x = dev_bf16(I.normal_bf16(g, (M, H)))
    wn = dev_bf16(I.normal_bf16(g, (H,), 1.0, 0.1))
    wt = dev_bf16(I.normal_bf16(g, (N, H), 0.0, 0.02))
    y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    # decode: 6 sequences, the step's token appended first
    lens = np.array([1, 17, 256, 257, 600, 1000], np.int32)
    S = len(lens)
    table, nblk = I.block_tables(g, lens)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    kc = torch.randn((nblk, HKV, BLK, D), generator=gen, device="cuda").to(torch.bfloat16)
    vc = torch.randn((nblk, HKV, D, BLK), generator=gen, device="cuda").to(torch.bfloat16)
    knew = dev_bf16(I.normal_bf16(g, (S, HKV, D)))
    vnew = dev_bf16(I.normal_bf16(g, (S, HKV, D)))
    slots = dev_i32([I.slots_for(table[s], [lens[s] - 1])[0] for s in range(S)])
    qd = dev_bf16(I.normal_bf16(g, (S, HQ, D)))
    tbl, lens_d = dev_i32(table), dev_i32(lens)
    max_len = int(lens.max())
    ws = torch.empty(ops.bi_attention_workspace_bytes(S, HQ, D, max_len) // 4 + 4, dtype=torch.float32,
                     device="cuda")
    dout = torch.empty((S, HQ, D), dtype=torch.bfloat16, device="cuda")

    # prefill: one 300-token prompt over its own cache
    P = 300
    ptable, pnblk = I.block_tables(g, [P])
    pk = torch.randn((pnblk, HKV, BLK, D), generator=gen, device="cuda").to(torch.bfloat16)
    pv = torch.randn((pnblk, HKV, D, BLK), generator=gen, device="cuda").to(torch.bfloat16)
    pq = dev_bf16(I.normal_bf16(g, (P, HQ, D)))
    pqs, plens, ptbl = dev_i32([0, P]), dev_i32([P]), dev_i32(ptable)
    pout = torch.empty((P, HQ, D), dtype=torch.bfloat16, device="cuda")

    def path():
        ops.bi_rmsnorm(x, wn, 1e-6, y=y, want_rstd=False)
        ops.bi_matmul(y, wt, c=c)
        ops.bi_kv_append(knew, vnew, slots, kc, vc)
        ops.bi_attention_decode(qd, kc, vc, tbl, lens_d, max_len, SCALE, ws=ws, out=dout)
        ops.bi_attention_prefill(pq, pqs, plens, pk, pv, ptbl, P, SCALE, out=pout)

    outs = (y, c, dout, pout)
    path()
    torch.cuda.synchronize()
    ref = [host_bits(t) for t in outs]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    torch.cuda.synchronize()

    other_a = dev_bf16(I.normal_bf16(g, (64, 256)))
    other_w = dev_bf16(I.normal_bf16(g, (128, 256)))
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        ops.bi_matmul(other_a, other_w)        # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("rmsnorm", "matmul", "decode", "prefill"), outs, ref):
            assert np.array_equal(host_bits(t), r), f"replay {rep}: {name} differs from the eager run"
        log(f"replay {rep}: bitwise equal to eager")
