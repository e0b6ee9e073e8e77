"""The invariance tests have teeth: libbi_nb.so (same ABI, batch-dependent
strategies for GEMM, RMSNorm and decode and chunk-aligned prefill splits, as
the pages describe ordinary
kernels) computes correct results -- within the oracle tolerance and
run-to-run deterministic -- whose bits nevertheless change with the batch, and
the same tests that pass on libbi.so detect it.  The toy experiment on
libbi_nb.so reports its count of distinct completions (the pages: 80 of 1000)."""
from __future__ import annotations

import math
import os
import time

import numpy as np
import pytest

from gpu_util import check_bf16, dev_bf16, dev_i32, host_bits, log, make_cache
from invariant_bi_rmsnorm_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
SCALE = 1.0 / math.sqrt(128)


@pytest.fixture
def nb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from invariant_bi_rmsnorm_amd import ops as o
    prev = o.use_library(o.NB_LIB_PATH)
    o.lib()
    yield o
    o.use_library(prev)


def test_nb_matmul_correct_but_batch_dependent(nb, orc):
    wt = I.llama_weight(4096)
    wd = dev_bf16(wt)
    x = I.llama_x(256)
    xd = dev_bf16(x)
    big = host_bits(nb.bi_matmul(xd, wd))
    small = host_bits(nb.bi_matmul(xd[:8], wd))
    check_bf16(small, orc.matmul_f64(x[:8], wt), "nb matmul M=8")
    check_bf16(big[:8], orc.matmul_f64(x[:8], wt), "nb matmul M=256")
    assert np.array_equal(host_bits(nb.bi_matmul(xd[:8], wd)), small)     # run-to-run stable
    diff = np.mean(small != big[:8])
    log(f"nb matmul: {diff:.3%} of row bits differ between M=8 and M=256")
    assert diff > 0


def test_nb_rmsnorm_correct_but_batch_dependent(nb, orc):
    w = I.llama_norm_weight()
    x = I.llama_x(64)
    y1, r1 = nb.bi_rmsnorm(dev_bf16(x[:4]), dev_bf16(w), I.LLAMA_EPS)
    y2, r2 = nb.bi_rmsnorm(dev_bf16(x), dev_bf16(w), I.LLAMA_EPS)
    y64, r64 = orc.rmsnorm_f64(x[:4], w, I.LLAMA_EPS)
    check_bf16(host_bits(y1), y64, "nb rmsnorm")
    assert np.max(np.abs(r1.cpu().numpy() / r64 - 1)) <= 1e-5
    differs = (not np.array_equal(host_bits(y1), host_bits(y2)[:4]) or
               not np.array_equal(r1.cpu().numpy().view(np.uint32), r2.cpu().numpy()[:4].view(np.uint32)))
    assert differs


def test_nb_decode_correct_but_batch_dependent(nb, orc):
    g = np.random.default_rng(3)
    L_t = 3001
    kt, vt = I.kv_sequence(I.TAG_DECODE, 9, 0, L_t)
    qt = I.queries(I.TAG_DECODE, 9, 1)
    c1, t1 = make_cache(g, [(kt, vt)])
    alone = host_bits(nb.bi_attention_decode(dev_bf16(qt), c1.k, c1.v, dev_i32(t1), dev_i32([L_t]), L_t, SCALE))[0]
    _, o64 = orc.attention(qt, [L_t - 1], kt, vt, SCALE)
    check_bf16(alone, o64[0], "nb decode")
    S = 64
    lens = I.loguniform_lengths(g, S, 4096)
    lens[5] = L_t
    kvs = [I.kv_sequence(I.TAG_DECODE, 10, s, int(L)) for s, L in enumerate(lens)]
    kvs[5] = (kt, vt)
    q = I.queries(I.TAG_DECODE, 10, S)
    q[5] = qt[0]
    c2, t2 = make_cache(g, kvs)
    inb = host_bits(nb.bi_attention_decode(dev_bf16(q), c2.k, c2.v, dev_i32(t2), dev_i32(lens),
                                           int(lens.max()), SCALE))[5]
    assert not np.array_equal(alone, inb)


def test_nb_prefill_correct_but_chunking_dependent(nb, orc):
    """libbi_nb.so's prefill starts its splits at each chunk's first cache
    block: a single-shot prompt, and chunks that start on multiples of 256,
    give the library's bits; 1000-token chunks change them (the library keeps
    them: test_prefill_chunked_equals_single_shot_and_decode), within the
    oracle's tolerance and run-to-run stable."""
    from invariant_bi_rmsnorm_amd import ops as o
    g = np.random.default_rng(6)
    P = 3001
    k, v = I.kv_sequence(I.TAG_PREFILL, 6, 0, P)
    q = I.queries(I.TAG_PREFILL, 6, P)
    cache, table = make_cache(g, [(k, v)])
    qd = dev_bf16(q)
    tbl = dev_i32(table)

    def run(sizes):
        outs, start = [], 0
        for c in sizes:
            out = o.bi_attention_prefill(qd[start:start + c], dev_i32([0, c]), dev_i32([start + c]), cache.k,
                                         cache.v, tbl, c, SCALE)
            outs.append(host_bits(out))
            start += c
        assert start == P
        return np.concatenate(outs)

    prev = o.use_library(o.DEFAULT_LIB_PATH)
    try:
        inv_single = run([P])
        inv_chunked = run([1000, 1000, 1001])
    finally:
        o.use_library(prev)
    assert np.array_equal(inv_chunked, inv_single)
    assert np.array_equal(run([P]), inv_single), "single shot: splits start at 0 in both builds"
    assert np.array_equal(run([512, 1024, P - 1536]), inv_single), "chunks on split boundaries"
    nb_chunked = run([1000, 1000, 1001])
    assert np.array_equal(run([1000, 1000, 1001]), nb_chunked)            # run-to-run stable
    assert np.array_equal(nb_chunked[:1000], inv_single[:1000])           # first chunk starts at 0
    rows_diff = np.mean(np.any(nb_chunked[1000:] != inv_single[1000:], axis=(1, 2)))
    log(f"nb prefill: {rows_diff:.1%} of the rows of chunks 2-3 differ from single shot")
    assert rows_diff > 0.5
    pos = np.r_[1000:1040, 2950:3001]
    _, o64 = orc.attention(q[pos], pos, k, v, SCALE)
    check_bf16(nb_chunked[pos], o64, "nb chunked prefill", axis=-1)


def test_nb_toy_experiment_gives_several_completions(nb):
    from invariant_bi_rmsnorm_amd.toy import ToyEngine, run_load_experiment
    n_runs = int(os.environ.get("BI_TOY_RUNS", "1000"))
    n_new = int(os.environ.get("BI_TOY_NEW", "256"))
    w = I.toy_weights(I.TOY)
    eng = ToyEngine(I.TOY, w, 4096, 1024, 64, 1024)
    t = time.time()
    hashes, stats = run_load_experiment(eng, I.toy_prompt(I.TOY, 64), n_runs, n_new, seed=5002, progress=log)
    uniq = len(set(hashes))
    log(f"nb toy experiment: {n_runs} runs x {n_new} tokens in {time.time() - t:.1f}s, {stats}, "
        f"unique completions: {uniq}")
    assert len(hashes) == n_runs
    assert uniq > 1


def test_nb_toy_sampled_experiment_gives_several_completions(nb):
    """The sampled (T = 0.8) experiment on the non-invariant build: the same
    seeds and schedule as the invariant test give several completions."""
    from invariant_bi_rmsnorm_amd.toy import ToyEngine, run_load_experiment
    n_runs = int(os.environ.get("BI_TOY_SAMPLED_RUNS", "300"))
    w = I.toy_weights(I.TOY)
    eng = ToyEngine(I.TOY, w, 4096, 1024, 64, 1024)
    t = time.time()
    hashes, stats = run_load_experiment(eng, I.toy_prompt(I.TOY, 64), n_runs, 64, seed=5003, progress=log,
                                        temperature=0.8)
    uniq = len(set(hashes))
    log(f"nb sampled toy experiment (T=0.8): {n_runs} runs x 64 tokens in {time.time() - t:.1f}s, {stats}, "
        f"unique completions: {uniq}")
    assert len(hashes) == n_runs
    assert uniq > 1


def test_nb_flips_happen_where_the_top2_margin_is_small(nb):
    """Where the non-invariant build's completions first leave the invariant
    one, the invariant trajectory's top-1/top-2 logit margin (bi_top2) is
    small: the flips the pages count are near-ties of the two best tokens."""
    from invariant_bi_rmsnorm_amd import ops as o
    from invariant_bi_rmsnorm_amd.toy import Request, ToyEngine, run_load_experiment
    w = I.toy_weights(I.TOY)
    prompt = I.toy_prompt(I.TOY, 64)
    n_new = 256
    # invariant reference, alone, with the margin of every step
    prev = o.use_library(o.DEFAULT_LIB_PATH)
    try:
        ref_eng = ToyEngine(I.TOY, w, 4096, 1024, 64, 1024)
        r = Request(0, prompt, n_new)
        margins = []
        work = [(r, len(prompt))]
        while not r.done:
            ref_eng.step(work, want_logits=True)
            _, m = o.bi_top2(ref_eng.logits[:1])
            margins.append(float(m.item()))
            work = [(r, 1)]
        ref = list(r.generated)
    finally:
        o.use_library(prev)
    margins = np.array(margins)
    # the non-invariant build under load
    eng = ToyEngine(I.TOY, w, 4096, 1024, 64, 1024)
    toks = []
    run_load_experiment(eng, prompt, 300, n_new, seed=5002, tokens_out=toks)
    firsts = sorted({next(i for i, (a, b) in enumerate(zip(t, ref)) if a != b) for t in toks if t != ref})
    flip_m = margins[firsts] if firsts else np.array([])
    log(f"nb flips: first divergence at steps {firsts[:20]}; invariant margins there "
        f"{np.round(flip_m, 4).tolist()[:20]}; median margin over all {len(margins)} steps "
        f"{np.median(margins):.3f}")
    assert len(firsts) > 0
    assert np.max(flip_m) < np.median(margins)
