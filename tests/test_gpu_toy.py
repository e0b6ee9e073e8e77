"""GPU tests of the toy greedy-decode step (include/bi_toy.h): its element-wise
ops against the oracle, first-step logits against the oracle's toy forward,
bitwise invariance of a sequence's logits under batch composition, chunking
and decode/prefill path, and the 1000-run greedy experiment under random
co-batched load, which must give exactly one distinct completion."""
from __future__ import annotations

import math
import os
import time

import numpy as np
import pytest

from gpu_util import bf16_f64, check_bf16, dev_bf16, dev_i32, host_bits, log
from test_toy_tolerance import TOY_MAX_BAR, TOY_RMS_BAR
from invariant_bi_rmsnorm_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from invariant_bi_rmsnorm_amd import ops as o
    o.lib()
    return o


@pytest.fixture(scope="module")
def toy_weights():
    t = time.time()
    w = I.toy_weights(I.TOY)
    log(f"toy weights generated in {time.time() - t:.1f}s")
    return w


def make_engine(w, cfg=I.TOY, num_blocks=4096, max_tokens=1024, max_seqs=64, max_kv_len=1024):
    from invariant_bi_rmsnorm_amd.toy import ToyEngine
    return ToyEngine(cfg, w, num_blocks, max_tokens, max_seqs, max_kv_len)


# ------------------------------------------------------------------ element-wise ops

def test_toy_ops_parity(ops, orc):
    g = np.random.default_rng(1)
    # embed / gather
    table = I.normal_bf16(g, (100, 256))
    ids = g.integers(0, 100, 37).astype(np.int32)
    ids[5] = 100                                  # out of range -> zeros
    out = host_bits(ops.bi_embed(dev_bf16(table), dev_i32(ids)))
    exp = table[np.clip(ids, 0, 99)].copy()
    exp[5] = 0
    assert np.array_equal(out, exp)
    src = I.normal_bf16(g, (50, 64))
    rows = np.array([3, 0, 49, 7], np.int32)
    assert np.array_equal(host_bits(ops.bi_gather_rows(dev_bf16(src), dev_i32(rows))), src[rows])
    # rope on q,k heads of a fused projection, in place
    T, Hq, Hkv, D = 40, 16, 4, 128
    qkv = I.normal_bf16(g, (T, (Hq + 2 * Hkv) * D))
    pos = g.integers(0, 1000, T).astype(np.int32)
    tab = ops.bi_rope_table(1024, D, 10000.0)
    xd = dev_bf16(qkv).view(T, Hq + 2 * Hkv, D)
    ops.bi_rope(xd[:, :Hq + Hkv], dev_i32(pos), tab, 1024)
    got = host_bits(xd).reshape(T, Hq + 2 * Hkv, D)
    ref = orc.rope(qkv.reshape(T, Hq + 2 * Hkv, D)[:, :Hq + Hkv], pos)
    diff = np.abs(I.bf16_to_f32(got[:, :Hq + Hkv]).astype(np.float64) - I.bf16_to_f32(ref).astype(np.float64))
    assert np.all(diff <= 1e-2 * 1.0 + np.abs(I.bf16_to_f32(ref)) * 2 ** -7)
    assert np.mean(got[:, :Hq + Hkv] == ref) > 0.99                      # rounding ties aside: same bits
    assert np.array_equal(got[:, Hq + Hkv:], qkv.reshape(T, Hq + 2 * Hkv, D)[:, Hq + Hkv:])   # v untouched
    # add, silu*mul
    a = I.normal_bf16(g, (1000,))
    b = I.normal_bf16(g, (1000,))
    assert np.array_equal(host_bits(ops.bi_add(dev_bf16(a), dev_bf16(b))), orc.add(a, b))
    gu = I.normal_bf16(g, (9, 2 * 512), 0, 2.0)
    s = host_bits(ops.bi_silu_mul(dev_bf16(gu)))
    sr = orc.silu_mul(np.ascontiguousarray(gu[:, :512]), np.ascontiguousarray(gu[:, 512:]))
    check_bf16(s, I.bf16_to_f32(sr).astype(np.float64), "silu_mul")


def test_rope_kv_append_equals_rope_then_append(ops):
    """The fused rotary embedding + cache append gives the bits of bi_rope on
    the q and k heads followed by bi_kv_append of k and v: the rotated
    projection and both caches, with slots outside the pool (no cache write)
    and positions outside the table (position 0)."""
    from gpu_util import PagedCache
    g = np.random.default_rng(17)
    T, Hq, Hkv, D, nblk = 45, 16, 4, 128, 8
    qkv = I.normal_bf16(g, (T, (Hq + 2 * Hkv) * D))
    pos = g.integers(0, 1000, T).astype(np.int32)
    pos[3], pos[4] = -1, 5000
    slots = g.permutation(nblk * 16)[:T].astype(np.int32)
    slots[7], slots[8] = -1, nblk * 16
    tab = ops.bi_rope_table(1024, D, 10000.0)
    results = []
    for fused in (False, True):
        x = dev_bf16(qkv)
        cache = PagedCache(nblk, Hkv)
        cache.k.fill_(float("nan"))
        cache.v.fill_(float("nan"))
        if fused:
            ops.bi_rope_kv_append(x, Hq, Hkv, dev_i32(pos), dev_i32(slots), tab, 1024, cache.k, cache.v)
        else:
            xv = x.view(T, Hq + 2 * Hkv, D)
            ops.bi_rope(xv[:, :Hq + Hkv], dev_i32(pos), tab, 1024)
            ops.bi_kv_append(xv[:, Hq:Hq + Hkv], xv[:, Hq + Hkv:], dev_i32(slots), cache.k, cache.v)
        results.append((host_bits(x), host_bits(cache.k), host_bits(cache.v)))
    for a, b, what in zip(results[0], results[1], ("qkv", "k cache", "v cache")):
        assert np.array_equal(a, b), what


# ------------------------------------------------------------------ first step vs oracle

def test_toy_first_step_logits_parity(ops, orc, toy_weights):
    from invariant_bi_rmsnorm_amd.toy import Request
    eng = make_engine(toy_weights)
    prompt = I.toy_prompt(I.TOY, 64)
    r = Request(0, prompt, 4)
    nxt, lg = eng.step([(r, 64)], want_logits=True)
    t = time.time()
    ref = orc.toy_forward(I.TOY, toy_weights, prompt)
    log(f"oracle toy forward: {time.time() - t:.1f}s")
    gpu = lg[0].astype(np.float64)
    rms = math.sqrt(float(np.mean(ref ** 2)))
    err = np.abs(gpu - ref)
    rms_err = math.sqrt(float(np.mean(err ** 2)))
    log(f"first-step logits: max err {err.max():.3e}, rms err {rms_err:.3e}, rms {rms:.3e}")
    # Each of the ~100 ops of the 8-layer forward rounds to bf16 and may land
    # one ulp away from the oracle's rounding; those differences travel
    # through the later layers.  The bar (derived in test_toy_tolerance.py from
    # an independent fp32 evaluation, which drifts 1.3e-2 RMS / 5e-2 max from
    # the oracle) is error RMS <= 2e-2 and max <= 1e-1 of the logits' RMS;
    # per-op parity at the 1e-2 bar is tested op by op.
    assert rms_err <= TOY_RMS_BAR * rms
    assert err.max() <= TOY_MAX_BAR * rms
    top2 = np.sort(ref)[-2:]
    if top2[1] - top2[0] > 2 * err.max():           # the oracle's choice is unambiguous
        assert int(nxt[0]) == int(np.argmax(ref))


# Ratios of the end-to-end bar to the drift of an independent fp32 evaluation
# from the oracle at full depth (test_toy_tolerance.py: 2e-2 over 1.28e-2 RMS,
# 1e-1 over 4.95e-2 max).  The depth test holds the GPU to the same multiples of
# that evaluation's drift at each depth.
DEPTH_RMS_RATIO = 1.6
DEPTH_MAX_RATIO = 2.0


@pytest.mark.parametrize("layers", [1, 2, 4])
def test_toy_logits_parity_at_each_depth(ops, orc, toy_weights, layers):
    """The decoder cut after `layers` layers (embedding, those layers, final
    norm, head) against the oracle's forward of the same cut model.  At depth 1
    the rounding differences of two correct evaluations have not yet
    compounded, so the bar is tight and pins the driver's wiring (QKV slicing,
    RoPE of q and k, GQA grouping, gate|up split, residual adds) one layer at a
    time, instead of only through the 8-layer bar."""
    from invariant_bi_rmsnorm_amd.toy import Request
    from toy_ref32 import toy_logits_fp32
    cfg = dict(I.TOY, layers=layers)
    w = dict(toy_weights, layers=toy_weights["layers"][:layers])
    eng = make_engine(w, cfg=cfg)
    prompt = I.toy_prompt(I.TOY, 64)
    r = Request(0, prompt, 4)
    nxt, lg = eng.step([(r, 64)], want_logits=True)
    ref = orc.toy_forward(cfg, w, prompt)
    alt = toy_logits_fp32(cfg, w, prompt)
    rms = math.sqrt(float(np.mean(ref ** 2)))
    drift = np.abs(alt - ref)
    bar_rms = DEPTH_RMS_RATIO * math.sqrt(float(np.mean(drift ** 2)))
    bar_max = DEPTH_MAX_RATIO * float(drift.max())
    err = np.abs(lg[0].astype(np.float64) - ref)
    rms_err = math.sqrt(float(np.mean(err ** 2)))
    log(f"depth {layers}: gpu rms err {rms_err / rms:.3e}, max {err.max() / rms:.3e} of RMS; "
        f"bars {bar_rms / rms:.3e}, {bar_max / rms:.3e} (fp32 evaluation x {DEPTH_RMS_RATIO}, x {DEPTH_MAX_RATIO})")
    assert rms_err <= bar_rms
    assert err.max() <= bar_max
    top2 = np.sort(ref)[-2:]
    if top2[1] - top2[0] > 2 * err.max():
        assert int(nxt[0]) == int(np.argmax(ref))


def test_toy_each_layer_from_gpu_input_bits_matches_the_oracle_layer(ops, orc, toy_weights):
    """Each of the 8 layers alone: the driver's residual stream after layer l
    (the model cut after l layers, 64-token prompt) against the oracle's layer
    l applied to the GPU's own stream after layer l - 1 (the embedding rows for
    l = 1).  No rounding difference carries over from earlier layers, so each
    layer's wiring (QKV slicing, RoPE of q and k, GQA grouping, gate|up split,
    residual adds) is pinned on its own; a wiring slip moves the stream by a
    sizeable part of a branch's RMS.

    The bar is set, as for the depth test, by how far an independent CPU
    evaluation of the same layer from the same input bits drifts from the
    oracle: error RMS within 1.6x and max error within 2x of that drift.  The
    CPU evaluation (fp32, each op rounded to bf16) rounds the softmax weights
    to bf16 before their sum and the value product, as the kernels' attention
    splits do.  That rounding dominates the drift of the stream: without it the
    fp32 evaluation leaves 10% of the stream values off the oracle's by an ulp
    at the first layer, with it 43%, as many as the GPU.  The per-op bar (1e-2
    of the output's RMS) is not used here: a layer chains about ten rounded
    ops, and even that CPU evaluation exceeds the per-op bar on each half of
    the layer (up to 2.8x on the attention half)."""
    import toy_layer_oracle as TL
    from invariant_bi_rmsnorm_amd.toy import Request
    from toy_ref32 import layer_fp32
    prompt = I.toy_prompt(I.TOY, 64)
    T = len(prompt)
    prev = np.ascontiguousarray(toy_weights["embed"][prompt])
    for l in range(1, I.TOY["layers"] + 1):
        cfg = dict(I.TOY, layers=l)
        w = dict(toy_weights, layers=toy_weights["layers"][:l])
        eng = make_engine(w, cfg=cfg, num_blocks=64, max_tokens=T, max_seqs=1, max_kv_len=T)
        eng.step([(Request(0, prompt, 1), T)])
        got = host_bits(eng.hidden_states(T))
        del eng
        lw = toy_weights["layers"][l - 1]
        ref = TL.layer(orc, I.TOY, lw, prev)
        alt = layer_fp32(I.TOY, lw, prev, bf16_weights=True)
        r64 = bf16_f64(ref)
        rms = math.sqrt(float(np.mean(r64 ** 2)))
        drift = np.abs(bf16_f64(alt) - r64)
        err = np.abs(bf16_f64(got) - r64)
        d_rms, e_rms = math.sqrt(float(np.mean(drift ** 2))), math.sqrt(float(np.mean(err ** 2)))
        log(f"layer {l}: gpu rms err {e_rms / rms:.3e}, max {err.max() / rms:.3e} of RMS; CPU evaluation "
            f"{d_rms / rms:.3e}, {drift.max() / rms:.3e}; bit-equal to the oracle: gpu "
            f"{np.mean(got == ref):.3f}, CPU evaluation {np.mean(alt == ref):.3f}")
        assert e_rms <= DEPTH_RMS_RATIO * d_rms, f"layer {l}"
        assert err.max() <= DEPTH_MAX_RATIO * drift.max(), f"layer {l}"
        prev = got


def test_toy_verify_step_logit_rows_match_the_oracle(ops, orc, toy_weights):
    """NEXT row f2's device path (page 5, "la température zéro n'est pas
    déterministe", section on selective determinism): one step feeds k = 8
    drafted tokens after the 64-token prompt with a logit row per token
    (n_logit_rows > S).  Each row is held to the oracle's forward of the same
    prefix (64 + j tokens, j = 0..8) at the end-to-end bar, and where the
    oracle's top-2 margin exceeds twice the row's error the chosen id is the
    oracle's argmax."""
    from invariant_bi_rmsnorm_amd.toy import Request
    eng = make_engine(toy_weights)
    prompt = I.toy_prompt(I.TOY, 64)
    k = 8
    toks, _ = _greedy_alone(eng, prompt, k)          # the drafts: the greedy tokens
    r = Request(1, prompt, 10 ** 6)
    _, lg0 = eng.step([(r, len(prompt))], want_logits=True)
    first = lg0[0].copy()                            # after the prompt (64 tokens)
    r.pending = list(toks[:k])                       # the k drafts as one chunk
    _, _, rows = eng.step([(r, k)], want_logits=True, all_rows=[0])
    L = eng.logits[:k].cpu().numpy()
    L = np.concatenate([L[1:], L[:1]])               # rows after draft 0 .. k-1, in order
    eng.release(r)
    gpu_rows = [first] + [L[j] for j in range(k)]
    ids = [int(np.argmax(first))] + [int(t) for t in rows[0]]
    for j in range(k + 1):
        prefix = np.concatenate([prompt, np.asarray(toks[:j], np.int32)])
        ref = orc.toy_forward(I.TOY, toy_weights, prefix)
        rms = math.sqrt(float(np.mean(ref ** 2)))
        err = np.abs(gpu_rows[j].astype(np.float64) - ref)
        rms_err = math.sqrt(float(np.mean(err ** 2)))
        log(f"verify row {j} (prefix {len(prefix)}): rms err {rms_err / rms:.3e}, max {err.max() / rms:.3e}")
        assert rms_err <= TOY_RMS_BAR * rms, f"row {j}"
        assert err.max() <= TOY_MAX_BAR * rms, f"row {j}"
        top2 = np.sort(ref)[-2:]
        if top2[1] - top2[0] > 2 * err.max():
            assert ids[j] == int(np.argmax(ref)), f"row {j}"


# ------------------------------------------------------------------ invariance

def test_toy_sequence_bits_independent_of_batch(ops, toy_weights):
    """One prompt decoded alone (single-chunk prefill, then decode) vs inside
    mixed batches (random chunking, random co-batched requests, shuffled
    order): every step's logits row is bitwise identical."""
    from invariant_bi_rmsnorm_amd.toy import Request
    prompt = I.toy_prompt(I.TOY, 64)
    n_new = 12
    eng = make_engine(toy_weights)
    r = Request(0, prompt, n_new)
    ref = []
    _, lg = eng.step([(r, 64)], want_logits=True)
    ref.append(lg[0].copy())
    while not r.done:
        _, lg = eng.step([(r, 1)], want_logits=True)
        ref.append(lg[0].copy())
    ref_tokens = list(r.generated)
    eng.release(r)
    g = np.random.default_rng(7)
    for trial in range(3):
        t = Request(100 + trial, prompt, n_new)
        others = [Request(200 + i, g.integers(0, I.TOY["vocab"], int(g.integers(1, 300))).astype(np.int32),
                          int(g.integers(1, 40))) for i in range(int(g.integers(1, 20)))]
        got = []
        step = 0
        while not t.done:
            live = [x for x in others if not x.done]
            dec = [x for x in live + [t] if x.decoding]
            pre = [x for x in live + [t] if not x.decoding]
            g.shuffle(dec)
            g.shuffle(pre)
            work = [(x, 1) for x in dec] + [(x, min(len(x.pending), int(g.integers(1, 48)))) for x in pre]
            _, lg = eng.step(work, want_logits=True)
            i = [w[0] for w in work].index(t)
            if t.length >= len(prompt):            # this step produced a token for t
                got.append(lg[i].copy())
            for x in others:
                if x.done and x.blocks:
                    eng.release(x)
            step += 1
        log(f"toy invariance trial {trial}: {step} steps, {len(others)} co-batched requests")
        assert t.generated == ref_tokens
        assert len(got) == len(ref)
        for a, b in zip(got, ref):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        eng.release(t)
        for x in others:
            eng.release(x)


# ------------------------------------------------------------------ the 1000-run experiment

def test_toy_1000_greedy_runs_collapse_to_one_completion(ops, toy_weights):
    from invariant_bi_rmsnorm_amd.toy import run_load_experiment
    n_runs = int(os.environ.get("BI_TOY_RUNS", "1000"))
    n_new = int(os.environ.get("BI_TOY_NEW", "256"))
    eng = make_engine(toy_weights)
    prompt = I.toy_prompt(I.TOY, 64)
    t = time.time()
    hashes, stats = run_load_experiment(eng, prompt, n_runs, n_new, seed=5002, progress=log)
    uniq = sorted(set(hashes))
    log(f"toy experiment: {n_runs} runs x {n_new} tokens in {time.time() - t:.1f}s, {stats}, "
        f"unique completions: {len(uniq)}")
    assert len(hashes) == n_runs
    assert stats["co_load_max"] >= 32 and stats["co_load_min"] <= 2
    assert len(uniq) == 1


def test_toy_sampled_runs_collapse_to_one_completion(ops, toy_weights):
    """Seeded sampling at T = 0.8 (every run of the prompt uses one seed; other
    requests their own): under random co-batched load the runs still give
    exactly one completion."""
    from invariant_bi_rmsnorm_amd.toy import run_load_experiment
    n_runs = int(os.environ.get("BI_TOY_SAMPLED_RUNS", "300"))
    eng = make_engine(toy_weights)
    prompt = I.toy_prompt(I.TOY, 64)
    t = time.time()
    hashes, stats = run_load_experiment(eng, prompt, n_runs, 64, seed=5003, progress=log, temperature=0.8)
    uniq = sorted(set(hashes))
    log(f"sampled toy experiment (T=0.8): {n_runs} runs x 64 tokens in {time.time() - t:.1f}s, {stats}, "
        f"unique completions: {len(uniq)}")
    assert len(hashes) == n_runs
    assert len(uniq) == 1


# ------------------------------------------------------------------ verify-and-rollback (NEXT row f2)

def _greedy_alone(eng, prompt, n_new):
    """The engine's greedy completion of `prompt` with no other request, and
    the fp32 logits row of every step."""
    from invariant_bi_rmsnorm_amd.toy import Request
    r = Request(0, prompt, n_new)
    work = [(r, len(prompt))]
    lg = []
    while not r.done:
        _, l = eng.step(work, want_logits=True)
        lg.append(l[0].copy())
        work = [(r, 1)]
    eng.release(r)
    return list(r.generated), lg


def test_toy_logit_rows_of_a_chunk_equal_token_by_token_decode(ops, toy_weights):
    """A chunk fed with a logit row per token (n_logit_rows > S) gives, bit for
    bit, the logits and argmax that decoding the same tokens one at a time
    gives: the invariant path can re-check k proposed tokens in one step."""
    from invariant_bi_rmsnorm_amd.toy import Request
    eng = make_engine(toy_weights)
    prompt = I.toy_prompt(I.TOY, 64)
    n = 24
    toks, lg = _greedy_alone(eng, prompt, n)
    r = Request(1, prompt, 10 ** 6)
    eng.step([(r, len(prompt))])                     # the prompt; its argmax is the first token
    assert r.generated[0] == toks[0]
    r.pending = list(toks[:n - 1])                   # then t0 .. t(n-2) as one chunk
    _, _, rows = eng.step([(r, n - 1)], want_logits=True, all_rows=[0])
    R = n - 1
    L = eng.logits[:R].cpu().numpy()
    L = np.concatenate([L[1:], L[:1]])               # the sequence's own (last) row comes first
    eng.release(r)
    assert np.array_equal(rows[0], np.array(toks[1:n]))
    assert np.array_equal(L.view(np.uint32), np.stack(lg[1:n]).view(np.uint32))


def test_toy_verify_rollback_equals_invariant_greedy(ops, toy_weights):
    """NEXT row f2 (verify-and-rollback): the non-invariant build drafts k
    tokens at a time under random co-batched load, the invariant build
    re-checks them with a logit row per token and rolls back at the first
    disagreement.  Every completion equals the invariant engine's own greedy
    completion: once with the drafts as they come, once with every draft at a
    position divisible by 5 corrupted, which forces rollbacks."""
    from invariant_bi_rmsnorm_amd.toy import ToyEngine, run_verify_rollback
    prompt = I.toy_prompt(I.TOY, 64)
    n_new, n_runs = 128, 40
    bi = make_engine(toy_weights)
    ref, _ = _greedy_alone(bi, prompt, n_new)
    prev = ops.use_library(ops.NB_LIB_PATH)
    try:
        nb = ToyEngine.sharing(bi)
    finally:
        ops.use_library(prev)
    V = I.TOY["vocab"]
    cases = (("drafts as decoded", None),
             ("every 5th position corrupted", lambda p, t: (t + 1) % V if p % 5 == 0 else t))
    for name, perturb in cases:
        toks = []
        t = time.time()
        hashes, st = run_verify_rollback(bi, nb, prompt, n_runs, n_new, seed=5010, k=8, tokens_out=toks,
                                         perturb=perturb)
        log(f"verify-rollback ({name}): {n_runs} runs x {n_new} tokens in {time.time() - t:.1f}s, {st}; "
            f"{n_runs * n_new / st['verifies']:.2f} tokens committed per invariant check, "
            f"{st['rollbacks']} of {st['verifies']} checks rolled back")
        assert len(toks) == n_runs
        assert all(tk == ref for tk in toks)
        assert st["drafted"] > 0 and st["verifies"] > 0
        if perturb is not None:
            assert st["rollbacks"] > 0


# ------------------------------------------------------------------ selective fp32 head (NEXT row f3)

def test_toy_selective_fp32_head_keeps_one_completion(ops, toy_weights):
    """With the head recomputed in fp32 for rows whose top-2 margin is below
    0.05, the runs under random co-batched load still give one completion (the
    margin, the choice to recompute and the recomputation are all per row)."""
    from invariant_bi_rmsnorm_amd.toy import run_load_experiment
    eng = make_engine(toy_weights)
    prompt = I.toy_prompt(I.TOY, 64)
    base, _ = _greedy_alone(eng, prompt, 128)
    toks = []
    t = time.time()
    hashes, stats = run_load_experiment(eng, prompt, 100, 128, seed=5020, tokens_out=toks, fp32_head_margin=0.05)
    first = next((i for i, (a, b) in enumerate(zip(toks[0], base)) if a != b), None)
    log(f"selective fp32 head (margin < 0.05): 100 runs x 128 tokens in {time.time() - t:.1f}s, {stats}, "
        f"unique completions {len(set(hashes))}; first token that differs from the bf16-head completion: {first}")
    assert len(hashes) == 100
    assert len(set(hashes)) == 1
