"""GPU tests of the paged KV append, decode attention (fixed 256-token splits)
and causal prefill attention: parity against the CPU oracle, and bitwise
invariance under batch composition, row position, block placement, chunking,
and decode vs prefill."""
from __future__ import annotations

import math

import numpy as np
import pytest

from gpu_util import (PagedCache, check_bf16, dev_bf16, dev_i32, host_bits, log, make_cache)
from invariant_bi_rmsnorm_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SCALE = 1.0 / math.sqrt(128)
HQ, HKV, D = I.ATT_HQ, I.ATT_HKV, I.ATT_D


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from invariant_bi_rmsnorm_amd import ops as o
    o.lib()
    return o


def decode(ops, cache, table, q_bits, lens, max_len=None):
    max_len = max_len or int(max(lens))
    out = ops.bi_attention_decode(dev_bf16(q_bits), cache.k, cache.v, dev_i32(table),
                                  dev_i32(lens), max_len, SCALE)
    return host_bits(out)


def prefill(ops, cache, table, q_bits, q_start, kv_lens):
    tq = np.diff(q_start)
    out = ops.bi_attention_prefill(dev_bf16(q_bits), dev_i32(q_start), dev_i32(kv_lens), cache.k,
                                   cache.v, dev_i32(table), int(tq.max()), SCALE)
    return host_bits(out)


# ------------------------------------------------------------------ append

@pytest.mark.parametrize("Hkv", [4, 12])
def test_kv_append_bitwise_layout(ops, Hkv):
    g = np.random.default_rng(Hkv)
    T, nblk = 50, 10
    qkv = I.normal_bf16(g, (T, (16 + 2 * Hkv) * D))       # a fused projection output
    k = qkv[:, 16 * D:(16 + Hkv) * D].reshape(T, Hkv, D)
    v = qkv[:, (16 + Hkv) * D:].reshape(T, Hkv, D)
    slots = g.permutation(nblk * 16)[:T].astype(np.int32)
    slots[7] = -1
    slots[9] = nblk * 16 + 3                               # out of range: skipped
    cache = PagedCache(nblk, Hkv)
    qd = dev_bf16(qkv).view(T, 16 + 2 * Hkv, D)
    ops.bi_kv_append(qd[:, 16:16 + Hkv], qd[:, 16 + Hkv:], dev_i32(slots), cache.k, cache.v)
    kc = host_bits(cache.k)
    vc = host_bits(cache.v)
    ek = np.full((nblk, Hkv, 16, D), 0x7FC0, np.uint16)
    ev = np.full((nblk, Hkv, D, 16), 0x7FC0, np.uint16)
    for t in range(T):
        s = int(slots[t])
        if 0 <= s < nblk * 16:
            ek[s // 16, :, s % 16, :] = k[t]
            ev[s // 16, :, :, s % 16] = v[t]
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)


# ------------------------------------------------------------------ decode

def oracle_decode(orc, q, k, v):
    L = k.shape[0]
    o16, o64 = orc.attention(q[None], [L - 1], k, v, SCALE)
    return o16[0], o64[0]


@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 4), (8, 8), (32, 2), (16, 8), (32, 4)])
def test_decode_parity_edge_lengths(ops, orc, hq, hkv):
    g = np.random.default_rng(hq * 10 + hkv)
    lens = np.array([1, 15, 16, 17, 255, 256, 257, 511, 1000, 2049, 4097], np.int32)
    log(f"decode parity Hq={hq} Hkv={hkv}")
    kvs = [I.kv_sequence(I.TAG_DECODE, 50 + hq + hkv, s, int(L), hkv) for s, L in enumerate(lens)]
    cache, table = make_cache(g, kvs, Hkv=hkv)
    q = I.queries(I.TAG_DECODE, 50 + hq + hkv, len(lens), hq)
    out = decode(ops, cache, table, q, lens)
    for s, (k, v) in enumerate(kvs):
        o16, o64 = oracle_decode(orc, q[s], k, v)
        check_bf16(out[s], o64, f"decode s={s} L={lens[s]}", axis=None)
        if lens[s] == 1:
            assert np.array_equal(out[s], v[0][np.arange(hq) // (hq // hkv)])   # single key: v itself


def test_decode_batch_invariance_and_block_placement(ops):
    g = np.random.default_rng(2)
    L_t = 3001
    kt, vt = I.kv_sequence(I.TAG_DECODE, 2, 999, L_t)
    qt = I.queries(I.TAG_DECODE, 2, 1)[0]
    # alone
    cache1, table1 = make_cache(g, [(kt, vt)])
    alone = decode(ops, cache1, table1, qt[None], np.array([L_t], np.int32))[0]
    for trial in range(4):
        S = int(g.integers(2, 64))
        pos = int(g.integers(0, S))
        lens = I.loguniform_lengths(g, S, 8192)
        lens[pos] = L_t
        kvs = [I.kv_sequence(I.TAG_DECODE, 20 + trial, s, int(L)) for s, L in enumerate(lens)]
        kvs[pos] = (kt, vt)
        q = I.queries(I.TAG_DECODE, 20 + trial, S)
        q[pos] = qt
        max_len = int(g.integers(max(L_t, int(lens.max())), 9000))
        caps = [int(L) for L in lens]
        caps[pos] = max_len                       # reserved but unused blocks for the target
        cache, table = make_cache(g, kvs, capacities=caps, extra_blocks=int(g.integers(0, 50)))
        out = decode(ops, cache, table, q, lens, max_len=max_len)
        log(f"decode invariance trial={trial} S={S} pos={pos}")
        assert np.array_equal(out[pos], alone)


def test_decode_repeat_bitwise(ops):
    g = np.random.default_rng(3)
    lens = I.loguniform_lengths(g, 24, 20000)
    kvs = [I.kv_sequence(I.TAG_DECODE, 3, s, int(L)) for s, L in enumerate(lens)]
    cache, table = make_cache(g, kvs)
    q = I.queries(I.TAG_DECODE, 3, 24)
    o0 = decode(ops, cache, table, q, lens)
    for _ in range(4):
        assert np.array_equal(decode(ops, cache, table, q, lens), o0)


# ------------------------------------------------------------------ prefill

@pytest.mark.parametrize("hq,hkv,P0,T", [(32, 8, 0, 700), (32, 8, 300, 513), (16, 4, 0, 300),
                                         (8, 8, 1000, 77), (32, 2, 5, 260), (16, 8, 40, 333),
                                         (32, 4, 257, 129)])
def test_prefill_parity(ops, orc, hq, hkv, P0, T):
    log(f"prefill parity Hq={hq} Hkv={hkv} P0={P0} T={T}")
    g = np.random.default_rng(P0 + T)
    L = P0 + T
    k, v = I.kv_sequence(I.TAG_PREFILL, 1, hq + P0, L, hkv)
    cache, table = make_cache(g, [(k, v)], Hkv=hkv)
    q = I.queries(I.TAG_PREFILL, 1 + P0, T, hq)
    out = prefill(ops, cache, table, q, np.array([0, T], np.int32), np.array([L], np.int32))
    o16, o64 = orc.attention(q, np.arange(P0, L), k, v, SCALE)
    check_bf16(out, o64, "prefill", axis=-1)


def test_prefill_chunked_equals_single_shot_and_decode(ops):
    g = np.random.default_rng(4)
    P = 3001
    k, v = I.kv_sequence(I.TAG_PREFILL, 4, 0, P)
    q = I.queries(I.TAG_PREFILL, 4, P)
    # single shot
    cache, table = make_cache(g, [(k, v)])
    single = prefill(ops, cache, table, q, np.array([0, P], np.int32), np.array([P], np.int32))
    for trial, sizes in enumerate([I.chunk_sizes(g, P), I.chunk_sizes(g, P, 1, 300), [1] * 5 + [P - 5]]):
        log(f"chunked trial={trial} chunks={len(sizes)}")
        table_c, nblk = I.block_tables(g, [P], int(g.integers(190, 260)))
        cc = PagedCache(nblk, HKV)
        outs = []
        start = 0
        for c in sizes:
            slots = I.slots_for(table_c[0], np.arange(start, start + c))
            cc.append(k[start:start + c], v[start:start + c], slots)       # append, then attend
            outs.append(prefill(ops, cc, table_c, q[start:start + c], np.array([0, c], np.int32),
                                np.array([start + c], np.int32)))
            start += c
        assert np.array_equal(np.concatenate(outs), single), f"trial {trial}"
    # decode at length p+1 equals prefill row p
    for p in (0, 15, 255, 256, 511, 1000, 2999, 3000):
        d = decode(ops, cache, table, q[p][None], np.array([p + 1], np.int32), max_len=P)
        assert np.array_equal(d[0], single[p]), f"decode vs prefill p={p}"


def test_prefill_varlen_batch_invariance(ops):
    g = np.random.default_rng(5)
    S = 6
    P0 = np.array([0, 40, 300, 0, 1000, 17], np.int32)
    T = np.array([300, 1, 257, 64, 33, 700], np.int32)
    L = P0 + T
    kvs = [I.kv_sequence(I.TAG_PREFILL, 5, s, int(l)) for s, l in enumerate(L)]
    qs = [I.queries(I.TAG_PREFILL, 50 + s, int(t)) for s, t in enumerate(T)]
    cache, table = make_cache(g, kvs)
    q_start = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    batch = prefill(ops, cache, table, np.concatenate(qs), q_start, L)
    for s in range(S):
        cache1, table1 = make_cache(g, [kvs[s]])
        alone = prefill(ops, cache1, table1, qs[s], np.array([0, T[s]], np.int32), L[s:s + 1])
        assert np.array_equal(batch[q_start[s]:q_start[s + 1]], alone), f"s={s}"


def test_decode_empty_sequences_and_one_split_calls(ops):
    """Sequences with no token (kv_len 0 or negative) get a zero output, and a
    call whose max_kv_len fits one split (the combine kernel is not launched)
    gives the same bits as the same work with a larger max_kv_len (combine
    launched, every sequence still one split), and as each sequence alone."""
    g = np.random.default_rng(21)
    lens = np.array([0, 5, 0, 200, -3], np.int32)
    kvs = [I.kv_sequence(I.TAG_DECODE, 21, s, max(1, int(l))) for s, l in enumerate(lens)]
    cache, table = make_cache(g, kvs, capacities=[300] * len(lens))
    q = I.queries(I.TAG_DECODE, 21, len(lens))
    outs = []
    for max_len in (200, 300):
        log(f"decode empty sequences max_kv_len={max_len}")
        out = torch.full((len(lens), HQ, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        ops.bi_attention_decode(dev_bf16(q), cache.k, cache.v, dev_i32(table), dev_i32(lens), max_len, SCALE,
                                out=out)
        outs.append(host_bits(out))
    assert np.array_equal(outs[0], outs[1])
    for s in (0, 2, 4):
        assert np.all(outs[0][s] == 0), f"sequence {s} (no token) must be zero"
    for s in (1, 3):
        alone = decode(ops, cache, table[s:s + 1], q[s:s + 1], lens[s:s + 1])
        assert np.array_equal(outs[0][s], alone[0]), f"s={s}"


def test_decode_long_sequences_fold_over_chunks(ops, orc):
    """Sequences longer than 128 splits (the combine folds them 128 at a time):
    decode equals the prefill row at the same length bit for bit, and matches
    the oracle."""
    g = np.random.default_rng(6)
    for L in (32769, 40000):
        log(f"long decode L={L}")
        k, v = I.kv_sequence(I.TAG_DECODE, 6, L, L)
        q = I.queries(I.TAG_DECODE, 6 + L, 1)
        cache, table = make_cache(g, [(k, v)])
        d = decode(ops, cache, table, q, np.array([L], np.int32))
        p = prefill(ops, cache, table, q, np.array([0, 1], np.int32), np.array([L], np.int32))
        assert np.array_equal(d[0], p[0])
        o16, o64 = oracle_decode(orc, q[0], k, v)
        check_bf16(d[0], o64, f"decode L={L}", axis=None)


def test_invalid_block_ids_are_masked_in_decode_and_prefill(ops, orc):
    """A block-table entry outside [0, num_blocks) names no cache block: its 16
    tokens take no part in the attention (score -inf, value 0), in decode and
    in prefill alike.  The result is the oracle's over the remaining keys, does
    not depend on what else shares the call (nothing stale reaches it), and
    decode at length p + 1 equals prefill row p bit for bit."""
    g = np.random.default_rng(8)
    L = 1000
    k, v = I.kv_sequence(I.TAG_DECODE, 8, 0, L)
    q = I.queries(I.TAG_DECODE, 8, L)
    cache, table = make_cache(g, [(k, v)], extra_blocks=8)
    nblk = cache.num_blocks
    bad_blocks = [20] + list(range(32, 48)) + [55]        # one block, one whole split, one more
    table = table.copy()
    table[0, 20] = nblk + 5
    table[0, 32:48] = nblk + 1000
    table[0, 55] = -7
    keep = np.ones(L, bool)
    for b in bad_blocks:
        keep[16 * b:16 * b + 16] = False
    # decode of the last row: the oracle over the keys that remain
    d_alone = decode(ops, cache, table, q[L - 1][None], np.array([L], np.int32))[0]
    o16, o64 = oracle_decode(orc, q[L - 1], k[keep], v[keep])
    check_bf16(d_alone, o64, "decode with invalid block ids", axis=None)
    # the same row beside other sequences (other items run before it on the same workgroups)
    S = 40
    lens = I.loguniform_lengths(g, S, 6000)
    pos = 17
    lens[pos] = L
    kvs = [I.kv_sequence(I.TAG_DECODE, 9, s, int(Ls)) for s, Ls in enumerate(lens)]
    kvs[pos] = (k, v)
    cache_b, table_b = make_cache(g, kvs)
    tb = table_b.copy()
    tb[pos, 20] = cache_b.num_blocks + 5
    tb[pos, 32:48] = cache_b.num_blocks + 1000
    tb[pos, 55] = -7
    qb = I.queries(I.TAG_DECODE, 9, S)
    qb[pos] = q[L - 1]
    d_batch = decode(ops, cache_b, tb, qb, lens)
    assert np.array_equal(d_batch[pos], d_alone)
    # prefill over the same table: every row equals decode at its length
    pre = prefill(ops, cache, table, q, np.array([0, L], np.int32), np.array([L], np.int32))
    assert np.array_equal(pre[L - 1], d_alone)
    for p in (0, 300, 319, 320, 335, 336, 511, 512, 600, 767, 768, 880, 890, 999):
        dp = decode(ops, cache, table, q[p][None], np.array([p + 1], np.int32), max_len=L)
        assert np.array_equal(dp[0], pre[p]), f"decode vs prefill p={p}"


@pytest.mark.parametrize("scale", [-1.0 / math.sqrt(128), 0.0, 4.0 / math.sqrt(128)])
def test_scale_sign_and_zero(ops, orc, scale):
    """Any scale: a negative one enters as negated queries with |scale| (exact),
    a zero one gives uniform weights.  Parity with the oracle at that scale, and
    decode at length p + 1 equals prefill row p bit for bit."""
    log(f"scale {scale}")
    g = np.random.default_rng(91)
    P0, T = 500, 200
    L = P0 + T
    k, v = I.kv_sequence(I.TAG_PREFILL, 9, 0, L)
    cache, table = make_cache(g, [(k, v)])
    q = I.queries(I.TAG_PREFILL, 9, T)
    out = host_bits(ops.bi_attention_prefill(dev_bf16(q), dev_i32(np.array([0, T], np.int32)),
                                             dev_i32(np.array([L], np.int32)), cache.k, cache.v,
                                             dev_i32(table), T, scale))
    o16, o64 = orc.attention(q, np.arange(P0, L), k, v, scale)
    check_bf16(out, o64, f"prefill scale={scale}", axis=-1)
    for r in (0, 99, 199):
        d = host_bits(ops.bi_attention_decode(dev_bf16(q[r][None]), cache.k, cache.v, dev_i32(table),
                                              dev_i32(np.array([P0 + r + 1], np.int32)), L, scale))
        assert np.array_equal(d[0], out[r]), f"decode vs prefill row {r} scale={scale}"
