"""GPU tests at the full sizes bench.py times, in the same launch
configuration: paged decode of 256 sequences with log-uniform KV lengths up to
32768 (Hq 32, Hkv 8, D 128, 16-token blocks), and causal prefill of one
8192-token prompt.  The oracle checks sampled rows one by one (all query heads
of a row); everything else is checked by properties that hold at any size:
bitwise invariance under batch composition and order, chunked == single-shot,
and decode at length p+1 == prefill row p.

The caches are drawn on the device with a seeded torch generator (normal,
then rounded to bf16), as bench.py does; the rows the oracle needs are copied
back and passed to it as plain bf16 bits."""
from __future__ import annotations

import math

import numpy as np
import pytest

from gpu_util import check_bf16, dev_bf16, dev_i32, host_bits, log
from invariant_bi_rmsnorm_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SCALE = 1.0 / math.sqrt(128)
HQ, HKV, D, BLK = I.ATT_HQ, I.ATT_HKV, I.ATT_D, I.BLOCK


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from invariant_bi_rmsnorm_amd import ops as o
    o.lib()
    return o


def device_cache(nblk, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    kc = torch.randn((nblk, HKV, BLK, D), generator=gen, device="cuda").to(torch.bfloat16)
    vc = torch.randn((nblk, HKV, D, BLK), generator=gen, device="cuda").to(torch.bfloat16)
    return kc, vc


def poison_tails(kc, vc, table, lens):
    """NaN into the unused slots of every sequence's last block."""
    nan = float("nan")
    for s, L in enumerate(lens):
        r = int(L) % BLK
        if r:
            blk = int(table[s, (int(L) - 1) // BLK])
            kc[blk, :, r:, :] = nan
            vc[blk, :, :, r:] = nan


def logical_kv(kc, vc, table_row, L):
    """K, V of one sequence in logical order, [L, Hkv, D] bf16 bits on the host."""
    nb = -(-L // BLK)
    blocks = torch.from_numpy(np.ascontiguousarray(table_row[:nb]).astype(np.int64)).cuda()
    k = kc[blocks].permute(0, 2, 1, 3).reshape(nb * BLK, HKV, D)[:L]
    v = vc[blocks].permute(0, 3, 1, 2).reshape(nb * BLK, HKV, D)[:L]
    return host_bits(k.contiguous()), host_bits(v.contiguous())


def test_decode_full_size_sampled_parity_and_invariance(ops, orc):
    S = 256
    g = np.random.default_rng([I.TAG_DECODE, 0, 0])
    lens = I.loguniform_lengths(g, S)
    edge = [1, 15, 16, 17, 255, 256, 257, 32767, 32768]
    lens[:len(edge)] = edge
    table, nblk = I.block_tables(g, lens)
    kc, vc = device_cache(nblk, 3000)
    poison_tails(kc, vc, table, lens)
    q = I.queries(I.TAG_DECODE, 0, S)
    tbl = dev_i32(table)
    max_len = int(lens.max())
    log(f"full-size decode: S={S}, {int(lens.sum())} KV tokens, max {max_len}")
    out = host_bits(ops.bi_attention_decode(dev_bf16(q), kc, vc, tbl, dev_i32(lens), max_len, SCALE))

    # oracle on sampled sequences (every query head of each)
    sample = list(range(len(edge))) + sorted(g.choice(np.arange(len(edge), S), 7, replace=False).tolist())
    for s in sample:
        L = int(lens[s])
        k, v = logical_kv(kc, vc, table[s], L)
        _, o64 = orc.attention(q[s][None], [L - 1], k, v, SCALE)
        check_bf16(out[s], o64[0], f"decode s={s} L={L}", axis=None)

    # a sequence alone equals its row in the batch
    for s in (8, int(sample[-1])):
        alone = host_bits(ops.bi_attention_decode(dev_bf16(q[s][None]), kc, vc, dev_i32(table[s][None]),
                                                  dev_i32(lens[s:s + 1]), int(lens[s]), SCALE))
        assert np.array_equal(alone[0], out[s]), f"alone vs batch s={s}"

    # the batch in another order gives the same rows
    perm = g.permutation(S)
    outp = host_bits(ops.bi_attention_decode(dev_bf16(q[perm]), kc, vc, dev_i32(table[perm]),
                                             dev_i32(lens[perm]), max_len, SCALE))
    assert np.array_equal(outp, out[perm])


def test_prefill_full_size_chunked_sampled_parity(ops, orc):
    P = 8192
    g = np.random.default_rng([I.TAG_PREFILL, 0, 0])
    table, nblk = I.block_tables(g, [P])
    kc, vc = device_cache(nblk, 4000)
    q = I.queries(I.TAG_PREFILL, 0, P)
    qd = dev_bf16(q)
    tbl = dev_i32(table)

    def run(start, c):
        return ops.bi_attention_prefill(qd[start:start + c], dev_i32(np.array([0, c], np.int32)),
                                        dev_i32(np.array([start + c], np.int32)), kc, vc, tbl, c, SCALE)

    log("full-size prefill: single shot")
    single = host_bits(run(0, P))
    for sizes in ([2048] * 4, I.chunk_sizes(g, P)):
        log(f"full-size prefill: {len(sizes)} chunks")
        outs, start = [], 0
        for c in sizes:
            outs.append(host_bits(run(start, c)))
            start += c
        assert np.array_equal(np.concatenate(outs), single), f"chunks {sizes}"

    k, v = logical_kv(kc, vc, table[0], P)
    rows = np.array(sorted({0, 1, 255, 256, 257, 511, 4095, 4096, 8191}
                           | set(g.choice(P, 7, replace=False).tolist())), np.int32)
    _, o64 = orc.attention(q[rows], rows, k, v, SCALE)
    check_bf16(single[rows], o64, "prefill sampled rows", axis=-1)

    for p in (255, 4096, 8191):
        d = host_bits(ops.bi_attention_decode(dev_bf16(q[p][None]), kc, vc, tbl,
                                              dev_i32(np.array([p + 1], np.int32)), P, SCALE))
        assert np.array_equal(d[0], single[p]), f"decode vs prefill p={p}"


def test_decode_largest_batch(ops, orc):
    """S = 2048, the largest batch the decode entry point takes (its work list
    prefix lives in LDS): short sequences drawn on the device; sampled rows
    against the oracle and against the same sequence decoded alone, bit for
    bit."""
    S = 2048
    g = np.random.default_rng([I.TAG_DECODE, 9, 0])
    lens = g.integers(1, 300, S).astype(np.int32)
    lens[:4] = [1, 256, 257, 299]
    table, nblk = I.block_tables(g, lens)
    kc, vc = device_cache(nblk, 9000)
    poison_tails(kc, vc, table, lens)
    q = I.queries(I.TAG_DECODE, 9, S)
    log(f"decode S={S}: {int(lens.sum())} KV tokens")
    out = host_bits(ops.bi_attention_decode(dev_bf16(q), kc, vc, dev_i32(table), dev_i32(lens),
                                            int(lens.max()), SCALE))
    for s in (0, 1, 2, 3, 1000, 2047):
        L = int(lens[s])
        alone = host_bits(ops.bi_attention_decode(dev_bf16(q[s][None]), kc, vc, dev_i32(table[s][None]),
                                                  dev_i32(lens[s:s + 1]), L, SCALE))
        assert np.array_equal(alone[0], out[s]), f"alone vs batch s={s}"
        k, v = logical_kv(kc, vc, table[s], L)
        _, o64 = orc.attention(q[s][None], [L - 1], k, v, SCALE)
        check_bf16(out[s], o64[0], f"decode S=2048 s={s} L={L}", axis=None)
