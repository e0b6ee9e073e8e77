"""bi_attention_decode_noalloc (the allocation-free decode: split partials in
the library's own scratch array) against bi_attention_decode (caller
workspace) on the same inputs: the two run the same kernels, so the outputs
must be bitwise equal.  Two calls in a row, the second smaller, so the second
call runs over what the first left in the shared scratch."""
from __future__ import annotations

import math

import numpy as np
import pytest

from gpu_util import dev_i32, host_bits, log, make_cache
from invariant_bi_rmsnorm_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SCALE = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from invariant_bi_rmsnorm_amd import ops as o
    o.lib()
    return o


def _case(seed, S, max_len, Hq=32, Hkv=8):
    g = np.random.default_rng(seed)
    lens = I.loguniform_lengths(g, S, max_len)
    lens[0] = max_len
    kvs = [I.kv_sequence(I.TAG_DECODE, seed, s, int(L), Hkv) for s, L in enumerate(lens)]
    cache, table = make_cache(g, kvs, Hkv=Hkv)
    q = I.queries(I.TAG_DECODE, seed, S, Hq)
    return lens, cache, table, q


def _both(ops, lens, cache, table, q_bits, max_len):
    from gpu_util import dev_bf16
    q = dev_bf16(q_bits)
    tbl, kl = dev_i32(table), dev_i32(lens)
    ref = ops.bi_attention_decode(q, cache.k, cache.v, tbl, kl, max_len, SCALE)
    out = torch.full_like(ref, float("nan"))
    ops.bi_attention_decode_noalloc(q, cache.k, cache.v, tbl, kl, max_len, SCALE, out=out)
    return host_bits(ref), host_bits(out)


def test_noalloc_decode_equals_workspace_decode_on_two_calls(ops):
    # first call: 48 sequences up to 8192 tokens (48 * 32 * 32 split partials, 31.5 MB of scratch)
    lens, cache, table, q = _case(71, 48, 8192)
    log(f"noalloc call 1: S=48 max_len=8192 ws={ops.bi_attention_workspace_bytes(48, 32, 128, 8192)}")
    ref, out = _both(ops, lens, cache, table, q, 8192)
    assert np.array_equal(out, ref)
    # second call, smaller (5 sequences up to 600 tokens, GQA 16/4): runs over the first call's partials
    lens2, cache2, table2, q2 = _case(72, 5, 600, Hq=16, Hkv=4)
    log("noalloc call 2: S=5 max_len=600 Hq=16 Hkv=4")
    ref2, out2 = _both(ops, lens2, cache2, table2, q2, 600)
    assert np.array_equal(out2, ref2)
    # the largest call the scratch holds: S * Hq * splits = 102 * 32 * 32 = 104448 <= 104856
    lens3, cache3, table3, q3 = _case(73, 102, 8192)
    assert ops.bi_attention_workspace_bytes(102, 32, 128, 8192) <= ops.NOALLOC_SCRATCH_BYTES
    assert ops.bi_attention_workspace_bytes(103, 32, 128, 8192) > ops.NOALLOC_SCRATCH_BYTES
    log("noalloc call 3: S=102 max_len=8192 (scratch nearly full)")
    ref3, out3 = _both(ops, lens3, cache3, table3, q3, 8192)
    assert np.array_equal(out3, ref3)


def test_noalloc_decode_rejects_more_than_its_scratch(ops):
    lens, cache, table, q = _case(74, 4, 300)
    from gpu_util import dev_bf16
    out = torch.empty((4, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ops.BiError) as e:
        # max_kv_len 2**20 with 4 sequences: 4 * 32 * 4096 partials, above 64 MiB
        tbl = dev_i32(np.zeros((4, 65536), np.int32))
        ops.bi_attention_decode_noalloc(dev_bf16(q), cache.k, cache.v, tbl, dev_i32(lens), 1 << 20, SCALE,
                                        out=out)
    assert e.value.status == ops.BI_ERR_WORKSPACE_TOO_SMALL
