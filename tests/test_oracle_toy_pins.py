"""Pins for the oracle's toy-decoder ops (RoPE, SiLU*mul, residual add) and for
the wiring of its toy forward, from closed forms, exact special cases and
compositions of already-pinned ops.  No GPU."""
from __future__ import annotations

import decimal
import math
from fractions import Fraction

import numpy as np

from exact import CTX, bf16_bits_to_fraction, dec, fraction_to_bf16_bits, near_bf16_tie
from invariant_bi_rmsnorm_amd import inputs as I


def F(b):
    return bf16_bits_to_fraction(int(b))


def bits_of(values):
    out = I.f32_to_bf16(np.asarray(values, dtype=np.float32))
    assert np.all(I.bf16_to_f32(out) == np.asarray(values, dtype=np.float32))
    return out


def small_cfg(**kw):
    c = dict(I.TOY)
    c.update(layers=2, hidden=256, heads=4, kv_heads=2, head_dim=128, mlp=512, vocab=700)
    c.update(kw)
    return c


# ---------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity(orc):
    g = np.random.default_rng(1)
    x = I.normal_bf16(g, (3, 4, 128))
    assert np.array_equal(orc.rope(x, [0, 0, 0]), x)


def test_rope_unit_vectors_closed_form(orc):
    # e_i turns in the plane (i, i+64) by pos * theta^(-2i/128): lands on
    # (cos, sin) there and is exactly zero elsewhere
    D = 128
    for i in (0, 1, 17, 63):
        for p in (1, 7, 1000):
            x = np.zeros((1, 1, D), np.uint16)
            x[0, 0, i] = bits_of([1.0])[0]
            y = orc.rope(x, [p])[0, 0]
            ang = p * 10000.0 ** (-2.0 * i / D)
            for j in range(D):
                if j == i:
                    assert int(y[j]) == fraction_to_bf16_bits(Fraction(math.cos(ang)))
                elif j == i + 64:
                    assert int(y[j]) == fraction_to_bf16_bits(Fraction(math.sin(ang)))
                else:
                    assert (int(y[j]) & 0x7FFF) == 0
            # the partner e_{i+64} goes to (-sin, cos)
            x2 = np.zeros((1, 1, D), np.uint16)
            x2[0, 0, i + 64] = bits_of([1.0])[0]
            y2 = orc.rope(x2, [p])[0, 0]
            assert int(y2[i]) == fraction_to_bf16_bits(Fraction(-math.sin(ang)))
            assert int(y2[i + 64]) == fraction_to_bf16_bits(Fraction(math.cos(ang)))


def test_rope_preserves_pair_norms_and_composes(orc):
    g = np.random.default_rng(2)
    x = I.normal_bf16(g, (1, 2, 128))
    xf = I.bf16_to_f32(x).astype(np.float64)
    y = I.bf16_to_f32(orc.rope(x, [37])).astype(np.float64)
    n0 = xf[..., :64] ** 2 + xf[..., 64:] ** 2
    n1 = y[..., :64] ** 2 + y[..., 64:] ** 2
    assert np.allclose(n0, n1, rtol=2e-2, atol=1e-3)
    # relative positions: <rope(q,p1), rope(k,p2)> depends on p1 - p2 only
    q = I.normal_bf16(g, (1, 1, 128))
    k = I.normal_bf16(g, (1, 1, 128))
    def dot(p1, p2):
        a = I.bf16_to_f32(orc.rope(q, [p1])).astype(np.float64).ravel()
        b = I.bf16_to_f32(orc.rope(k, [p2])).astype(np.float64).ravel()
        return float(a @ b)
    assert abs(dot(10, 3) - dot(107, 100)) < 0.05 * (1 + abs(dot(10, 3)))


# ---------------------------------------------------------------- SiLU * mul, add

def test_silu_mul_closed_forms(orc):
    g = bits_of([0.0, 2.0, -2.0, 1.0, -30.0, 8.0])
    u = bits_of([5.0, 1.0, 1.0, -3.0, 1.0, 0.5])
    out = orc.silu_mul(g, u)
    for gi, ui, oi in zip(g, u, out):
        gv, uv = F(gi), F(ui)
        e = CTX.exp(dec(-gv))
        exact = Fraction(CTX.divide(dec(gv), decimal.Decimal(1) + e)) * uv
        if not near_bf16_tie(exact, 1e-12):
            assert int(oi) == fraction_to_bf16_bits(exact)
    # silu(x) - silu(-x) = x
    x = I.normal_bf16(np.random.default_rng(3), (50,))
    ones = bits_of([1.0] * 50)
    a = I.bf16_to_f32(orc.silu_mul(x, ones)).astype(np.float64)
    b = I.bf16_to_f32(orc.silu_mul(x ^ np.uint16(0x8000), ones)).astype(np.float64)
    assert np.allclose(a - b, I.bf16_to_f32(x), rtol=1e-2, atol=1e-2)


def test_add_exact_and_rounded(orc):
    a = bits_of([1.0, 0.5, -3.0, 256.0, 1.0])
    b = bits_of([2.0, 0.25, 3.0, 1.0, 2.0 ** -9])
    out = orc.add(a, b)
    assert [int(v) for v in out] == [fraction_to_bf16_bits(F(x) + F(y)) for x, y in zip(a, b)]
    assert int(out[3]) == int(bits_of([256.0])[0])      # 257 rounds to even (256)
    assert (int(out[2]) & 0x7FFF) == 0


# ---------------------------------------------------------------- toy forward wiring

def test_toy_forward_without_blocks_is_norm_then_head(orc):
    # Wo = Wd = 0: the residual stream stays the embedding, so the logits are
    # final_norm(embed[last]) @ lm_head^T, a composition of pinned ops
    cfg = small_cfg()
    w = I.toy_weights(cfg)
    for lw in w["layers"]:
        lw["wo"][:] = 0
        lw["wd"][:] = 0
    ids = I.toy_prompt(cfg, 9)
    got = orc.toy_forward(cfg, w, ids)
    xn, _ = orc.rmsnorm(w["embed"][ids[-1:]], w["final_norm"], cfg["eps"])
    want = orc.matmul_f64(xn, w["lm_head"])[0]
    assert np.array_equal(got, want)


def test_toy_forward_single_token_attention_is_value_projection(orc):
    # one token, one layer, Wd = 0: attention over a single key returns v, so
    # h = embed + (v @ Wo^T) with v = rmsnorm(embed) @ Wv^T
    cfg = small_cfg(layers=1)
    w = I.toy_weights(cfg)
    w["layers"][0]["wd"][:] = 0
    ids = np.array([123], np.int32)
    got = orc.toy_forward(cfg, w, ids)
    lw = w["layers"][0]
    D, Hq, Hkv = cfg["head_dim"], cfg["heads"], cfg["kv_heads"]
    e = w["embed"][ids]
    xn, _ = orc.rmsnorm(e, lw["attn_norm"], cfg["eps"])
    v = orc.matmul(xn, lw["wqkv"][(Hq + Hkv) * D:])                      # [1, Hkv*D]
    attn = np.concatenate([v[:, (h // (Hq // Hkv)) * D:(h // (Hq // Hkv) + 1) * D] for h in range(Hq)], axis=1)
    o = orc.matmul(attn, lw["wo"])
    h = orc.add(e, o)
    xf, _ = orc.rmsnorm(h, w["final_norm"], cfg["eps"])
    want = orc.matmul_f64(xf, w["lm_head"])[0]
    assert np.array_equal(got, want)


def test_toy_forward_is_causal_and_deterministic(orc):
    cfg = small_cfg()
    w = I.toy_weights(cfg)
    ids = I.toy_prompt(cfg, 12)
    a = orc.toy_forward(cfg, w, ids)
    b = orc.toy_forward(cfg, w, ids)
    assert np.array_equal(a, b)
    c = orc.toy_forward(cfg, w, np.concatenate([ids[:6], (ids[6:] + 1) % cfg["vocab"]]))
    assert not np.array_equal(a, c)           # later tokens do matter for the last position
