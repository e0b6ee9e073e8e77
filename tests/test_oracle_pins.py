"""Pins for the CPU oracle: closed forms, exact special cases, invariants and
brute force on tiny inputs.  Each check is chosen so that a plausible mistake
in the oracle (dropped term, wrong sign or index, transposed operand, wrong
rounding rule, H-1 instead of H, eps outside the root, missing scale, wrong
GQA group) fails at least one of them.

No GPU; runs in a few seconds.
"""
from __future__ import annotations

import decimal
import math
import os
import subprocess
import sys
from fractions import Fraction

import numpy as np
import pytest

from exact import (CTX, bf16_bits_to_fraction, dec, fraction_to_bf16_bits,
                   near_bf16_tie)
from invariant_bi_rmsnorm_amd import inputs as I


def F(b):
    return bf16_bits_to_fraction(int(b))


def bits_of(values):
    """Exact small doubles -> bf16 bits (values must be bf16-representable)."""
    out = I.f32_to_bf16(np.asarray(values, dtype=np.float32))
    assert np.all(I.bf16_to_f32(out) == np.asarray(values, dtype=np.float32))
    return out


# ---------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_exact_rational_rounding(orc):
    g = np.random.default_rng(11)
    # random doubles over many binades, plus exact ties and near-ties
    x = g.standard_normal(4000) * np.exp2(g.integers(-140, 127, 4000))
    base = I.bf16_to_f32(g.integers(0, 0x7F7F, 500).astype(np.uint16)).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.abs(base) + 1e-300)) - 7)
    ties = base + ulp / 2
    near = np.concatenate([ties * (1 + 1e-15), ties * (1 - 1e-15)])
    x = np.concatenate([x, ties, near, -ties])
    x = x[np.isfinite(x) & (x != 0)]
    got = orc.round_bf16(x)
    for xi, gi in zip(x, got):
        assert int(gi) == fraction_to_bf16_bits(Fraction(float(xi))), xi


def test_round_bf16_special_values(orc):
    got = orc.round_bf16([0.0, -0.0, math.inf, -math.inf, math.nan,
                          3.4e38, -3.4e38, 1e-45, 2.0 ** -133, 1.0 + 2.0 ** -8,
                          1.0 + 3 * 2.0 ** -9])
    assert list(got[:4]) == [0x0000, 0x8000, 0x7F80, 0xFF80]
    assert (int(got[4]) & 0x7F80) == 0x7F80 and (int(got[4]) & 0x7F) != 0   # NaN
    assert int(got[5]) == 0x7F80 and int(got[6]) == 0xFF80                # overflow
    assert int(got[7]) == 0 and int(got[8]) == 1                          # subnormal
    assert int(got[9]) == 0x3F80                                          # tie -> even
    assert int(got[10]) == 0x3F81                                         # above tie


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_row_eps0_returns_weight(orc):
    H = 64
    g = np.random.default_rng(1)
    w = I.normal_bf16(g, (H,), 1.0, 0.1)
    for c in (0.5, -2.0, 8.0, -0.125):
        x = np.tile(bits_of([c]), (1, H))
        y, r = orc.rmsnorm(x, w, 0.0)
        wneg = w ^ np.uint16(0x8000) if c < 0 else w
        assert np.array_equal(y[0], wneg)            # y = sign(c) * w exactly
        assert r[0] == np.float32(1.0 / abs(c))      # rstd = 1/|c| exactly


def test_rmsnorm_one_hot_divides_by_H(orc):
    # x = a e_j, eps = 0: mean square = a^2/H -> rstd = sqrt(H)/|a| = 16/|a| for H=256
    H = 256
    g = np.random.default_rng(2)
    w = I.normal_bf16(g, (H,), 1.0, 0.1)
    for a, j in ((2.0, 0), (-0.5, 37), (4.0, 255)):
        x = np.zeros((1, H), dtype=np.uint16)
        x[0, j] = bits_of([a])[0]
        y, r = orc.rmsnorm(x, w, 0.0)
        assert r[0] == np.float32(16.0 / abs(a))
        expect = fraction_to_bf16_bits(Fraction(16) * (1 if a > 0 else -1) * F(w[j]))
        assert int(y[0, j]) == expect
        others = np.delete(y[0], j)
        assert np.all((others & 0x7FFF) == 0)         # exactly zero elsewhere


def test_rmsnorm_eps_inside_root(orc):
    # x = 0 row, eps = 1/4 -> rstd = 2 exactly; y = 0
    H = 8
    w = bits_of([1.0] * H)
    y, r = orc.rmsnorm(np.zeros((1, H), np.uint16), w, 0.25)
    assert r[0] == 2.0 and np.all((y & 0x7FFF) == 0)
    # x = 0.75 constant (mean square 9/16), eps = 7/16 -> rstd = 1 exactly -> y = x * w
    x = np.tile(bits_of([0.75]), (1, H))
    w = bits_of([1.0, -1.5, 2.0, 0.25, 3.0, -0.5, 1.25, 1.0])
    y, r = orc.rmsnorm(x, w, 7.0 / 16.0)
    assert r[0] == 1.0
    assert [int(b) for b in y[0]] == [fraction_to_bf16_bits(Fraction(3, 4) * F(b)) for b in w]


def test_rmsnorm_H1_closed_form(orc):
    for xv, wv, eps in ((3.0, 0.5, 16.0), (-0.75, 2.0, 0.4375)):
        y, r = orc.rmsnorm(bits_of([[xv]]), bits_of([wv]), eps)
        # rstd = 1/sqrt(x^2 + eps): chosen so x^2 + eps is a perfect square
        root = math.sqrt(xv * xv + eps)
        assert root == int(root) or root * 4 == int(root * 4)
        assert r[0] == np.float32(1.0 / root)
        assert int(y[0, 0]) == fraction_to_bf16_bits(Fraction(xv) * Fraction(wv) / Fraction(root))


def test_rmsnorm_scale_invariance_eps0(orc):
    g = np.random.default_rng(3)
    x = I.normal_bf16(g, (5, 96))
    w = I.normal_bf16(g, (96,), 1.0, 0.1)
    y0, r0 = orc.rmsnorm(x, w, 0.0)
    for k in (-3, 5):
        xs = I.f32_to_bf16(I.bf16_to_f32(x) * np.float32(2.0 ** k))
        y1, r1 = orc.rmsnorm(xs, w, 0.0)
        assert np.array_equal(y0, y1)
        assert np.allclose(r1, r0 * 2.0 ** -k, rtol=1e-7, atol=0)


def test_rmsnorm_brute_force_decimal(orc):
    g = np.random.default_rng(4)
    for H in (1, 3, 7, 16):
        x = I.normal_bf16(g, (3, H))
        w = I.normal_bf16(g, (H,), 1.0, 0.1)
        eps = 1e-6
        y, r = orc.rmsnorm(x, w, eps)
        y64, r64 = orc.rmsnorm_f64(x, w, eps)
        for m in range(3):
            ss = sum(F(b) * F(b) for b in x[m])
            ms = ss / H + Fraction(eps)
            rstd = CTX.divide(decimal.Decimal(1), CTX.sqrt(dec(ms)))
            assert abs(float(rstd) - r64[m]) <= 2e-16 * float(rstd)
            assert r[m] == np.float32(float(rstd))
            for j in range(H):
                exact = F(x[m, j]) * F(w[j]) * Fraction(rstd)
                if not near_bf16_tie(exact, 1e-10):
                    assert int(y[m, j]) == fraction_to_bf16_bits(exact)
                assert abs(y64[m, j] - float(exact)) <= 1e-15 * abs(float(exact)) + 1e-300


def test_rmsnorm_rows_independent_and_weight_multiplies(orc):
    g = np.random.default_rng(5)
    x = I.normal_bf16(g, (6, 32))
    w = I.normal_bf16(g, (32,), 1.0, 0.1)
    y, r = orc.rmsnorm(x, w, 1e-6)
    for m in range(6):
        y1, r1 = orc.rmsnorm(x[m:m + 1], w, 1e-6)
        assert np.array_equal(y1[0], y[m]) and r1[0] == r[m]
    yz, _ = orc.rmsnorm(x, np.zeros(32, np.uint16), 1e-6)   # w = 0 -> y = 0 (not 1+w)
    assert np.all((yz & 0x7FFF) == 0)


# ---------------------------------------------------------------- matmul

def test_matmul_small_integers_exact(orc):
    g = np.random.default_rng(6)
    M, N, K = 7, 40, 512
    A = g.integers(-4, 5, (M, K))
    W = g.integers(-4, 5, (K, N))            # logical [K,N]
    a = bits_of(A.astype(np.float32))
    wt = bits_of(W.T.astype(np.float32))     # stored [N,K]
    exact = A @ W                            # int64, independent library product
    c32 = orc.matmul(a, wt, out="f32")
    assert np.array_equal(c32.astype(np.int64), exact)
    c16 = orc.matmul(a, wt, out="bf16")
    for (m, n), v in np.ndenumerate(exact):
        assert int(c16[m, n]) == fraction_to_bf16_bits(Fraction(int(v)))


def test_matmul_permutation_weight(orc):
    g = np.random.default_rng(7)
    K = 24
    a = I.normal_bf16(g, (5, K))
    perm = g.permutation(K)
    W = np.zeros((K, K), np.float32)
    W[perm, np.arange(K)] = 1.0               # C[:, n] = A[:, perm[n]]
    c = orc.matmul(a, bits_of(W.T), out="bf16")
    assert np.array_equal(c, a[:, perm])


def test_matmul_rank_one(orc):
    for K in (64, 4096):
        a = np.tile(bits_of([0.5]), (3, K))
        wt = np.tile(bits_of([-0.25]), (5, K))
        c = orc.matmul(a, wt, out="f32")
        assert np.all(c == np.float32(-0.125 * K))


def test_matmul_brute_force_fractions(orc):
    g = np.random.default_rng(8)
    for (M, N, K) in ((1, 1, 1), (2, 3, 5), (4, 8, 8), (3, 2, 7)):
        a = I.normal_bf16(g, (M, K))
        wt = I.normal_bf16(g, (N, K), 0.0, 0.05)
        c16 = orc.matmul(a, wt, out="bf16")
        c64 = orc.matmul_f64(a, wt)
        for m in range(M):
            for n in range(N):
                exact = sum(F(a[m, k]) * F(wt[n, k]) for k in range(K))
                assert c64[m, n] == float(exact)    # exact: few bf16 products fit in a double
                assert int(c16[m, n]) == fraction_to_bf16_bits(exact)


def test_matmul_non_square_orientation(orc):
    # wt is [N,K]; a transposed operand or swapped index cannot pass this
    g = np.random.default_rng(9)
    A = g.integers(-3, 4, (3, 5))
    W = g.integers(-3, 4, (5, 2))
    c = orc.matmul(bits_of(A.astype(np.float32)), bits_of(W.T.astype(np.float32)), out="f32")
    assert c.shape == (3, 2)
    assert np.array_equal(c.astype(np.int64), A @ W)


# ---------------------------------------------------------------- attention

def _rand_att(g, T, L, Hq, Hkv, D):
    q = I.normal_bf16(g, (T, Hq, D))
    k = I.normal_bf16(g, (L, Hkv, D))
    v = I.normal_bf16(g, (L, Hkv, D))
    return q, k, v


def test_attention_single_key_returns_value(orc):
    g = np.random.default_rng(10)
    q, k, v = _rand_att(g, 1, 1, 4, 2, 16)
    o16, o64 = orc.attention(q, [0], k, v, 1 / math.sqrt(16))
    for h in range(4):
        assert np.array_equal(o16[0, h], v[0, h // 2])


def test_attention_zero_query_is_mean_of_visible_values(orc):
    g = np.random.default_rng(11)
    L, D = 9, 8
    q = np.zeros((3, 2, D), np.uint16)
    _, k, v = _rand_att(g, 1, L, 2, 1, D)
    pos = [0, 4, 8]
    o16, _ = orc.attention(q, pos, k, v, 0.3)
    for t, p in enumerate(pos):
        for d in range(D):
            mean = sum(F(v[j, 0, d]) for j in range(p + 1)) / (p + 1)
            assert int(o16[t, 0, d]) == fraction_to_bf16_bits(mean)


def test_attention_scale_zero_is_uniform(orc):
    g = np.random.default_rng(12)
    q, k, v = _rand_att(g, 1, 5, 1, 1, 4)
    o16, _ = orc.attention(q, [4], k, v, 0.0)
    for d in range(4):
        mean = sum(F(v[j, 0, d]) for j in range(5)) / 5
        assert int(o16[0, 0, d]) == fraction_to_bf16_bits(mean)


def test_attention_equal_values_return_that_value(orc):
    g = np.random.default_rng(13)
    q, k, _ = _rand_att(g, 4, 50, 4, 1, 32)
    row = I.normal_bf16(g, (32,))
    v = np.tile(row, (50, 1, 1))
    o16, _ = orc.attention(q, [0, 10, 33, 49], k, v, 0.1)
    assert np.all(o16 == row[None, None, :])


def test_attention_causal_ignores_future_keys(orc):
    g = np.random.default_rng(14)
    q, k, v = _rand_att(g, 3, 40, 2, 2, 8)
    pos = [5, 20, 39]
    o1, _ = orc.attention(q, pos, k, v, 0.35)
    k2, v2 = k.copy(), v.copy()
    k2[21:] ^= np.uint16(0x1234)
    v2[21:] ^= np.uint16(0x0101)
    o2, _ = orc.attention(q, pos, k2, v2, 0.35)
    assert np.array_equal(o1[:2], o2[:2])       # rows at 5 and 20 never see 21..
    assert not np.array_equal(o1[2], o2[2])


def test_attention_gqa_group_mapping(orc):
    # Hq=4, Hkv=2: heads 0,1 read kv head 0; heads 2,3 read kv head 1
    g = np.random.default_rng(15)
    q, k, v = _rand_att(g, 1, 6, 4, 2, 8)
    c0 = I.normal_bf16(g, (8,))
    c1 = I.normal_bf16(g, (8,))
    v[:, 0, :] = c0
    v[:, 1, :] = c1
    o16, _ = orc.attention(q, [5], k, v, 0.5)
    assert np.array_equal(o16[0, 0], c0) and np.array_equal(o16[0, 1], c0)
    assert np.array_equal(o16[0, 2], c1) and np.array_equal(o16[0, 3], c1)


def test_attention_brute_force_decimal(orc):
    g = np.random.default_rng(16)
    L, D, Hq, Hkv = 6, 4, 2, 1
    q, k, v = _rand_att(g, 2, L, Hq, Hkv, D)
    scale = 0.5
    pos = [2, 5]
    o16, o64 = orc.attention(q, pos, k, v, scale)
    for t, p in enumerate(pos):
        for h in range(Hq):
            s = [Fraction(scale) * sum(F(q[t, h, d]) * F(k[j, 0, d]) for d in range(D))
                 for j in range(p + 1)]
            e = [CTX.exp(dec(x)) for x in s]           # no max shift: exact identity
            z = sum(e, decimal.Decimal(0))
            for d in range(D):
                num = sum((ej * dec(F(v[j, 0, d])) for j, ej in enumerate(e)), decimal.Decimal(0))
                exact = Fraction(CTX.divide(num, z))
                assert abs(o64[t, h, d] - float(exact)) <= 1e-14 * max(1.0, abs(float(exact)))
                if not near_bf16_tie(exact, 1e-9):
                    assert int(o16[t, h, d]) == fraction_to_bf16_bits(exact)


def test_attention_score_shift_invariance(orc):
    # adding a vector u with q.u = c to every key shifts all scores of q by
    # scale*c; softmax is unchanged
    g = np.random.default_rng(17)
    D = 8
    q, k, v = _rand_att(g, 1, 12, 1, 1, D)
    q[0, 0] = bits_of([1.0, 0, 0, 0, 0, 0, 0, 0])
    k[..., 0] = bits_of(g.integers(-2, 3, k.shape[:2]).astype(np.float32))
    k2 = I.f32_to_bf16(I.bf16_to_f32(k) + np.array([3.0] + [0] * 7, np.float32))
    assert np.array_equal(k2[..., 1:], k[..., 1:])
    assert np.all(I.bf16_to_f32(k2)[..., 0] == I.bf16_to_f32(k)[..., 0] + 3.0)
    o1, a1 = orc.attention(q, [11], k, v, 0.7)
    o2, a2 = orc.attention(q, [11], k2, v, 0.7)
    assert np.allclose(a1, a2, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- argmax

def test_argmax_ties_lowest_index_and_nan(orc):
    g = np.random.default_rng(18)
    x = g.standard_normal((50, 300)).astype(np.float32)
    for r in range(0, 50, 3):
        i, j = sorted(g.choice(300, 2, replace=False))
        x[r, i] = x[r, j] = x[r].max() + 1.0           # planted tie
    ids = orc.argmax(x)
    for r in range(50):
        m = x[r].max()
        assert ids[r] == min(i for i in range(300) if x[r, i] == m)
    x[7, 123] = np.nan
    assert orc.argmax(x[7:8])[0] == -1


# ---------------------------------------------------------------- addmm

def test_addmm_bias_row_added_once(orc):
    g = np.random.default_rng(47)
    a = bits_of(g.integers(-8, 9, (5, 64)).astype(np.float64))
    w = bits_of(g.integers(-8, 9, (7, 64)).astype(np.float64))
    b = bits_of(g.integers(-100, 101, 7).astype(np.float64) / 4)
    exact = (I.bf16_to_f32(a).astype(np.int64) @ I.bf16_to_f32(w).astype(np.int64).T).astype(np.float64) \
        + I.bf16_to_f32(b).astype(np.float64)[None]
    assert np.array_equal(orc.addmm_f64(a, w, b), exact)
    assert np.array_equal(orc.addmm_f64(np.zeros_like(a), w, b)[3], I.bf16_to_f32(b).astype(np.float64))


# ---------------------------------------------------------------- mean

def test_mean_closed_forms_and_brute_force(orc):
    H = 4096
    x = np.zeros((4, H), np.uint16)
    x[0] = bits_of([1.5])[0]                                   # constant row
    x[1, 17] = bits_of([1.0])[0]                               # one-hot: 1/H
    x[2, :H // 2] = bits_of([2.0])[0]
    x[2, H // 2:] = bits_of([-2.0])[0]                         # cancels to 0
    x[3] = bits_of(np.arange(H) % 7 - 3.0)                     # small integers
    m = orc.mean(x)
    assert m[0] == 1.5 and m[1] == 1.0 / H and m[2] == 0.0
    assert m[3] == float(Fraction(int(np.sum(np.arange(H) % 7 - 3)), H))
    g = np.random.default_rng(46)
    y = I.normal_bf16(g, (5, 33))
    ref = [sum((F(b) for b in row), Fraction(0)) / 33 for row in y]
    assert np.allclose(orc.mean(y), [float(r) for r in ref], rtol=1e-15, atol=0)


# ---------------------------------------------------------------- log_softmax

def test_log_softmax_uniform_row_is_minus_log_V(orc):
    for V in (1, 2, 7, 32000):
        x = np.full((2, V), 3.25, np.float32)
        x[1] = -11.0
        y = orc.log_softmax(x)
        assert np.allclose(y, -math.log(V), rtol=0, atol=1e-12)


def test_log_softmax_two_entries_closed_form(orc):
    g = np.random.default_rng(40)
    x = g.uniform(-20, 20, (30, 2)).astype(np.float32)
    y = orc.log_softmax(x)
    for r in range(30):
        a, b = float(x[r, 0]), float(x[r, 1])
        assert abs(y[r, 0] + math.log1p(math.exp(b - a))) < 1e-12
        assert abs(y[r, 1] + math.log1p(math.exp(a - b))) < 1e-12


def test_log_softmax_one_large_entry_closed_form(orc):
    V = 1000
    for a in (0.5, 7.0, 40.0):
        x = np.zeros((1, V), np.float32)
        x[0, 3] = a
        y = orc.log_softmax(x)[0]
        z = math.exp(a) + (V - 1)
        assert abs(y[3] - (a - math.log(z))) < 1e-12
        assert np.allclose(np.delete(y, 3), -math.log(z), rtol=0, atol=1e-12)


def test_log_softmax_shift_invariance_and_normalisation(orc):
    g = np.random.default_rng(41)
    x = np.round(g.standard_normal((20, 500)) * 4).astype(np.float32)     # integers: x + c exact
    y = orc.log_softmax(x)
    y2 = orc.log_softmax(x + np.float32(1000.0))                            # exp(1000) overflows unshifted
    assert np.allclose(y, y2, rtol=0, atol=1e-10)
    assert np.allclose(np.exp(y).sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.argmax(y, axis=1) == np.argmax(x, axis=1))


def test_log_softmax_brute_force_decimal(orc):
    g = np.random.default_rng(42)
    x = (g.integers(-300, 300, (6, 7)) / 16).astype(np.float32)           # exact in float32
    y = orc.log_softmax(x)
    with decimal.localcontext(CTX):
        for r in range(6):
            s = sum(dec(float(v)).exp() for v in x[r])
            lse = s.ln()
            for i in range(7):
                assert abs(float(dec(float(x[r, i])) - lse) - y[r, i]) < 1e-12


def test_log_softmax_masked_entries_and_nan(orc):
    g = np.random.default_rng(43)
    x = g.standard_normal((3, 64)).astype(np.float32)
    x[0, ::3] = -np.inf                                   # masked logits
    y = orc.log_softmax(x)
    keep = np.isfinite(x[0])
    assert np.all(y[0, ~keep] == -np.inf)
    assert np.allclose(y[0, keep], orc.log_softmax(x[0:1, keep])[0], rtol=0, atol=1e-12)
    x[1] = -np.inf                                        # nothing left to normalise over
    x[2, 5] = np.nan
    y = orc.log_softmax(x)
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))


# ---------------------------------------------------------------- seeded sampling

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_philox_known_answer_vectors(orc):
    rows = []
    for line in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")):
        if line.strip() and not line.startswith("#"):
            c, k, o = (np.array([int(w, 16) for w in part.split()], np.uint64) for part in line.split("|"))
            rows.append((c, k, o))
    assert len(rows) == 3
    for c, k, o in rows:
        assert np.array_equal(orc.philox4x32_10(c[None].astype(np.uint32), k[None].astype(np.uint32))[0],
                              o.astype(np.uint32))


def _chi2(counts, p):
    n = counts.sum()
    return float(((counts - n * p) ** 2 / (n * p)).sum())


def test_sample_frequencies_follow_softmax_over_temperature(orc):
    # Gumbel-max picks i with probability softmax(x / T)_i; 60000 seeded draws
    # per case, chi-square with 3 degrees of freedom against 16.27 (p = 0.001)
    x = np.array([[0.0, 1.0, 2.0, 3.0]], np.float32)
    for T in (1.0, 0.5, 2.0):
        n = 60000
        ids = orc.sample(np.repeat(x, n, axis=0), T, np.arange(n, dtype=np.uint64) * 7919 + 3,
                         np.full(n, 5, np.uint64))
        counts = np.bincount(ids, minlength=4).astype(np.float64)
        p = np.exp(x[0] / T) / np.exp(x[0] / T).sum()
        assert _chi2(counts, p) < 16.27, (T, counts, p)


def test_sample_small_temperature_is_argmax_and_draws_are_reproducible(orc):
    g = np.random.default_rng(44)
    x = np.round(g.standard_normal((40, 300)) * 8).astype(np.float32)
    x += np.arange(300, dtype=np.float32)[None] * 1e-3               # no exact ties
    seeds = g.integers(0, 2 ** 63, 40).astype(np.uint64)
    offs = g.integers(0, 2 ** 40, 40).astype(np.uint64)
    assert np.array_equal(orc.sample(x, 1e-4, seeds, offs), orc.argmax(x))
    a = orc.sample(x, 1.0, seeds, offs)
    assert np.array_equal(a, orc.sample(x, 1.0, seeds, offs))        # same key and counter, same draw
    assert not np.array_equal(a, orc.sample(x, 1.0, seeds, offs + 1))  # another counter, another draw
    # equal logits: the choice is the largest noise, so it moves with the seed
    u = orc.sample(np.zeros((200, 50), np.float32), 1.0, np.arange(200, dtype=np.uint64),
                   np.zeros(200, np.uint64))
    assert len(set(u.tolist())) > 30
    x[3, 17] = np.nan
    assert orc.sample(x[3:4], 1.0, seeds[3:4], offs[3:4])[0] == -1


# ---------------------------------------------------------------- top-2 margin

def test_top2_margin_cases(orc):
    x = np.array([[1.0, 5.0, 3.0, 5.0],          # tie at the top: lowest index, margin 0
                  [0.0, -1.0, 2.5, 2.0],         # 2.5 - 2.0
                  [7.0, 0.0, 0.0, 0.0],
                  [-np.inf, -np.inf, 1.0, -np.inf],
                  [1.0, np.nan, 0.0, 0.0]], np.float32)
    ids, m = orc.top2(x)
    assert ids.tolist() == [1, 2, 0, 2, -1]
    assert m[0] == 0.0 and m[1] == np.float32(0.5) and m[2] == np.float32(7.0) and m[3] == np.inf
    assert np.isnan(m[4])
    ids1, m1 = orc.top2(np.array([[3.0]], np.float32))
    assert ids1[0] == 0 and m1[0] == np.inf                 # no second candidate
    g = np.random.default_rng(45)
    x = g.standard_normal((30, 1000)).astype(np.float32)
    ids, m = orc.top2(x)
    srt = np.sort(x, axis=1)
    assert np.array_equal(ids, orc.argmax(x))
    assert np.array_equal(m, (srt[:, -1] - srt[:, -2]).astype(np.float32))


def test_lm_head_f64_one_hot_closed_form(orc):
    """h = a e_k: mean of squares a^2/H, so every logit is
    a / sqrt(a^2/H + eps) * w_k * W[v][k] (pins the 1/H, eps inside the root,
    the weight and the column of W that is read; k = H-1 pins the last term)."""
    H, V, eps = 64, 7, 1e-6
    g = np.random.default_rng(71)
    w = I.normal_bf16(g, (H,))
    wt = I.normal_bf16(g, (V, H))
    wd, wtd = orc.bf16_to_f64(w), orc.bf16_to_f64(wt)
    for k, a_bits in ((0, 0x3FC0), (H - 1, 0xC020), (17, 0x4100)):        # 1.5, -2.5, 8.0
        h = np.zeros((1, H), np.uint16)
        h[0, k] = a_bits
        a = float(orc.bf16_to_f64(np.array([a_bits], np.uint16))[0])
        exp = a / math.sqrt(a * a / H + eps) * wd[k] * wtd[:, k]
        got = orc.lm_head_f64(h, w, eps, wt)[0]
        assert np.allclose(got, exp, rtol=1e-13, atol=0), k


def test_lm_head_f64_factorised_form_and_scale_invariance(orc):
    """The head equals rstd * (W @ (w * h)) summed in another grouping, and
    with eps = 0 it does not change when h is scaled by 2 (exact in bf16)."""
    g = np.random.default_rng(72)
    R, H, V = 5, 96, 40
    h = I.normal_bf16(g, (R, H))
    w = I.normal_bf16(g, (H,))
    wt = I.normal_bf16(g, (V, H))
    hd, wd, wtd = orc.bf16_to_f64(h), orc.bf16_to_f64(w), orc.bf16_to_f64(wt)
    got = orc.lm_head_f64(h, w, 1e-5, wt)
    rstd = 1.0 / np.sqrt(np.mean(hd * hd, axis=1) + 1e-5)
    exp = rstd[:, None] * ((hd * wd[None, :]) @ wtd.T)
    scale = np.abs(hd * wd[None, :]) @ np.abs(wtd.T) * rstd[:, None]
    assert np.all(np.abs(got - exp) <= 1e-13 * scale)
    h2 = orc.round_bf16(2.0 * hd)
    a = orc.lm_head_f64(h, w, 0.0, wt)
    b = orc.lm_head_f64(h2, w, 0.0, wt)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- sanity

def test_float_addition_order_matters():
    # The premise of the method (post 論文／ブログ「Defeating Nondeterminism in
    # LLM Inference」の技術的なポイント; page hakusoku.com, section
    # 浮動小数点演算の非結合性): a different summation order can give a
    # different float result.  The tests must be able to see that.
    a = np.float32(1e8); b = np.float32(1.0); c = np.float32(-1e8)
    assert (a + c) + b == np.float32(1.0)
    assert a + (c + b) == np.float32(0.0)


def test_oracle_thread_count_invariant(tmp_path):
    code = (
        "import numpy as np, oracle\n"
        "from invariant_bi_rmsnorm_amd import inputs as I\n"
        "g=np.random.default_rng(3); x=I.normal_bf16(g,(64,512)); w=I.normal_bf16(g,(512,),1,0.1)\n"
        "wt=I.normal_bf16(g,(96,512),0,0.02)\n"
        "y,r=oracle.rmsnorm(x,w,1e-6); c=oracle.matmul(x,wt,'f32')\n"
        "print(hash(y.tobytes())^hash(r.tobytes())^hash(c.tobytes()))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for nt in ("1", "8"):
        env = dict(os.environ, OMP_NUM_THREADS=nt, PYTHONHASHSEED="0")
        outs.append(subprocess.run([sys.executable, "-c", code], cwd=root, env=env,
                                   capture_output=True, text=True, check=True).stdout)
    assert outs[0] == outs[1]
