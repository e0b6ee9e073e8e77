"""An independent fp32 evaluation of the toy decoder forward (numpy), used only
to measure how far two correct evaluations of the bf16 model drift apart when
they round differently.  That spread sets the end-to-end bar for the GPU's
toy logits; each op is held to the per-op bar separately."""
from __future__ import annotations

import math

import numpy as np

from invariant_bi_rmsnorm_amd import inputs as I


def _f(b):
    return I.bf16_to_f32(b)


def _r16(x):
    return I.f32_to_bf16(np.asarray(x, np.float32))


def _ops(cfg: dict):
    D = cfg["head_dim"]
    eps = np.float32(cfg["eps"])

    def rms(x, wt):
        xf = _f(x).astype(np.float32)
        r = 1 / np.sqrt((xf * xf).mean(-1, keepdims=True) + eps)
        return _r16(xf * r * _f(wt))

    def mm(a, wt):
        return _r16(_f(a).astype(np.float32) @ _f(wt).astype(np.float32).T)

    def rope(x, pos):
        half = D // 2
        i = np.arange(half)
        ang = pos[:, None].astype(np.float64) * cfg["rope_theta"] ** (-2.0 * i / D)
        c = np.cos(ang).astype(np.float32)[:, None, :]
        s = np.sin(ang).astype(np.float32)[:, None, :]
        xf = _f(x)
        a, b = xf[..., :half], xf[..., half:]
        return _r16(np.concatenate([a * c - b * s, b * c + a * s], -1))

    return rms, mm, rope


def layer_fp32(cfg: dict, lw: dict, h, bf16_weights: bool = False) -> np.ndarray:
    """One decoder layer in fp32 over the T tokens of one prompt (positions
    0..T-1): h [T, hidden] bf16 bits -> the residual stream after it (bf16 bits).
    bf16_weights: the softmax weights exp(s - max) are rounded to bf16 before
    their sum and the value product, the weights' rounding the library's
    attention splits apply (prompts of at most 256 tokens are one split)."""
    T = h.shape[0]
    D, Hq, Hkv, F = cfg["head_dim"], cfg["heads"], cfg["kv_heads"], cfg["mlp"]
    G = Hq // Hkv
    rms, mm, rope = _ops(cfg)
    pos = np.arange(T)
    causal = np.tril(np.ones((T, T), bool))
    xn = rms(h, lw["attn_norm"])
    qkv = mm(xn, lw["wqkv"]).reshape(T, Hq + 2 * Hkv, D)
    q = rope(qkv[:, :Hq], pos)
    k = rope(qkv[:, Hq:Hq + Hkv], pos)
    v = qkv[:, Hq + Hkv:]
    out = np.zeros((T, Hq, D), np.float32)
    for hh in range(Hq):
        s = (_f(q[:, hh]) @ _f(k[:, hh // G]).T) / np.float32(math.sqrt(D))
        s = np.where(causal, s, -np.inf)
        p = np.exp(s - s.max(-1, keepdims=True))
        if bf16_weights:
            p = _f(_r16(p))
            out[:, hh] = (p @ _f(v[:, hh // G])) / p.sum(-1, keepdims=True)
        else:
            p /= p.sum(-1, keepdims=True)
            out[:, hh] = p @ _f(v[:, hh // G])
    o = mm(_r16(out).reshape(T, -1), lw["wo"])
    h = _r16(_f(h) + _f(o))
    xn = rms(h, lw["mlp_norm"])
    gu = _f(mm(xn, lw["wgu"]))
    g, u = gu[:, :F], gu[:, F:]
    d = mm(_r16(g / (1 + np.exp(-g)) * u), lw["wd"])
    return _r16(_f(h) + _f(d))


def toy_logits_fp32(cfg: dict, w: dict, ids, bf16_weights: bool = False) -> np.ndarray:
    rms, _, _ = _ops(cfg)
    h = w["embed"][np.asarray(ids)]
    for lw in w["layers"]:
        h = layer_fp32(cfg, lw, h, bf16_weights)
    xn = rms(h[-1:], w["final_norm"])
    return (_f(xn) @ _f(w["lm_head"]).astype(np.float32).T)[0].astype(np.float64)
