"""The toy decoder's forward one layer at a time, composed from the oracle's
per-op functions (test infrastructure: the oracle's own toy forward runs all
layers in one call and returns only the last token's logits).

The layer is the pre-norm step of the greedy decoder (page "la température
zéro n'est pas déterministe", introduction: greedy decoding of one prompt; the
model is read as a Llama-style decoder): RMSNorm -> QKV projection -> RoPE on
q and k -> causal attention over the prompt -> O projection -> residual add ->
RMSNorm -> gate|up projection -> SiLU(gate) * up -> down projection ->
residual add, each op rounded to bf16 as the model stores it.  Pinned on the
CPU to the oracle's toy forward (the same ops in the same order give the same
bits, test_toy_layer_oracle.py)."""
from __future__ import annotations

import math

import numpy as np


def attn_half(orc, cfg: dict, lw: dict, h):
    """The attention half of a layer over the T tokens of one prompt at
    positions 0..T-1: h [T, hidden] bf16 bits -> (the stream after the
    attention add, the O projection added to it), bf16 bits."""
    H, D, Hq, Hkv = cfg["hidden"], cfg["head_dim"], cfg["heads"], cfg["kv_heads"]
    T = h.shape[0]
    pos = np.arange(T, dtype=np.int32)
    xn, _ = orc.rmsnorm(h, lw["attn_norm"], cfg["eps"])
    qkv = orc.matmul(xn, lw["wqkv"])
    q = np.ascontiguousarray(qkv[:, :Hq * D]).reshape(T, Hq, D)
    k = np.ascontiguousarray(qkv[:, Hq * D:(Hq + Hkv) * D]).reshape(T, Hkv, D)
    v = np.ascontiguousarray(qkv[:, (Hq + Hkv) * D:]).reshape(T, Hkv, D)
    qr = orc.rope(q, pos, cfg["rope_theta"])
    kr = orc.rope(k, pos, cfg["rope_theta"])
    att, _ = orc.attention(qr, pos, kr, v, 1.0 / math.sqrt(D))
    a_out = orc.matmul(att.reshape(T, Hq * D), lw["wo"])
    return orc.add(h, a_out), a_out


def mlp_half(orc, cfg: dict, lw: dict, mid):
    """The MLP half: mid [T, hidden] bf16 bits -> (the stream after the MLP
    add, the down projection added to it), bf16 bits."""
    F = cfg["mlp"]
    xn, _ = orc.rmsnorm(mid, lw["mlp_norm"], cfg["eps"])
    gu = orc.matmul(xn, lw["wgu"])
    act = orc.silu_mul(np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:]))
    m_out = orc.matmul(act, lw["wd"])
    return orc.add(mid, m_out), m_out


def layer(orc, cfg: dict, lw: dict, h):
    """One decoder layer: h [T, hidden] bf16 bits -> the stream after it."""
    mid, _ = attn_half(orc, cfg, lw, h)
    return mlp_half(orc, cfg, lw, mid)[0]


def last_logits(orc, cfg: dict, w: dict, h):
    """Final RMSNorm of the last token, then the output head in float64."""
    xn, _ = orc.rmsnorm(h[-1:], w["final_norm"], cfg["eps"])
    return orc.matmul_f64(xn, w["lm_head"])[0]


def forward(orc, cfg: dict, w: dict, ids):
    """Embedding rows, every layer, the head: logits of the last token."""
    h = np.ascontiguousarray(w["embed"][np.asarray(ids)])
    for lw in w["layers"][:cfg["layers"]]:
        h = layer(orc, cfg, lw, h)
    return last_logits(orc, cfg, w, h)
