"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This module holds no arithmetic of the method: it only draws random numbers
(numpy PCG64), converts them to bf16 bit patterns and lays out index tables.
Everything is generated on the CPU so that both sides read identical bits.

Recipe (workload shapes from the pages' experiment are not published; these
Llama-shaped synthetic stand-ins follow the configurations listed in the
build's baseline file):

* bf16 values: float64 normal -> float32 (round to nearest even) -> bf16
  (round to nearest even on the bit pattern).
* Seeds: ``np.random.default_rng((tag, trial, index...))`` -- a SeedSequence
  over a tuple, so every (config, trial, sequence) stream is independent and
  reproducible on its own (a test can regenerate one sampled sequence without
  generating the whole batch).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# configuration tags used in the seed tuples
TAG_TINY = 1
TAG_LLAMA = 2
TAG_DECODE = 3
TAG_PREFILL = 4
TAG_TOY = 5

BLOCK = 16          # tokens per KV-cache block
SPLIT = 256         # tokens per attention split (fixed size)


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def f32_to_bf16(a) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even, NaN kept."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(g: np.random.Generator, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float64)
    if std != 1.0:
        x *= std
    if mean != 0.0:
        x += mean
    return f32_to_bf16(x.astype(np.float32))


def normal_bf16_fast(g: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) bf16 drawn in float32 (used for the multi-GB KV caches)."""
    return f32_to_bf16(g.standard_normal(size=shape, dtype=np.float32))


# ----------------------------------------------------------------------------
# Tiny invariance check: x [B,256] ~ N(0,1) with row 0 one fixed vector,
# RMSNorm eps 1e-6 with w ~ N(1, 0.1), then x @ W with W [256,512] ~ N(0, 0.05)
# ----------------------------------------------------------------------------
TINY_H = 256
TINY_N = 512
TINY_EPS = 1e-6
TINY_BATCHES = (1, 2, 3, 8)


def tiny_weights():
    g = rng(TAG_TINY, 0, 0)
    w = normal_bf16(g, (TINY_H,), 1.0, 0.1)
    wt = normal_bf16(g, (TINY_N, TINY_H), 0.0, 0.05)   # stored [N,K]
    return w, wt


def tiny_x(B: int, trial: int = 0) -> np.ndarray:
    x = normal_bf16(rng(TAG_TINY, 1 + trial, B), (B, TINY_H))
    x[0] = normal_bf16(rng(TAG_TINY, 1, 0), (TINY_H,))   # row 0 fixed for every B
    return x


# ----------------------------------------------------------------------------
# Llama-8B-shaped projections: RMSNorm over 4096, then [M,4096]x[4096,4096]
# and [M,4096]x[4096,14336]; inputs N(0,1), weights N(0,0.02).
# ----------------------------------------------------------------------------
LLAMA_H = 4096
LLAMA_N = (4096, 14336)
LLAMA_EPS = 1e-6
M_SWEEP = tuple(range(1, 65)) + (128, 256, 512, 1024, 2048)


def llama_norm_weight() -> np.ndarray:
    return normal_bf16(rng(TAG_LLAMA, 0, 0), (LLAMA_H,), 1.0, 0.1)


def llama_weight(N: int) -> np.ndarray:
    """Stored [N,K] = [N,4096]."""
    return normal_bf16(rng(TAG_LLAMA, 0, N), (N, LLAMA_H), 0.0, 0.02)


def llama_x(M: int, trial: int = 0) -> np.ndarray:
    x = normal_bf16(rng(TAG_LLAMA, 1 + trial, M), (M, LLAMA_H))
    x[0] = normal_bf16(rng(TAG_LLAMA, 1, 0), (LLAMA_H,))   # row 0 fixed for every M
    return x


# ----------------------------------------------------------------------------
# Paged attention: 32 query heads, 8 KV heads, head_dim 128, block 16, split 256.
# KV lengths log-uniform in [1, 32768].
# ----------------------------------------------------------------------------
ATT_HQ = 32
ATT_HKV = 8
ATT_D = 128
ATT_MAX_LEN = 32768
EDGE_LENGTHS = (1, 15, 16, 17, 255, 256, 257, 32767, 32768)


def loguniform_lengths(g: np.random.Generator, S: int, max_len: int = ATT_MAX_LEN) -> np.ndarray:
    u = g.uniform(0.0, math.log(max_len), size=S)
    return np.clip(np.rint(np.exp(u)), 1, max_len).astype(np.int32)


def kv_sequence(tag: int, trial: int, s: int, L: int, Hkv: int = ATT_HKV, D: int = ATT_D):
    """Logical K, V [L,Hkv,D] bf16 bits of one sequence (its own seed stream)."""
    g = rng(tag, trial, 1000 + s)
    k = normal_bf16_fast(g, (L, Hkv, D))
    v = normal_bf16_fast(g, (L, Hkv, D))
    return k, v


def kv_sequences(tag: int, trial: int, lengths, Hkv: int = ATT_HKV, D: int = ATT_D, threads: int = 8):
    lengths = [int(x) for x in lengths]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda sl: kv_sequence(tag, trial, sl[0], sl[1], Hkv, D),
                           enumerate(lengths)))


def queries(tag: int, trial: int, T: int, Hq: int = ATT_HQ, D: int = ATT_D) -> np.ndarray:
    return normal_bf16(rng(tag, trial, 7), (T, Hq, D))


def block_tables(g: np.random.Generator, capacities, num_blocks: int | None = None):
    """Random physical placement: a permutation of the block pool is dealt
    out to the sequences in order.  capacities[s] = tokens sequence s may hold.

    Returns (block_table [S, max_blocks] int32 padded with -1, num_blocks).
    """
    caps = [int(c) for c in capacities]
    nb = [max(1, -(-c // BLOCK)) for c in caps]
    total = sum(nb)
    if num_blocks is None:
        num_blocks = total
    if num_blocks < total:
        raise ValueError("block pool too small")
    perm = g.permutation(num_blocks).astype(np.int32)
    max_blocks = max(nb) if nb else 1
    table = np.full((len(caps), max_blocks), -1, dtype=np.int32)
    o = 0
    for s, n in enumerate(nb):
        table[s, :n] = perm[o:o + n]
        o += n
    return table, num_blocks


def slots_for(table_row: np.ndarray, positions) -> np.ndarray:
    """Cache slot (block*16 + offset) of each absolute token position."""
    pos = np.asarray(positions, dtype=np.int64)
    return (table_row[pos // BLOCK].astype(np.int64) * BLOCK + pos % BLOCK).astype(np.int32)


# ----------------------------------------------------------------------------
# Chunked prefill: prompts of 512..8192 tokens, chunks of 256..2048 tokens.
# ----------------------------------------------------------------------------

def chunk_sizes(g: np.random.Generator, P: int, lo: int = 256, hi: int = 2048):
    out = []
    left = P
    while left > 0:
        c = int(g.integers(lo, hi + 1))
        c = min(c, left)
        out.append(c)
        left -= c
    return out


# ----------------------------------------------------------------------------
# Toy decoder: 8 layers, hidden 2048, 16 heads (4 KV), MLP 5632, vocab 32000.
# ----------------------------------------------------------------------------
TOY = dict(layers=8, hidden=2048, heads=16, kv_heads=4, head_dim=128,
           mlp=5632, vocab=32000, eps=1e-6, rope_theta=10000.0)


def toy_weights(cfg: dict = TOY, seed: int = 0):
    """Random-init bf16 weights, linear layers stored [out,in]."""
    H = cfg["hidden"]; Hq = cfg["heads"]; Hkv = cfg["kv_heads"]; D = cfg["head_dim"]
    F = cfg["mlp"]; V = cfg["vocab"]
    g = rng(TAG_TOY, seed, 0)
    w = {"embed": normal_bf16(g, (V, H)), "layers": []}
    for _ in range(cfg["layers"]):
        w["layers"].append({
            "attn_norm": normal_bf16(g, (H,), 1.0, 0.1),
            "wqkv": normal_bf16(g, ((Hq + 2 * Hkv) * D, H), 0.0, 0.02),
            "wo": normal_bf16(g, (H, Hq * D), 0.0, 0.02),
            "mlp_norm": normal_bf16(g, (H,), 1.0, 0.1),
            "wgu": normal_bf16(g, (2 * F, H), 0.0, 0.02),
            "wd": normal_bf16(g, (H, F), 0.0, 0.02),
        })
    w["final_norm"] = normal_bf16(g, (H,), 1.0, 0.1)
    w["lm_head"] = normal_bf16(g, (V, H), 0.0, 0.02)
    return w


def toy_prompt(cfg: dict = TOY, n: int = 64, seed: int = 1) -> np.ndarray:
    return rng(TAG_TOY, seed, 1).integers(0, cfg["vocab"], size=n).astype(np.int32)
