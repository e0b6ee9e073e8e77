"""Helpers for the GPU tests: moving bf16 bit patterns to and from the device,
the parity tolerance, and building a paged KV cache through bi_kv_append."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from invariant_bi_rmsnorm_amd import inputs as I

DEV = "cuda"


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.array(bits, dtype=np.uint16, order="C", copy=True).view(np.int16)
    return torch.from_numpy(a).to(DEV).view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.array(a, dtype=np.int32, order="C", copy=True)).to(DEV)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return I.bf16_to_f32(bits).astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits, subnormal floor 2^-133)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.exp2(np.maximum(e - 7, -133))


def check_bf16(gpu_bits: np.ndarray, ref64: np.ndarray, what: str, rel: float = 1e-2,
               axis=None) -> float:
    """Parity bar for bf16 outputs.

    Each element must satisfy |gpu - exact| <= rel * RMS(exact) + ulp_bf16(exact):
    rel * RMS bounds the arithmetic (fp32 accumulation) error; one bf16 ulp of
    the exact value covers the final rounding of the stored result, which alone
    exceeds 1e-2 * RMS for |value| > ~2.6 RMS.  RMS is taken over the whole
    tensor (axis=None) or per row (axis=-1 over the trailing dims).
    Returns the worst (|err| - ulp)/ (rel*RMS) ratio (<= 1 passes).
    """
    g = bf16_f64(gpu_bits).reshape(ref64.shape)
    if axis is None:
        rms = math.sqrt(float(np.mean(ref64 ** 2)))
        rms_b = np.full(ref64.shape, rms)
    else:
        flat = ref64.reshape(ref64.shape[0], -1)
        rms_r = np.sqrt(np.mean(flat ** 2, axis=1))
        rms_b = np.broadcast_to(rms_r.reshape((-1,) + (1,) * (ref64.ndim - 1)), ref64.shape)
    err = np.abs(g - ref64)
    bound = rel * rms_b + bf16_ulp(ref64)
    bad = ~(err <= bound)
    ratio = float(np.max((err - bf16_ulp(ref64)) / np.maximum(rel * rms_b, 1e-300)))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first {idx.tolist()}; "
                             f"gpu={g[tuple(idx[0])]} ref={ref64[tuple(idx[0])]} bound={bound[tuple(idx[0])]}")
    return ratio


def nan_bf16(shape) -> torch.Tensor:
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)


class PagedCache:
    """A paged KV cache filled through bi_kv_append (the product's own append)."""

    def __init__(self, num_blocks: int, Hkv: int, D: int = 128):
        self.Hkv, self.D, self.num_blocks = Hkv, D, num_blocks
        self.k = nan_bf16((num_blocks, Hkv, 16, D))       # poisoned: unused slots hold NaN
        self.v = nan_bf16((num_blocks, Hkv, D, 16))

    def append(self, k_bits: np.ndarray, v_bits: np.ndarray, slots: np.ndarray):
        from invariant_bi_rmsnorm_amd import ops
        if len(slots) == 0:
            return
        ops.bi_kv_append(dev_bf16(k_bits), dev_bf16(v_bits), dev_i32(slots), self.k, self.v)


def make_cache(g, kvs, capacities=None, extra_blocks: int = 0, Hkv: int = I.ATT_HKV):
    """Place sequences (list of (k, v) [L,Hkv,D]) in a cache with a random
    block permutation; returns (cache, block_table np [S, max_blocks])."""
    lens = [k.shape[0] for k, _ in kvs]
    caps = capacities or lens
    total = sum(max(1, -(-c // 16)) for c in caps)
    table, nblk = I.block_tables(g, caps, total + extra_blocks)
    cache = PagedCache(nblk, Hkv)
    ks, vs, sl = [], [], []
    for s, (k, v) in enumerate(kvs):
        ks.append(k); vs.append(v)
        sl.append(I.slots_for(table[s], np.arange(k.shape[0])))
    cache.append(np.concatenate(ks), np.concatenate(vs), np.concatenate(sl))
    return cache, table
