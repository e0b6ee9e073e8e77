"""CPU oracle for the batch-invariant forward path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never imports, links or calls anything here, and this package
never imports the product: the two share only the seeded input bits.

The arithmetic lives in ``oracle.c`` (plain C, double precision, one final
rounding); this module only builds it with gcc and marshals numpy arrays.
Every function documents the passage of the pages it follows; the C file
states the formulas.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.environ.get("BI_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (OpenMP over independent rows)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
               "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _gpu_in_use() -> bool:
    """True once this process has initialised the GPU through torch: from then
    on no compiler may be started as a child process."""
    import sys
    torch = sys.modules.get("torch")
    try:
        return bool(torch is not None and torch.cuda.is_initialized())
    except Exception:
        return False


def require_built() -> str:
    """Path of liboracle.so; raises if it has not been built (it is built by
    ``python __graft_entry__.py build`` or ``oracle.build()``, before any GPU work)."""
    if not os.path.exists(_LIB):
        raise RuntimeError(f"{_LIB} is not built: run `python __graft_entry__.py build` "
                           "(or oracle.build()) before starting GPU work")
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        if _gpu_in_use():
            require_built()
        build(force=False)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    D = ctypes.c_double
    lib.or_round_bf16.argtypes = [P, P, I64]
    lib.or_bf16_to_f64.argtypes = [P, P, I64]
    lib.or_rmsnorm.argtypes = [P, I64, P, P, I64, P, I64, I64, D]
    lib.or_rmsnorm_f64.argtypes = [P, I64, P, P, I64, P, I64, I64, D]
    lib.or_matmul.argtypes = [P, I64, P, I64, P, I64, ctypes.c_int, I64, I64, I64]
    lib.or_matmul_f64.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64]
    lib.or_addmm_f64.argtypes = [P, I64, P, I64, P, P, I64, I64, I64, I64]
    lib.or_attention.argtypes = [P, I64, P, P, P, I64, I32, I32, I32, D, P, P, P]
    lib.or_argmax.argtypes = [P, I64, I64, I64, P]
    lib.or_log_softmax.argtypes = [P, I64, P, I64, I64, I64]
    lib.or_mean.argtypes = [P, I64, P, I64, I64]
    lib.or_philox4x32_10.argtypes = [P, P, P, I64]
    lib.or_top2.argtypes = [P, I64, I64, I64, P, P]
    lib.or_lm_head_f64.argtypes = [P, I64, P, D, P, I64, P, I64, I64, I64, I64]
    lib.or_sample.argtypes = [P, I64, I64, I64, ctypes.c_float, P, P, P, P]
    lib.or_num_threads.restype = ctypes.c_int
    lib.or_set_num_threads.argtypes = [ctypes.c_int]
    lib.or_rope.argtypes = [P, P, P, I64, I32, I32, D]
    lib.or_silu_mul.argtypes = [P, P, P, I64]
    lib.or_add.argtypes = [P, P, P, I64]
    lib.or_toy_scratch_bytes.argtypes = [P, I64]
    lib.or_toy_scratch_bytes.restype = I64
    lib.or_toy_forward.argtypes = [P, P, P, P, P, P, I64, P, P]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns as uint16, got {a.dtype}")
    return a


def num_threads() -> int:
    return int(_load().or_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the row-parallel loops from now on (the results do not depend on it)."""
    _load().or_set_num_threads(int(n))


# --------------------------------------------------------------------------
# bf16 conversion (the oracle's own, independent of numpy's float32 path)
# --------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round doubles straight to bf16 bit patterns, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().or_round_bf16(_p(x), _p(out), x.size)
    return out


def bf16_to_f64(bits) -> np.ndarray:
    bits = _u16(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().or_bf16_to_f64(_p(bits), _p(out), bits.size)
    return out


# --------------------------------------------------------------------------
# RMSNorm -- table row "RMSNorm", post "Defeating Nondeterminism in LLM
# Inference の技術的なポイント" (mobiles-han.blogspot.com), section
# 対応策：バッチ不変なカーネル設計.  Formula: Llama convention (see oracle.c).
# --------------------------------------------------------------------------

def rmsnorm(x, w, eps: float):
    """x [M,H] bf16 bits, w [H] -> (y [M,H] bf16 bits, rstd [M] float32)."""
    x = _u16(x); w = _u16(w)
    M, H = x.shape
    y = np.empty((M, H), dtype=np.uint16)
    rstd = np.empty(M, dtype=np.float32)
    _load().or_rmsnorm(_p(x), H, _p(w), _p(y), H, _p(rstd), M, H, float(eps))
    return y, rstd


def rmsnorm_f64(x, w, eps: float):
    """Unrounded twin: (y [M,H] float64, rstd [M] float64)."""
    x = _u16(x); w = _u16(w)
    M, H = x.shape
    y = np.empty((M, H), dtype=np.float64)
    rstd = np.empty(M, dtype=np.float64)
    _load().or_rmsnorm_f64(_p(x), H, _p(w), _p(y), H, _p(rstd), M, H, float(eps))
    return y, rstd


# --------------------------------------------------------------------------
# Matmul -- table row 行列乗算（MatMul）, same section.  wt is the weight
# stored [N,K] (transposed, K-contiguous); the product is x @ wt.T.
# --------------------------------------------------------------------------

def matmul(a, wt, out: str = "bf16"):
    a = _u16(a); wt = _u16(wt)
    M, K = a.shape
    N, K2 = wt.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if out == "bf16":
        c = np.empty((M, N), dtype=np.uint16); f32 = 0
    elif out == "f32":
        c = np.empty((M, N), dtype=np.float32); f32 = 1
    else:
        raise ValueError(out)
    _load().or_matmul(_p(a), K, _p(wt), K, _p(c), N, f32, M, N, K)
    return c


def matmul_f64(a, wt):
    a = _u16(a); wt = _u16(wt)
    M, K = a.shape
    N, K2 = wt.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    c = np.empty((M, N), dtype=np.float64)
    _load().or_matmul_f64(_p(a), K, _p(wt), K, _p(c), N, M, N, K)
    return c


def addmm_f64(a, wt, bias):
    """bias [N] + a [M,K] @ wt[N,K]^T, all bf16 bits, in float64."""
    a = _u16(a); wt = _u16(wt); bias = _u16(bias)
    M, K = a.shape
    N, K2 = wt.shape
    if K != K2 or bias.shape != (N,):
        raise ValueError("shapes")
    c = np.empty((M, N), dtype=np.float64)
    _load().or_addmm_f64(_p(a), K, _p(wt), K, _p(bias), _p(c), N, M, N, K)
    return c


# --------------------------------------------------------------------------
# Attention -- table row アテンション (Attention), same section; cache and
# fresh tokens form one key sequence as in the FixedAttention sketch of the
# post 「非決定モード → 決定モード」に切り替える例, section 注意点・補足実装.
# --------------------------------------------------------------------------

def attention(q, q_pos, k, v, scale: float):
    """Causal attention over one sequence in logical order.

    q [T,Hq,D], k/v [L,Hkv,D] bf16 bits; q_pos [T] absolute positions.
    Returns (out bf16 bits [T,Hq,D], out float64 [T,Hq,D]).
    """
    q = _u16(q); k = _u16(k); v = _u16(v)
    T, Hq, D = q.shape
    L, Hkv, D2 = k.shape
    if D2 != D or v.shape != k.shape or Hq % Hkv or D > 1024:
        raise ValueError("bad attention shapes")
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    if q_pos.shape != (T,) or (T and (q_pos.min() < 0 or q_pos.max() >= L)):
        raise ValueError("q_pos must lie in [0, L)")
    scratch = np.empty(max(1, T * Hq * L), dtype=np.float64)
    o64 = np.empty((T, Hq, D), dtype=np.float64)
    o16 = np.empty((T, Hq, D), dtype=np.uint16)
    _load().or_attention(_p(q), T, _p(q_pos), _p(k), _p(v), L, Hq, Hkv, D,
                         float(scale), _p(scratch), _p(o64), _p(o16))
    return o16, o64


# --------------------------------------------------------------------------
# Greedy choice -- page "la température zéro n'est pas déterministe",
# section "Le mensonge de la température zéro": argmax at every step.
# --------------------------------------------------------------------------

def argmax(logits):
    """logits [rows,V] float32 -> ids [rows] int32; ties -> lowest index; NaN -> -1."""
    x = np.ascontiguousarray(logits, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, V = x.shape
    ids = np.empty(rows, dtype=np.int32)
    _load().or_argmax(_p(x), V, rows, V, _p(ids))
    return ids


# --------------------------------------------------------------------------
# Toy decoder ops (page "la température zéro n'est pas déterministe",
# introduction: greedy decoding of one prompt repeated 1000 times; the model is
# read as a Llama-style pre-norm decoder, see oracle.c).
# --------------------------------------------------------------------------

def rope(x, pos, theta: float = 10000.0):
    """x [T,H,D] bf16 bits, pos [T] -> rotated bf16 bits (rotate-half pairing)."""
    x = _u16(x)
    T, H, Dm = x.shape
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    y = np.empty_like(x)
    _load().or_rope(_p(x), _p(y), _p(pos), T, H, Dm, float(theta))
    return y


def silu_mul(g, u):
    g = _u16(g); u = _u16(u)
    out = np.empty_like(g)
    _load().or_silu_mul(_p(g), _p(u), _p(out), g.size)
    return out


def add(a, b):
    a = _u16(a); b = _u16(b)
    out = np.empty_like(a)
    _load().or_add(_p(a), _p(b), _p(out), a.size)
    return out


def mean(x):
    """x [rows, H] bf16 bits -> row means, float64 [rows]."""
    x = _u16(x)
    rows, H = x.shape
    out = np.empty(rows, np.float64)
    _load().or_mean(_p(x), H, _p(out), rows, H)
    return out


def log_softmax(x, ld=None):
    """x [rows, V] float32 -> log_softmax over the last dimension, float64 [rows, V]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, V = x.shape
    y = np.empty((rows, V), dtype=np.float64)
    _load().or_log_softmax(_p(x), V, _p(y), V, rows, V)
    return y


def philox4x32_10(ctr, key):
    """ctr [n, 4] uint32, key [n, 2] uint32 -> [n, 4] uint32 (Philox4x32-10)."""
    ctr = np.ascontiguousarray(ctr, dtype=np.uint32).reshape(-1, 4)
    key = np.ascontiguousarray(key, dtype=np.uint32).reshape(-1, 2)
    out = np.empty_like(ctr)
    _load().or_philox4x32_10(_p(ctr), _p(key), _p(out), ctr.shape[0])
    return out


def sample(x, temperature: float, seeds, offsets, with_scores: bool = False):
    """Gumbel-max sampling of each row of x [rows, V] float32 at temperature > 0.
    Returns ids int32 [rows] (and the float64 scores [rows, V] if asked)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, V = x.shape
    seeds = np.ascontiguousarray(seeds, dtype=np.uint64)
    offsets = np.ascontiguousarray(offsets, dtype=np.uint64)
    ids = np.empty(rows, dtype=np.int32)
    sc = np.empty((rows, V), dtype=np.float64) if with_scores else None
    _load().or_sample(_p(x), V, rows, V, float(np.float32(temperature)), _p(seeds), _p(offsets),
                      _p(ids), _p(sc) if sc is not None else None)
    return (ids, sc) if with_scores else ids


def top2(x):
    """x [rows, V] float32 -> (argmax ids int32 [rows], margins float32 [rows])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, V = x.shape
    ids = np.empty(rows, np.int32)
    m = np.empty(rows, np.float32)
    _load().or_top2(_p(x), V, rows, V, _p(ids), _p(m))
    return ids, m


def lm_head_f64(h, w, eps: float, wt):
    """Output head without the bf16 rounding of the normalized hidden state:
    h [R,H] bf16 bits (before the final norm), w [H], wt [V,H] bf16 bits ->
    logits [R,V] float64 (page arxiv-daily-jp.pages.dev/paper/2609.26621,
    abstract)."""
    h = _u16(h); w = _u16(w); wt = _u16(wt)
    R, H = h.shape
    V, H2 = wt.shape
    if H != H2:
        raise ValueError("hidden sizes differ")
    out = np.empty((R, V), dtype=np.float64)
    _load().or_lm_head_f64(_p(h), H, _p(w), float(eps), _p(wt), H, _p(out), V, R, V, H)
    return out


class _ToyCfg(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("mlp", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("eps", ctypes.c_double), ("rope_theta", ctypes.c_double)]


def toy_forward(cfg: dict, w: dict, ids):
    """Logits (float64 [vocab]) of the last of the prompt tokens `ids` (positions
    0..T-1), weights as produced by invariant_bi_rmsnorm_amd.inputs.toy_weights."""
    c = _ToyCfg(cfg["layers"], cfg["hidden"], cfg["heads"], cfg["kv_heads"], cfg["head_dim"],
                cfg["mlp"], cfg["vocab"], float(cfg["eps"]), float(cfg["rope_theta"]))
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T = ids.size
    keep = []
    ptrs = []
    for lw in w["layers"]:
        for k in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd"):
            a = _u16(lw[k]); keep.append(a); ptrs.append(a.ctypes.data)
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    nbytes = int(_load().or_toy_scratch_bytes(ctypes.byref(c), T))
    scratch = np.empty(nbytes, dtype=np.uint8)
    logits = np.empty(cfg["vocab"], dtype=np.float64)
    emb = _u16(w["embed"]); fn = _u16(w["final_norm"]); lm = _u16(w["lm_head"])
    _load().or_toy_forward(ctypes.byref(c), _p(emb), arr, _p(fn), _p(lm), _p(ids), T,
                           _p(scratch), _p(logits))
    return logits
