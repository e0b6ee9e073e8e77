"""Thin Python binding of libbi.so (the C ABI in include/bi.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libbi.so.  PyTorch provides device memory (output tensors are
allocated with torch when the caller does not pass them) and the current HIP
stream.  There is no fallback: if libbi.so is missing or no GPU is present,
calls raise.

Tensor conventions: bf16 data as torch.bfloat16 device tensors, fp32 as
torch.float32, indices as torch.int32, all contiguous in their last dimension.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("BI_LIB") or os.path.join(_HERE, "libbi.so")
# non-invariant baseline library (same ABI); see use_library()
NB_LIB_PATH = os.path.join(_HERE, "libbi_nb.so")
DEFAULT_LIB_PATH = LIB_PATH

BI_OK = 0
BI_ERR_INVALID_ARGUMENT = 1
BI_ERR_UNSUPPORTED = 2
BI_ERR_WORKSPACE_TOO_SMALL = 3
BI_ERR_NO_DEVICE = 4
BI_ERR_LAUNCH = 5
BI_BF16 = 0
BI_F32 = 1

# (name, restype, argtypes) of every symbol declared in include/bi.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_SZ = ctypes.c_size_t
SIGNATURES = {
    "bi_abi_version": (ctypes.c_int, []),
    "bi_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bi_rmsnorm": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _P, _I64, _I64, _F, _P]),
    "bi_matmul": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _I64, ctypes.c_int, _I64, _I64, _I64, _P]),
    "bi_addmm": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _I64, ctypes.c_int, _I64, _I64, _I64, _P]),
    "bi_kv_append": (ctypes.c_int, [_P, _P, _I64, _P, _I64, _P, _P, _I64, _I32, _I32, _P]),
    "bi_attention_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "bi_attention_decode": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _P, _I32, _P, _P, _I64,
                                           _I32, _I32, _I32, _I32, _I32, _F, _P, _SZ, _P]),
    "bi_attention_decode_noalloc": (ctypes.c_int, [_P, _I64, _P, _P, _I64, _P, _I32, _P, _P, _I64,
                                                   _I32, _I32, _I32, _I32, _I32, _F, _P]),
    "bi_attention_prefill": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _P, _I32, _P, _I64,
                                            _I32, _I64, _I32, _I32, _I32, _I32, _F, _P]),
    "bi_argmax": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P]),
    "bi_log_softmax": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _I64, _P]),
    "bi_mean": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _P]),
    "bi_sample": (ctypes.c_int, [_P, _I64, _I64, _I64, _F, _P, _P, _P, _P]),
    "bi_top2": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "bi_lm_head_f32": (ctypes.c_int, [_P, _I64, _P, _F, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _F, _P]),
    "bi_probe_mfma_bf16": (ctypes.c_int, [_P, _P, _P, _P]),
    "bi_probe_copy": (ctypes.c_int, [_P, _P, _I64, _P]),
    "bi_probe_read": (ctypes.c_int, [_P, _I64, _P, _P]),
    "bi_probe_lds_fill": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P]),
    # include/bi_toy.h
    "bi_embed": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _I64, _P]),
    "bi_rope_table": (ctypes.c_int, [_P, _I32, _I32, ctypes.c_double, _P]),
    "bi_rope": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _I64, _P, _I32, _P]),
    "bi_rope_kv_append": (ctypes.c_int, [_P, _I64, _I32, _I32, _I32, _P, _P, _I64, _P, _I32, _P, _P, _I64, _P]),
    "bi_add": (ctypes.c_int, [_P, _P, _P, _I64, _P]),
    "bi_add_rmsnorm": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _I64, _F, _P]),
    "bi_silu_mul": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _I64, _P]),
    "bi_gather_rows": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _I64, _P, _I64, _P]),
    "bi_toy_workspace_bytes": (_SZ, [_P, _I32, _I32, _I32]),
    "bi_toy_step": (ctypes.c_int, [_P, _P, _P, _P, _SZ, _P, _P, _P]),
}

# entry points the non-invariant baseline build (libbi_nb.so) does not export
OPTIONAL_IN_BASELINE = {"bi_attention_decode_noalloc"}
# bi_attention_decode_noalloc's limit on bi_attention_workspace_bytes (include/bi.h)
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class BiError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_string(status)})")


def lib():
    """Load libbi.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libbi.so not found at {LIB_PATH}; build it with "
                "`python -m invariant_bi_rmsnorm_amd._build` (there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            if name in OPTIONAL_IN_BASELINE and not hasattr(L, name):
                continue
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def use_library(path: str):
    """Route the binding to another build of the same ABI (e.g. NB_LIB_PATH,
    the non-invariant baseline); returns the previous path.  Each library is
    loaded once and kept."""
    global LIB_PATH, _lib
    prev = LIB_PATH
    if path != LIB_PATH:
        _loaded[LIB_PATH] = _lib
        LIB_PATH = path
        _lib = _loaded.get(path)
    return prev


_loaded = {}


def status_string(s: int) -> str:
    return lib().bi_status_string(int(s)).decode()


def _check(status: int, fn: str):
    if status != BI_OK:
        raise BiError(status, fn)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous in its last dimension")


def _need_shape(t: torch.Tensor, shape, name: str):
    """Exact shape (None = any extent) and a dense layout: the C side sees only
    the pointer and the sizes passed with it."""
    if t.dim() != len(shape) or any(d is not None and t.shape[i] != d for i, d in enumerate(shape)):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_dense(t: torch.Tensor, dtype, shape, name: str):
    _need(t, dtype, name)
    _need_shape(t, shape, name)


def _row_stride(t: torch.Tensor, row_extent: int) -> int:
    """Elements between consecutive rows; a one-row tensor may carry any stride
    (torch keeps 0 or odd strides on size-1 dimensions), so use the row extent."""
    if t.shape[0] <= 1:
        return max(row_extent, 1)
    return t.stride(0)


def _ld(t: torch.Tensor) -> int:
    return _row_stride(t, t.shape[1]) if t.dim() >= 2 else t.shape[-1]


def abi_version() -> int:
    return int(lib().bi_abi_version())


# ---------------------------------------------------------------------------
def bi_rmsnorm(x: torch.Tensor, w: torch.Tensor, eps: float, y: torch.Tensor = None,
               rstd: torch.Tensor = None, want_rstd: bool = True, stream=None):
    _need(x, torch.bfloat16, "x")
    M, H = x.shape
    _need_dense(w, torch.bfloat16, (H,), "w")
    if y is None:
        y = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, "y")
    if tuple(y.shape) != (M, H):
        raise ValueError(f"y must have shape {(M, H)}")
    if rstd is None and want_rstd:
        rstd = torch.empty((M,), dtype=torch.float32, device=x.device)
    if rstd is not None:
        _need_dense(rstd, torch.float32, (M,), "rstd")
    _check(lib().bi_rmsnorm(_ptr(x), _ld(x), _ptr(w), _ptr(y), _ld(y), _ptr(rstd), M, H,
                            float(eps), _stream(stream)), "bi_rmsnorm")
    return y, rstd


def bi_matmul(a: torch.Tensor, wt: torch.Tensor, out_dtype=torch.bfloat16, c: torch.Tensor = None,
              stream=None) -> torch.Tensor:
    """c = a @ wt.T with wt stored [N, K]."""
    _need(a, torch.bfloat16, "a"); _need(wt, torch.bfloat16, "wt")
    M, K = a.shape
    N, K2 = wt.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=a.device)
    code = BI_BF16 if c.dtype == torch.bfloat16 else BI_F32 if c.dtype == torch.float32 else None
    if code is None:
        raise ValueError("c must be bfloat16 or float32")
    _need(c, c.dtype, "c")
    if tuple(c.shape) != (M, N):
        raise ValueError(f"c must have shape {(M, N)}")
    _check(lib().bi_matmul(_ptr(a), _ld(a), _ptr(wt), _ld(wt), _ptr(c), _ld(c), code, M, N, K,
                           _stream(stream)), "bi_matmul")
    return c


def bi_addmm(a: torch.Tensor, wt: torch.Tensor, bias: torch.Tensor, out_dtype=torch.bfloat16,
             c: torch.Tensor = None, stream=None) -> torch.Tensor:
    """c = bias + a @ wt.T with wt stored [N, K], bias [N] (bf16)."""
    _need(a, torch.bfloat16, "a"); _need(wt, torch.bfloat16, "wt")
    M, K = a.shape
    N, K2 = wt.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    _need_dense(bias, torch.bfloat16, (N,), "bias")
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=a.device)
    code = BI_BF16 if c.dtype == torch.bfloat16 else BI_F32 if c.dtype == torch.float32 else None
    if code is None:
        raise ValueError("c must be bfloat16 or float32")
    _need(c, c.dtype, "c")
    if tuple(c.shape) != (M, N):
        raise ValueError(f"c must have shape {(M, N)}")
    _check(lib().bi_addmm(_ptr(a), _ld(a), _ptr(wt), _ld(wt), _ptr(bias), _ptr(c), _ld(c), code, M, N, K,
                          _stream(stream)), "bi_addmm")
    return c


def bi_kv_append(k_new: torch.Tensor, v_new: torch.Tensor, slots: torch.Tensor,
                 k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None):
    """k_new/v_new [T, Hkv, D] (rows may be strided views of a wider tensor)."""
    T, Hkv, D = k_new.shape
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, torch.bfloat16, n)
        if t.numel() and (t.stride(2) != 1 or (Hkv > 1 and t.stride(1) != D)):
            raise ValueError(f"{n}: heads must be contiguous [Hkv, D] inside a token row")
    ld = _row_stride(k_new, Hkv * D)
    if ld != _row_stride(v_new, Hkv * D):
        raise ValueError("k_new and v_new must share the row stride")
    _need_dense(slots, torch.int32, (T,), "slots")
    num_blocks = k_cache.shape[0]
    _need_dense(k_cache, torch.bfloat16, (num_blocks, Hkv, 16, D), "k_cache")
    _need_dense(v_cache, torch.bfloat16, (num_blocks, Hkv, D, 16), "v_cache")
    _check(lib().bi_kv_append(_ptr(k_new), _ptr(v_new), ld, _ptr(slots), T,
                              _ptr(k_cache), _ptr(v_cache), num_blocks, Hkv, D, _stream(stream)),
           "bi_kv_append")


def bi_attention_workspace_bytes(S: int, Hq: int, D: int, max_kv_len: int) -> int:
    return int(lib().bi_attention_workspace_bytes(S, Hq, D, max_kv_len))


def _heads_view(q: torch.Tensor, name: str):
    """[rows, H, D] view whose heads are contiguous inside a row; returns (H, D, ld)."""
    _need(q, torch.bfloat16, name)
    if q.dim() != 3:
        raise ValueError(f"{name} must be [rows, heads, head_dim]")
    rows, H, D = q.shape
    if q.numel() and (q.stride(2) != 1 or (H > 1 and q.stride(1) != D)):
        raise ValueError(f"{name}: heads must be contiguous [H, D] inside a row")
    return H, D, _row_stride(q, H * D)


def _check_paged(k_cache, v_cache, block_table, D):
    nb, Hkv = k_cache.shape[0], k_cache.shape[1]
    _need_dense(k_cache, torch.bfloat16, (nb, Hkv, 16, D), "k_cache")
    _need_dense(v_cache, torch.bfloat16, (nb, Hkv, D, 16), "v_cache")
    if block_table.dim() != 2:
        raise ValueError("block_table must be [S, max_blocks]")


def bi_attention_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        block_table: torch.Tensor, kv_lens: torch.Tensor, max_kv_len: int,
                        scale: float, ws: torch.Tensor = None, out: torch.Tensor = None,
                        stream=None) -> torch.Tensor:
    """q [S, Hq, D] (rows may be strided); k_cache [nblk, Hkv, 16, D]; returns out [S, Hq, D]."""
    S = q.shape[0]
    Hq, D, ldq = _heads_view(q, "q")
    Hkv = k_cache.shape[1]
    _check_paged(k_cache, v_cache, block_table, D)
    _need_dense(block_table, torch.int32, (S, None), "block_table")
    _need_dense(kv_lens, torch.int32, (S,), "kv_lens")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=q.device)
    _, _, ldo = _heads_view(out, "out")
    if tuple(out.shape) != (S, Hq, D):
        raise ValueError(f"out must have shape {(S, Hq, D)}")
    need = bi_attention_workspace_bytes(S, Hq, D, max_kv_len)
    if ws is None:
        ws = torch.empty((max(need, 16) + 3) // 4, dtype=torch.float32, device=q.device)
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous device tensor")
    _check(lib().bi_attention_decode(_ptr(q), ldq, _ptr(k_cache), _ptr(v_cache),
                                     k_cache.shape[0], _ptr(block_table), block_table.shape[1],
                                     _ptr(kv_lens), _ptr(out), ldo, S, Hq, Hkv, D,
                                     int(max_kv_len), float(scale), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
           "bi_attention_decode")
    return out


def bi_attention_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_table: torch.Tensor, kv_lens: torch.Tensor, max_kv_len: int,
                                scale: float, out: torch.Tensor, stream=None) -> torch.Tensor:
    """bi_attention_decode without a workspace argument (the library's own
    scratch holds the split partials); `out` [S, Hq, D] must be passed, so the
    call allocates nothing."""
    S = q.shape[0]
    Hq, D, ldq = _heads_view(q, "q")
    Hkv = k_cache.shape[1]
    _check_paged(k_cache, v_cache, block_table, D)
    _need_dense(block_table, torch.int32, (S, None), "block_table")
    _need_dense(kv_lens, torch.int32, (S,), "kv_lens")
    _, _, ldo = _heads_view(out, "out")
    if tuple(out.shape) != (S, Hq, D):
        raise ValueError(f"out must have shape {(S, Hq, D)}")
    L = lib()
    if not hasattr(L, "bi_attention_decode_noalloc"):
        raise RuntimeError(f"bi_attention_decode_noalloc is not exported by {LIB_PATH}")
    _check(L.bi_attention_decode_noalloc(_ptr(q), ldq, _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
                                         _ptr(block_table), block_table.shape[1], _ptr(kv_lens), _ptr(out),
                                         ldo, S, Hq, Hkv, D, int(max_kv_len), float(scale), _stream(stream)),
           "bi_attention_decode_noalloc")
    return out


def bi_attention_prefill(q: torch.Tensor, q_start: torch.Tensor, kv_lens: torch.Tensor,
                         k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                         max_q_len: int, scale: float, out: torch.Tensor = None,
                         stream=None) -> torch.Tensor:
    """q [T, Hq, D] (rows may be strided), rows grouped by q_start [S+1]; returns out [T, Hq, D]."""
    T = q.shape[0]
    Hq, D, ldq = _heads_view(q, "q")
    Hkv = k_cache.shape[1]
    _check_paged(k_cache, v_cache, block_table, D)
    _need_dense(q_start, torch.int32, (None,), "q_start")
    S = q_start.shape[0] - 1
    _need_dense(kv_lens, torch.int32, (S,), "kv_lens")
    _need_dense(block_table, torch.int32, (S, None), "block_table")
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=q.device)
    _, _, ldo = _heads_view(out, "out")
    if tuple(out.shape) != (T, Hq, D):
        raise ValueError(f"out must have shape {(T, Hq, D)}")
    _check(lib().bi_attention_prefill(_ptr(q), ldq, _ptr(q_start), _ptr(kv_lens),
                                      _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
                                      _ptr(block_table), block_table.shape[1], _ptr(out), ldo,
                                      S, T, Hq, Hkv, D, int(max_q_len), float(scale),
                                      _stream(stream)), "bi_attention_prefill")
    return out


def bi_argmax(logits: torch.Tensor, ids: torch.Tensor = None, stream=None) -> torch.Tensor:
    _need(logits, torch.float32, "logits")
    rows, V = logits.shape
    if ids is None:
        ids = torch.empty((rows,), dtype=torch.int32, device=logits.device)
    _need_dense(ids, torch.int32, (rows,), "ids")
    _check(lib().bi_argmax(_ptr(logits), _ld(logits), rows, V, _ptr(ids), _stream(stream)),
           "bi_argmax")
    return ids


def bi_mean(x: torch.Tensor, out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Row means of x [rows, H] (bf16) as fp32 [rows]."""
    _need(x, torch.bfloat16, "x")
    rows, H = x.shape
    if out is None:
        out = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _need_dense(out, torch.float32, (rows,), "out")
    _check(lib().bi_mean(_ptr(x), _ld(x), _ptr(out), rows, H, _stream(stream)), "bi_mean")
    return out


def bi_log_softmax(x: torch.Tensor, out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """log_softmax over the last dimension of x [rows, V] (fp32); out may be x."""
    _need(x, torch.float32, "x")
    rows, V = x.shape
    if out is None:
        out = torch.empty((rows, V), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, "out")
    if tuple(out.shape) != (rows, V):
        raise ValueError(f"out must have shape {(rows, V)}")
    _check(lib().bi_log_softmax(_ptr(x), _ld(x), _ptr(out), _ld(out), rows, V, _stream(stream)),
           "bi_log_softmax")
    return out


def bi_sample(logits: torch.Tensor, temperature: float, seeds: torch.Tensor, offsets: torch.Tensor,
              ids: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Seeded Gumbel-max sampling of each row of logits [rows, V] (fp32) at
    temperature > 0; seeds and offsets are uint64 [rows] (torch.int64 storage)."""
    _need(logits, torch.float32, "logits")
    rows, V = logits.shape
    _need_dense(seeds, torch.int64, (rows,), "seeds")
    _need_dense(offsets, torch.int64, (rows,), "offsets")
    if ids is None:
        ids = torch.empty((rows,), dtype=torch.int32, device=logits.device)
    _need_dense(ids, torch.int32, (rows,), "ids")
    _check(lib().bi_sample(_ptr(logits), _ld(logits), rows, V, float(temperature), _ptr(seeds),
                           _ptr(offsets), _ptr(ids), _stream(stream)), "bi_sample")
    return ids


def bi_top2(logits: torch.Tensor, stream=None):
    """(argmax ids int32 [rows], top1 - top2 margins fp32 [rows]) of logits [rows, V] fp32."""
    _need(logits, torch.float32, "logits")
    rows, V = logits.shape
    ids = torch.empty((rows,), dtype=torch.int32, device=logits.device)
    margin = torch.empty((rows,), dtype=torch.float32, device=logits.device)
    _check(lib().bi_top2(_ptr(logits), _ld(logits), rows, V, _ptr(ids), _ptr(margin), _stream(stream)),
           "bi_top2")
    return ids, margin


def bi_lm_head_f32(h: torch.Tensor, norm_w: torch.Tensor, eps: float, lm_head: torch.Tensor,
                   out: torch.Tensor = None, margin: torch.Tensor = None, threshold: float = 0.0,
                   stream=None) -> torch.Tensor:
    """fp32 logits [R, V] of h [R, H] (bf16, before the final norm) through the
    unrounded final norm and lm_head [V, H]; with margin [R], only rows whose
    margin is below threshold are written (the others of `out` are left)."""
    _need(h, torch.bfloat16, "h"); _need(lm_head, torch.bfloat16, "lm_head")
    _need_dense(norm_w, torch.bfloat16, (h.shape[1],), "norm_w")
    R, H = h.shape
    V, H2 = lm_head.shape
    if H != H2:
        raise ValueError("hidden sizes differ")
    if out is None:
        out = torch.empty((R, V), dtype=torch.float32, device=h.device)
    _need_dense(out, torch.float32, (R, V), "out")
    if margin is not None:
        _need_dense(margin, torch.float32, (R,), "margin")
    _check(lib().bi_lm_head_f32(_ptr(h), _ld(h), _ptr(norm_w), float(eps), _ptr(lm_head), _ld(lm_head),
                                _ptr(out), _ld(out), R, V, H, _ptr(margin) if margin is not None else None,
                                float(threshold), _stream(stream)), "bi_lm_head_f32")
    return out


def bi_probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    for t, n in ((src, "src"), (dst, "dst")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    _check(lib().bi_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "bi_probe_copy")


# words of the probes' sink array (BI_PROBE_SINK_WORDS in include/bi.h)
PROBE_SINK_WORDS = 8192


def _probe_sink(sink: Optional[torch.Tensor], device) -> torch.Tensor:
    if sink is None:
        return torch.zeros(PROBE_SINK_WORDS, dtype=torch.int32, device=device)
    _need_dense(sink, torch.int32, (PROBE_SINK_WORDS,), "sink")
    return sink


def bi_probe_read(src: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Streams src once (achievable HBM read rate); returns the sink words,
    whose xor is the xor of src's 32-bit words (words past the grid stay 0)."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    sink = _probe_sink(sink, src.device)
    _check(lib().bi_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)),
           "bi_probe_read")
    return sink


def bi_probe_lds_fill(src: torch.Tensor, span_bytes: int, workgroups: int, iters: int,
                      sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Global -> LDS fill of workgroups * 8 * iters * 8 KB from the first
    span_bytes of src (include/bi.h)."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    if span_bytes > src.numel() * src.element_size():
        raise ValueError("span beyond src")
    sink = _probe_sink(sink, src.device)
    _check(lib().bi_probe_lds_fill(_ptr(src), int(span_bytes), int(workgroups), int(iters), _ptr(sink),
                                   _stream(stream)), "bi_probe_lds_fill")
    return sink


def bi_probe_mfma_bf16(a: torch.Tensor, b: torch.Tensor, stream=None) -> torch.Tensor:
    _need_dense(a, torch.bfloat16, (16, 32), "a")
    _need_dense(b, torch.bfloat16, (32, 16), "b")
    c = torch.empty((16, 16), dtype=torch.float32, device=a.device)
    _check(lib().bi_probe_mfma_bf16(_ptr(a), _ptr(b), _ptr(c), _stream(stream)), "bi_probe_mfma_bf16")
    return c


# ---------------------------------------------------------------------------
# include/bi_toy.h element-wise ops
# ---------------------------------------------------------------------------

def bi_embed(table: torch.Tensor, ids: torch.Tensor, out: torch.Tensor = None, stream=None):
    _need(table, torch.bfloat16, "table")
    V, H = table.shape
    _need_shape(table, (V, H), "table")
    _need_dense(ids, torch.int32, (None,), "ids")
    T = ids.shape[0]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=table.device)
    _check(lib().bi_embed(_ptr(table), V, H, _ptr(ids), T, _ptr(out), _ld(out), _stream(stream)),
           "bi_embed")
    return out


def bi_rope_table(max_pos: int, D: int, theta: float, stream=None) -> torch.Tensor:
    t = torch.empty((max_pos * D,), dtype=torch.float32, device="cuda")
    _check(lib().bi_rope_table(_ptr(t), max_pos, D, float(theta), _stream(stream)), "bi_rope_table")
    return t


def bi_rope(x: torch.Tensor, pos: torch.Tensor, table: torch.Tensor, max_pos: int, stream=None):
    """In place on x [T, H, D] (rows may be strided)."""
    H, D, ld = _heads_view(x, "x")
    _need_dense(pos, torch.int32, (x.shape[0],), "pos")
    _need_dense(table, torch.float32, (max_pos * D,), "table")
    _check(lib().bi_rope(_ptr(x), ld, H, D, _ptr(pos), x.shape[0], _ptr(table), max_pos,
                         _stream(stream)), "bi_rope")
    return x


def bi_add(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor = None, stream=None):
    _need_dense(a, torch.bfloat16, tuple(a.shape), "a")
    _need_dense(b, torch.bfloat16, tuple(a.shape), "b")
    if out is None:
        out = torch.empty_like(a)
    _need_dense(out, torch.bfloat16, tuple(a.shape), "out")
    _check(lib().bi_add(_ptr(a), _ptr(b), _ptr(out), a.numel(), _stream(stream)), "bi_add")
    return out


def bi_rope_kv_append(qkv: torch.Tensor, Hq: int, Hkv: int, pos: torch.Tensor, slots: torch.Tensor,
                      table: torch.Tensor, max_pos: int, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      stream=None):
    """qkv [T, >= (Hq + 2 Hkv) D]: q and k heads rotated in place, k and v
    appended to the paged cache at slots."""
    T, D = qkv.shape[0], k_cache.shape[-1]
    _need(qkv, torch.bfloat16, "qkv")
    _need_dense(pos, torch.int32, (T,), "pos")
    _need_dense(slots, torch.int32, (T,), "slots")
    _check(lib().bi_rope_kv_append(_ptr(qkv), _ld(qkv), Hq, Hkv, D, _ptr(pos), _ptr(slots), T, _ptr(table),
                                   int(max_pos), _ptr(k_cache), _ptr(v_cache), k_cache.shape[0], _stream(stream)),
           "bi_rope_kv_append")


def bi_add_rmsnorm(h: torch.Tensor, r: torch.Tensor, w: torch.Tensor, eps: float, y: torch.Tensor = None,
                   want_rstd: bool = True, stream=None):
    """h [M, H] <- bf16(h + r) in place, then (y, rstd) = RMSNorm of the new h."""
    M, H = h.shape
    _need_dense(h, torch.bfloat16, (M, H), "h")
    _need_dense(r, torch.bfloat16, (M, H), "r")
    _need_dense(w, torch.bfloat16, (H,), "w")
    if y is None:
        y = torch.empty_like(h)
    _need_dense(y, torch.bfloat16, (M, H), "y")
    rstd = torch.empty((M,), dtype=torch.float32, device=h.device) if want_rstd else None
    _check(lib().bi_add_rmsnorm(_ptr(h), _ld(h), _ptr(r), _ld(r), _ptr(w), _ptr(y), _ld(y),
                                _ptr(rstd) if rstd is not None else None, M, H, float(eps), _stream(stream)),
           "bi_add_rmsnorm")
    return y, rstd


def bi_silu_mul(gu: torch.Tensor, out: torch.Tensor = None, stream=None):
    """gu [T, 2F] (gate | up) -> out [T, F]."""
    _need(gu, torch.bfloat16, "gu")
    T, F2 = gu.shape
    F = F2 // 2
    if out is None:
        out = torch.empty((T, F), dtype=torch.bfloat16, device=gu.device)
    _check(lib().bi_silu_mul(_ptr(gu), _ld(gu), F, _ptr(out), _ld(out), T, _stream(stream)),
           "bi_silu_mul")
    return out


def bi_gather_rows(src: torch.Tensor, rows: torch.Tensor, out: torch.Tensor = None, stream=None):
    _need(src, torch.bfloat16, "src"); _need(rows, torch.int32, "rows")
    n, W = src.shape
    R = rows.shape[0]
    if out is None:
        out = torch.empty((R, W), dtype=torch.bfloat16, device=src.device)
    _check(lib().bi_gather_rows(_ptr(src), _ld(src), n, _ptr(rows), R, W, _ptr(out), _ld(out),
                                _stream(stream)), "bi_gather_rows")
    return out
