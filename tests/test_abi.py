"""The C ABI: libbi.so builds for gfx950, loads, exports every symbol that
include/bi.h declares, and its host-side validation rejects bad arguments
before any launch (so these run without a GPU: no compute call is made)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def declared_symbols():
    syms = set()
    for name in sorted(os.listdir(INCLUDE)):
        if name.endswith(".h"):
            text = open(os.path.join(INCLUDE, name)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            syms |= set(re.findall(r"\b(bi_[a-z0-9_]+)\s*\(", text))
    return sorted(syms)


@pytest.fixture(scope="module")
def L():
    from invariant_bi_rmsnorm_amd import ops
    if not os.path.exists(ops.LIB_PATH):
        from invariant_bi_rmsnorm_amd import _build
        _build.build()
    return ops.lib()


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ("bi_rmsnorm", "bi_matmul", "bi_kv_append", "bi_attention_decode",
              "bi_attention_prefill", "bi_attention_workspace_bytes", "bi_argmax"):
        assert s in syms


def test_library_exports_every_declared_symbol(L):
    from invariant_bi_rmsnorm_amd import ops
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(bi_[a-z0-9_]+)$", out, flags=re.M))
    for s in declared_symbols():
        assert s in exported, s
        assert hasattr(L, s)
    assert set(ops.SIGNATURES) == set(declared_symbols())


def test_library_links_no_oracle_code(L):
    from invariant_bi_rmsnorm_amd import ops
    out = subprocess.run(["nm", "-D", ops.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert not re.search(r"\bor_(rmsnorm|matmul|attention|argmax)", out)
    ldd = subprocess.run(["ldd", ops.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in ldd


def test_gfx950_code_object_present():
    from invariant_bi_rmsnorm_amd import ops
    data = open(ops.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", data))
    assert targets == {b"gfx950"}


def test_version_and_status_strings(L):
    from invariant_bi_rmsnorm_amd import ops
    assert ops.abi_version() == 1
    assert ops.status_string(0) == "ok"
    assert "unsupported" in ops.status_string(2)
    assert ops.status_string(99) == "unknown status"


def test_missing_library_fails_loudly(tmp_path):
    code = ("import os; os.environ['BI_LIB']='/nonexistent/libbi.so'\n"
            "from invariant_bi_rmsnorm_amd import ops\n"
            "try:\n    ops.lib()\nexcept RuntimeError as e:\n    print('RAISED', e)\n")
    r = subprocess.run(["python", "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert "RAISED" in r.stdout and "no fallback" in r.stdout


# Fake, never-dereferenced "device" addresses: validation must fail first.
A16 = 0x10000          # 16-byte aligned
MIS = 0x10002          # misaligned


def test_rmsnorm_validation(L):
    f = L.bi_rmsnorm
    assert f(A16, 4096, A16, A16, 4096, None, 0, 4096, 1e-6, None) == 0       # M == 0 no-op
    assert f(None, 4096, A16, A16, 4096, None, 4, 4096, 1e-6, None) == 1      # null x
    assert f(A16, 4000, A16, A16, 4096, None, 4, 4096, 1e-6, None) == 1      # ldx < H
    assert f(MIS, 4096, A16, A16, 4096, None, 4, 4096, 1e-6, None) == 1      # misaligned
    assert f(A16, 4096, A16, A16, 4096, None, -1, 4096, 1e-6, None) == 1     # negative M
    assert f(A16, 4096, A16, A16, 4096, None, 4, 4096, -1.0, None) == 1      # eps < 0
    assert f(A16, 4104, A16, A16, 4104, None, 4, 4100, 1e-6, None) == 2      # H % 8
    assert f(A16, 32768, A16, A16, 32768, None, 4, 32768, 1e-6, None) == 2   # H too large


def test_matmul_validation(L):
    f = L.bi_matmul
    assert f(A16, 4096, A16, 4096, A16, 4096, 0, 0, 4096, 4096, None) == 0    # M == 0
    assert f(None, 4096, A16, 4096, A16, 4096, 0, 8, 4096, 4096, None) == 1
    assert f(A16, 4096, A16, 4096, A16, 4096, 7, 8, 4096, 4096, None) == 1    # bad dtype
    assert f(A16, 4096, A16, 4000, A16, 4096, 0, 8, 4096, 4096, None) == 1    # ldw < K
    assert f(A16, 4096, A16, 4096, MIS, 4096, 1, 8, 4096, 4096, None) == 1    # fp32 c misaligned
    assert f(A16, 4128, A16, 4128, A16, 4096, 0, 8, 4096, 4100, None) == 2    # K % 64
    assert f(A16, 4096, A16, 4096, A16, 4098, 0, 8, 4098, 4096, None) == 1    # ldc % 4
    assert f(A16, 4096, A16, 4096, A16, 4096, 0, 8, 4094, 4096, None) == 2    # N % 4
    # sizes the kernels' 32-bit tile arithmetic cannot hold (tiles up to 256 tall, down to 16 x 16)
    assert f(A16, 4096, A16, 4096, A16, 4096, 0, 2**31 - 200, 4096, 4096, None) == 2
    assert f(A16, 4096, A16, 4096, A16, 1 << 20, 0, 1 << 20, 1 << 20, 4096, None) == 2
    assert f(A16, 1 << 24, A16, 4096, A16, 4096, 0, 8, 4096, 4096, None) == 2    # lda >= 2^24


def test_kv_append_validation(L):
    f = L.bi_kv_append
    assert f(A16, A16, 1024, A16, 0, A16, A16, 10, 8, 128, None) == 0
    assert f(A16, A16, 1000, A16, 3, A16, A16, 10, 8, 128, None) == 1      # ld < Hkv*D
    assert f(A16, A16, 1024, A16, 3, A16, A16, 10, 8, 64, None) == 2       # D != 128
    assert f(None, A16, 1024, A16, 3, A16, A16, 10, 8, 128, None) == 1


def test_attention_validation(L):
    ws = L.bi_attention_workspace_bytes(4, 32, 128, 1000)
    # alignment slack, work counter, then per split and query head a 128-float o
    # row and (for Hkv == Hq, the bound) a 32-float (m, l) line
    assert ws == 255 + 256 + 4 * 32 * 4 * (128 + 32) * 4
    dec = L.bi_attention_decode
    args = [A16, 4096, A16, A16, 100, A16, 64, A16, A16, 4096, 4, 32, 8, 128, 1000, 0.088, A16, ws, None]
    bad = list(args); bad[17] = ws - 4
    assert dec(*bad) == 3                                     # workspace too small
    bad = list(args); bad[12] = 6
    assert dec(*bad) == 1                                     # Hq % Hkv
    bad = list(args); bad[13] = 64
    assert dec(*bad) == 2                                     # D != 128
    bad = list(args); bad[14] = 64 * 16 + 1
    assert dec(*bad) == 1                                     # max_kv_len > capacity
    bad = list(args); bad[10] = 0
    assert dec(*bad) == 0                                     # S == 0
    bad = list(args); bad[11] = 512; bad[12] = 512; bad[1] = bad[9] = 512 * 128
    assert dec(*bad) == 2                                     # Hkv > 256
    # (split, KV head) work items beyond 2^30: refused before any device call
    huge = list(args); huge[10] = 2048; huge[11] = 256; huge[12] = 256; huge[1] = huge[9] = 256 * 128
    huge[6] = 1 << 16; huge[14] = 1 << 20; huge[17] = L.bi_attention_workspace_bytes(2048, 256, 128, 1 << 20)
    assert dec(*huge) == 2
    pre = L.bi_attention_prefill
    pargs = [A16, 4096, A16, A16, A16, A16, 100, A16, 64, A16, 4096, 2, 300, 32, 8, 128, 200, 0.088, None]
    bad = list(pargs); bad[14] = 3
    assert pre(*bad) == 1                                     # Hq % Hkv
    bad = list(pargs); bad[13] = 24; bad[14] = 8
    assert pre(*bad) == 2                                     # group 3 unsupported
    bad = list(pargs); bad[12] = 0
    assert pre(*bad) == 0                                     # T == 0
    bad = list(pargs); bad[8] = 4097
    assert pre(*bad) == 2                                     # block table wider than 4096


def test_attention_decode_noalloc_validation(L):
    """The allocation-free decode rejects, on the host and before any device
    call, what bi_attention_decode rejects, plus any call whose split partials
    would not fit the library's 64 MiB scratch."""
    from invariant_bi_rmsnorm_amd import ops
    f = L.bi_attention_decode_noalloc
    args = [A16, 4096, A16, A16, 100, A16, 2048, A16, A16, 4096, 4, 32, 8, 128, 1000, 0.088, None]
    bad = list(args); bad[12] = 6
    assert f(*bad) == 1                                       # Hq % Hkv
    bad = list(args); bad[13] = 64
    assert f(*bad) == 2                                       # D != 128
    bad = list(args); bad[0] = None
    assert f(*bad) == 1                                       # null q
    bad = list(args); bad[10] = 0
    assert f(*bad) == 0                                       # S == 0: no-op
    # the limit: the work counter (with alignment slack) and S * Hq *
    # ceil(max_kv_len / 256) rows of 128 + 32 floats in 64 MiB
    assert ops.NOALLOC_SCRATCH_BYTES == 64 << 20
    limit_splits = (ops.NOALLOC_SCRATCH_BYTES - 511) // (160 * 4)
    assert limit_splits == 104856
    assert L.bi_attention_workspace_bytes(1, 1, 128, 256 * limit_splits) <= ops.NOALLOC_SCRATCH_BYTES
    assert L.bi_attention_workspace_bytes(1, 1, 128, 256 * (limit_splits + 1)) > ops.NOALLOC_SCRATCH_BYTES
    big = list(args); big[10] = 256; big[14] = 32768          # 256 * 32 * 128 splits
    assert L.bi_attention_workspace_bytes(256, 32, 128, 32768) > ops.NOALLOC_SCRATCH_BYTES
    assert f(*big) == 3                                       # BI_ERR_WORKSPACE_TOO_SMALL
    edge = list(args); edge[10] = 63; edge[14] = 2048 * 16    # 63 * 32 * 128 = 258048 splits: too many
    assert f(*edge) == 3


def test_probe_copy_validation(L):
    assert L.bi_probe_copy(A16, A16, 0, None) == 0
    assert L.bi_probe_copy(A16, A16, 17, None) == 1
    assert L.bi_probe_copy(MIS, A16, 32, None) == 1


def test_rope_kv_append_validation(L):
    f = L.bi_rope_kv_append
    ld = (16 + 2 * 4) * 128
    ok = (A16, ld, 16, 4, 128, A16, A16, 3, A16, 64, A16, A16, 10, None)
    assert f(*ok[:7], 0, *ok[8:]) == 0                                    # T == 0: no-op
    assert f(A16, ld - 8, *ok[2:]) == 1                                    # ld too small
    assert f(A16, ld + 4, *ok[2:]) == 1                                    # ld % 8
    assert f(MIS, *ok[1:]) == 1                                            # misaligned qkv
    assert f(*ok[:5], None, *ok[6:]) == 1                                  # no positions
    assert f(*ok[:4], 64, *ok[5:]) == 2                                    # D != 128
    assert f(*ok[:12], 0, None) == 1                                       # empty pool


def test_add_rmsnorm_validation(L):
    f = L.bi_add_rmsnorm
    assert f(A16, 64, A16, 64, A16, A16 + 4096, 64, None, 0, 64, 1e-6, None) == 0      # M == 0: no-op
    assert f(A16, 64, A16, 63, A16, A16 + 4096, 64, None, 2, 64, 1e-6, None) == 1      # ldr < H
    assert f(A16, 64, None, 64, A16, A16 + 4096, 64, None, 2, 64, 1e-6, None) == 1     # no r
    assert f(A16, 64, MIS, 64, A16, A16 + 4096, 64, None, 2, 64, 1e-6, None) == 1      # misaligned r
    assert f(A16, 64, A16, 64, A16, A16, 64, None, 2, 64, 1e-6, None) == 1             # y == h
    assert f(A16, 64, A16, 64, A16, A16 + 4096, 64, None, 2, 60, 1e-6, None) == 2      # H % 8
    assert f(A16, 64, A16, 64, A16, A16 + 4096, 64, None, 2, 64, -1.0, None) == 1      # eps < 0


def test_probe_read_and_lds_fill_validation(L):
    assert L.bi_probe_read(A16, 0, A16, None) == 0
    assert L.bi_probe_read(A16, 17, A16, None) == 1
    assert L.bi_probe_read(MIS, 32, A16, None) == 1
    assert L.bi_probe_read(A16, 32, None, None) == 1
    f = L.bi_probe_lds_fill
    assert f(A16, 1000, 1, 1, A16, None) == 1          # span not a whole number of KB
    assert f(A16, 0, 1, 1, A16, None) == 1
    assert f(A16, 1024, 0, 1, A16, None) == 1
    assert f(A16, 1024, 8193, 1, A16, None) == 1        # more workgroups than sink words
    assert f(A16, 1024, 1, 0, A16, None) == 1
    assert f(MIS, 1024, 1, 1, A16, None) == 1
    assert f(A16, 1024, 1, 1, None, None) == 1


def test_argmax_validation(L):
    f = L.bi_argmax
    assert f(A16, 100, 0, 100, A16, None) == 0
    assert f(A16, 99, 2, 100, A16, None) == 1
    assert f(None, 100, 2, 100, A16, None) == 1


def test_lm_head_f32_validation(L):
    f = L.bi_lm_head_f32
    nan = float("nan")

    def call(h=A16, ldh=2048, w=A16, eps=1e-6, W=A16, ldw=2048, out=A16, ldo=100, R=2, V=100, H=2048,
             margin=None, thr=0.1):
        return f(h, ldh, w, eps, W, ldw, out, ldo, R, V, H, margin, thr, None)
    assert call(R=0) == 0
    assert call(R=-1) == 1
    assert call(ldo=99) == 1 and call(ldh=2047) == 1 and call(ldw=1024) == 1
    assert call(eps=-1.0) == 1 and call(eps=nan) == 1 and call(thr=nan) == 1
    assert call(h=MIS) == 1 and call(W=None) == 1 and call(margin=MIS) == 1
    assert call(H=2000) == 2                 # H % 512
    assert call(ldh=8192, ldw=8192, H=8192) == 2
    assert call(R=70000) == 2


def test_toy_entry_validation(L):
    assert L.bi_embed(A16, 10, 64, A16, 0, A16, 64, None) == 0
    assert L.bi_embed(None, 10, 64, A16, 3, A16, 64, None) == 1
    assert L.bi_embed(A16, 10, 60, A16, 3, A16, 64, None) == 2            # H % 8
    assert L.bi_add(A16, A16, A16, 12, None) == 2                          # n % 8
    assert L.bi_add(A16, None, A16, 16, None) == 1
    assert L.bi_silu_mul(A16, 100, 64, A16, 64, 2, None) == 1              # ldgu < 2F
    assert L.bi_rope(A16, 100, 1, 128, A16, 2, A16, 10, None) == 1         # ldx < H*D
    assert L.bi_rope_table(None, 10, 128, 10000.0, None) == 1
    assert L.bi_gather_rows(A16, 64, 5, A16, 2, 64, A16, 60, None) == 1    # ldd < W
    assert L.bi_toy_workspace_bytes(None, 10, 2, 100) == 0
    assert L.bi_toy_step(None, None, None, None, 0, None, None, None) == 1


def test_toy_step_logit_rows_validation(L):
    """n_logit_rows: 0 means S; otherwise S <= R <= T, checked before anything
    runs (fake device pointers; every call here returns on the host)."""
    import ctypes
    from invariant_bi_rmsnorm_amd import inputs as I
    from invariant_bi_rmsnorm_amd.toy import _Cfg, _Step, _Weights
    c = I.TOY
    cfg = _Cfg(c["layers"], c["hidden"], c["heads"], c["kv_heads"], c["head_dim"], c["mlp"], c["vocab"],
               1024, float(c["eps"]), float(c["rope_theta"]))
    w = _Weights(A16, A16, A16, A16, A16, A16, 16, A16)

    def step(R, ws_bytes=0, margin=0.0):
        st = _Step(4, 2, 0, 2, 16, 1, A16, A16, A16, A16, A16, A16, A16, R, margin)
        return L.bi_toy_step(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(st), A16, ws_bytes, A16, None, None)
    for bad in (-1, 1, 5):                      # negative, below S, above T
        assert step(bad) == 1, bad
    assert step(0, margin=-0.5) == 1 and step(0, margin=float("nan")) == 1
    assert step(0, margin=float("inf")) == 3 and step(0, margin=0.05) == 3
    for ok in (0, 2, 3, 4):                     # accepted, then the empty workspace is too small
        assert step(ok) == 3, ok
    need = L.bi_toy_workspace_bytes(ctypes.byref(cfg), 4, 4, 16)
    assert need > L.bi_toy_workspace_bytes(ctypes.byref(cfg), 4, 2, 16) > 0


def test_binding_shape_checks():
    """The binding refuses tensors whose shape, dtype or layout disagrees with
    what it passes to the C side (the library sees only pointers and sizes)."""
    import torch
    from invariant_bi_rmsnorm_amd import ops
    ops._need_shape(torch.zeros(2, 3), (2, None), "x")
    with pytest.raises(ValueError):
        ops._need_shape(torch.zeros(2, 3), (3, None), "x")
    with pytest.raises(ValueError):
        ops._need_shape(torch.zeros(2, 3), (2, 3, 1), "x")
    with pytest.raises(ValueError):
        ops._need_shape(torch.zeros(3, 2).t(), (2, 3), "x")           # not contiguous
    with pytest.raises(ValueError):
        ops._need(torch.zeros(2, 3, dtype=torch.bfloat16), torch.bfloat16, "x")   # host tensor


def test_log_softmax_validation(L):
    f = L.bi_log_softmax
    assert f(A16, 100, A16, 100, 0, 100, None) == 0            # rows == 0 no-op
    assert f(A16, 99, A16, 100, 4, 100, None) == 1             # ldx < V
    assert f(A16, 100, A16, 99, 4, 100, None) == 1             # ldy < V
    assert f(A16, 100, A16, 100, 4, 0, None) == 1              # V == 0
    assert f(None, 100, A16, 100, 4, 100, None) == 1           # null x
    assert f(A16 + 2, 100, A16, 100, 4, 100, None) == 1        # misaligned
    assert f(A16, 100, A16, 128, 4, 100, None) == 1            # in place with different ld


def test_sample_validation(L):
    f = L.bi_sample
    assert f(A16, 100, 0, 100, 1.0, A16, A16, A16, None) == 0          # rows == 0
    assert f(A16, 99, 2, 100, 1.0, A16, A16, A16, None) == 1           # ld < V
    assert f(A16, 100, 2, 100, 0.0, A16, A16, A16, None) == 1          # T == 0 (use argmax)
    assert f(A16, 100, 2, 100, -1.0, A16, A16, A16, None) == 1
    assert f(A16, 100, 2, 100, float("inf"), A16, A16, A16, None) == 1
    assert f(A16, 100, 2, 100, float("nan"), A16, A16, A16, None) == 1
    assert f(A16, 100, 2, 100, 1.0, None, A16, A16, None) == 1         # null seeds
    assert f(A16, 100, 2, 100, 1.0, A16 + 4, A16, A16, None) == 1      # misaligned seeds


def test_top2_validation(L):
    f = L.bi_top2
    assert f(A16, 100, 0, 100, A16, A16, None) == 0
    assert f(A16, 99, 2, 100, A16, A16, None) == 1
    assert f(A16, 100, 2, 100, A16, None, None) == 1
    assert f(A16 + 2, 100, 2, 100, A16, A16, None) == 1


def test_mean_validation(L):
    f = L.bi_mean
    assert f(A16, 4096, A16, 0, 4096, None) == 0
    assert f(A16, 4000, A16, 2, 4096, None) == 1       # ldx < H
    assert f(MIS, 4096, A16, 2, 4096, None) == 1
    assert f(A16, 4100, A16, 2, 4100, None) == 1       # ldx % 8
    assert f(A16, 4096, A16, 2, 4092, None) == 2       # H % 8
    assert f(A16, 32768, A16, 2, 32768, None) == 2     # H > 16384


def test_addmm_validation(L):
    f = L.bi_addmm
    assert f(A16, 4096, A16, 4096, A16, A16, 4096, 0, 0, 8, 4096, None) == 0     # M == 0
    assert f(A16, 4096, A16, 4096, None, A16, 4096, 0, 4, 8, 4096, None) == 1    # null bias
    assert f(A16, 4096, A16, 4096, A16 + 4, A16, 4096, 0, 4, 8, 4096, None) == 1  # bias misaligned
    assert f(A16, 4096, A16, 4000, A16, A16, 4096, 0, 4, 8, 4096, None) == 1     # ldw < K
