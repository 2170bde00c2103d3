"""Host-side checks of the C ABI (CPU only: no kernel is launched).

The library must load without a GPU, export every function include/tp_mlp.h
declares, and reject bad arguments with the documented status before making
any HIP call.
"""
import ctypes
import os
import re

import pytest

from tensor_transformer_layer_fwd_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_mlp.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(tp_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def test_header_and_binding_agree():
    names = declared_functions()
    assert "tp_column_linear_fwd" in names and "tp_reduce_partials" in names
    assert set(names) == set(L.SIGNATURES), set(names) ^ set(L.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in L.STATUS.items():
        assert L.tp_status_string(code).startswith(name)
    assert L.tp_status_string(12345) == "unknown tp_status"
    assert L.tp_last_hip_error() == 0


def test_workspace_size_query(lib):
    n = L.tp_linear_bwd_wgrad_workspace_size(4096, 1536, 768, L.TP_BF16)
    assert n > 0 and n % 4 == 0
    # fp32 needs only the column-sum partials: ceil(T/64) * n floats
    assert L.tp_linear_bwd_wgrad_workspace_size(512, 24, 12, L.TP_F32) == 8 * 12 * 4
    assert L.tp_linear_bwd_wgrad_workspace_size(64, 24, 12, L.TP_F32) == 0
    out = ctypes.c_size_t(7)
    assert lib.tp_linear_bwd_wgrad_workspace_size(0, 5, 5, L.TP_BF16, ctypes.byref(out)) == -2
    assert lib.tp_linear_bwd_wgrad_workspace_size(5, 5, 5, 7, ctypes.byref(out)) == -3
    assert lib.tp_linear_bwd_wgrad_workspace_size(5, 5, 5, 1, None) == -1
    for q in (lib.tp_linear_bwd_workspace_size, lib.tp_mlp_bwd_workspace_size):
        assert q(0, 5, 5, L.TP_BF16, ctypes.byref(out)) == -2
        assert q(5, 5, 5, 7, ctypes.byref(out)) == -3
        assert q(5, 5, 5, 1, None) == -1


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation


def test_column_fwd_validation(lib):
    f = lib.tp_column_linear_fwd
    ok = dict(X=FAKE, A=FAKE, b=None, Y=FAKE, U=FAKE, T=8, h=4, n=4, ldx=4, lda=4, ldy=4,
              dt=1, act=1)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["X"], a["A"], a["b"], a["Y"], a["U"], a["T"], a["h"], a["n"], a["ldx"],
                 a["lda"], a["ldy"], a["dt"], a["act"], None)

    assert call(X=None) == -1
    assert call(Y=None) == -1
    assert call(U=None) == -1            # GeLU needs the pre-activation buffer
    assert call(dt=2) == -3
    assert call(act=9) == -4
    assert call(T=0) == -2
    assert call(n=-1) == -2
    assert call(h=1 << 31) == -2
    assert call(ldx=3) == -2
    assert call(lda=3) == -2
    assert call(ldy=3) == -2


def test_other_entry_points_validation(lib):
    assert lib.tp_row_linear_fwd_partial(FAKE, FAKE, None, 8, 4, 4, 4, 4, 4, 1, None) == -1
    assert lib.tp_row_linear_fwd_partial(FAKE, FAKE, FAKE, 8, 4, 4, 3, 4, 4, 1, None) == -2
    assert lib.tp_row_linear_fwd_partial(FAKE, FAKE, FAKE, 8, 4, 4, 4, 4, 4, 5, None) == -3
    d = lib.tp_linear_bwd_dgrad
    assert d(FAKE, FAKE, None, 1, FAKE, 8, 4, 4, 4, 4, 4, 4, 1, 1, None) == -1  # GeLU needs U
    assert d(FAKE, FAKE, FAKE, 3, FAKE, 8, 4, 4, 4, 4, 4, 4, 1, 1, None) == -4
    assert d(FAKE, FAKE, FAKE, 1, FAKE, 8, 4, 4, 4, 4, 4, 4, 0, 1, None) == -3  # f32 in, bf16 out
    assert d(FAKE, FAKE, FAKE, 1, FAKE, 8, 4, 4, 4, 4, 3, 4, 1, 1, None) == -2  # ld_u < k
    assert d(FAKE, FAKE, None, 0, FAKE, 8, 4, 4, 4, 3, 4, 4, 1, 0, None) == -2  # ld_w < n
    w = lib.tp_linear_bwd_wgrad
    assert w(FAKE, FAKE, None, None, 8, 4, 4, 4, 4, 4, 0, 1, None, 0, None) == -1
    assert w(FAKE, FAKE, FAKE, None, 8, 4, 4, 4, 4, 3, 0, 1, None, 0, None) == -2
    # a shape that needs split-K partials, with no workspace
    need = L.tp_linear_bwd_wgrad_workspace_size(4096, 256, 256, L.TP_BF16)
    assert need > 0
    assert w(FAKE, FAKE, FAKE, None, 4096, 256, 256, 256, 256, 256, 0, 1, None, 0, None) == -5
    assert w(FAKE, FAKE, FAKE, None, 4096, 256, 256, 256, 256, 256, 0, 1, FAKE, 64, None) == -5
    # bias gradient over more than one row chunk needs the column-sum partials
    assert w(FAKE, FAKE, FAKE, FAKE, 1000, 4, 4, 4, 4, 4, 0, 0, None, 0, None) == -5
    assert w(FAKE, FAKE, FAKE, FAKE, 65, 4, 4, 4, 4, 4, 0, 0, None, 0, None) == -5
    r = lib.tp_reduce_partials
    arr = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert r(None, 2, None, FAKE, 8, 4, 4, 4, 1, None) == -1
    assert r(arr, 0, None, FAKE, 8, 4, 4, 4, 1, None) == -2
    assert r(arr, 17, None, FAKE, 8, 4, 4, 4, 1, None) == -2
    assert r(arr, 2, None, FAKE, 8, 4, 3, 4, 1, None) == -2
    assert r(arr, 2, None, FAKE, 8, 4, 4, 4, 2, None) == -3
    arr0 = (ctypes.c_void_p * 2)(0x1000, None)
    assert r(arr0, 2, None, FAKE, 8, 4, 4, 4, 1, None) == -1
    b = lib.tp_bias_act
    assert b(FAKE, None, None, 8, 4, 4, 4, 0, 1, 1, None) == -1
    assert b(FAKE, None, FAKE, 8, 4, 4, 4, 0, 1, 5, None) == -4
    assert b(FAKE, None, FAKE, 8, 4, 3, 4, 0, 1, 1, None) == -2


def test_gemm_plan_query(lib):
    # the workloads' products all land on the pipelined kernels
    for M, N, K in [(4096, 1536, 768), (4096, 768, 1536), (2048, 6144, 12288),
                    (2048, 12288, 6144), (6144, 1024, 256)]:
        tile, sk, kc = L.tp_gemm_plan(M, N, K)
        assert tile in (10, 11, 12, 13, 14, 15) and sk == 1 and kc == K
    tile, sk, kc = L.tp_gemm_plan(768, 1536, 4096, allow_split=True)
    assert tile >= 10 and sk >= 1 and kc * sk == 4096 and kc % 64 == 0
    # ragged shapes use the general kernel
    assert L.tp_gemm_plan(680, 1536, 768)[0] == 0
    assert L.tp_gemm_plan(4096, 1536, 700)[0] == 0
    # the plan never splits without permission and agrees with the workspace size
    for M, N, K in [(768, 1536, 4096), (256, 256, 4096), (1536, 768, 4096)]:
        tile, sk, kc = L.tp_gemm_plan(M, N, K, allow_split=True)
        ws = L.tp_linear_bwd_wgrad_workspace_size(K, M, N, L.TP_BF16)
        assert ws >= (sk * M * N * 4 if sk > 1 else 0)
        assert L.tp_gemm_plan(M, N, K, allow_split=False)[1] == 1
    assert lib.tp_gemm_plan(0, 5, 5, 0, None, None, None) == -2


def test_linear_bwd_plan(lib):
    """The pairing query: shape-only, agreeing with the workspace query."""
    # the MLP layers of the GPT-2-small shard (T=4096, h=768, F=1536) and of
    # the 175B-class shard (T=2048, h=12288, F=6144)
    # fc1: weight gradient 128x128, data gradient 128x192: 200 blocks against
    # 264 with both on 128x128 (the cost model ties them; fewer blocks win)
    assert L.tp_linear_bwd_plan(4096, 768, 1536) == (2, 1)
    # fc2: both on 256x192 with the weight gradient in 4 K slices, 224 blocks
    # (one round of the CUs) where 128x128 + 128x192 would need 328
    assert L.tp_linear_bwd_plan(4096, 1536, 768) == (3, 4)
    # the 175B-class shard: both products already fill the CUs for several
    # rounds each, so pairing saves no round and the paired kernel's slower
    # blocks lose (652 and 668 us against 572 and 613 us for the two calls)
    assert L.tp_linear_bwd_plan(2048, 12288, 6144) == (0, 1)
    assert L.tp_linear_bwd_plan(2048, 6144, 12288) == (0, 1)
    # the ~350M shard (T=6144, h=F=1024, QKV width 768): the data gradient's
    # own 128x256 tile has no paired kernel, and both on 128x128 in 2 slices
    # beats the two calls
    assert L.tp_gemm_plan(6144, 1024, 1024)[0] == 12
    assert L.tp_linear_bwd_plan(6144, 1024, 1024) == (1, 2)
    assert L.tp_linear_bwd_plan(6144, 1024, 768) == (1, 2)
    # no pipelined tile fits a ragged layer
    assert L.tp_linear_bwd_plan(300, 129, 200) == (0, 1)
    assert L.tp_linear_bwd_plan(4096, 768, 1000) == (0, 1)
    for T, k, n in [(4096, 768, 1536), (4096, 256, 256), (8192, 256, 256), (2048, 12288, 6144)]:
        pr, sk = L.tp_linear_bwd_plan(T, k, n)
        assert pr in (0, 1, 2, 3) and 1 <= sk <= 16
        if pr and sk > 1:   # split partials live in the workspace
            assert L.tp_linear_bwd_workspace_size(T, k, n, L.TP_BF16) >= sk * k * n * 4
    assert lib.tp_linear_bwd_plan(0, 8, 8, None, None) == -2
    assert lib.tp_linear_bwd_plan(8, 8, -1, None, None) == -2
    assert lib.tp_linear_bwd_plan(64, 128, 128, None, None) == 0


def test_linear_bwd_validation(lib):
    """tp_linear_bwd runs every check of both gradients before any launch."""
    f = lib.tp_linear_bwd
    # dOut W U act In dIn dW dbias T k n ld_dout ld_w ld_u ld_in ld_din ld_dw acc dt out_dt ws bytes s
    ok = [FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, 8, 4, 4, 4, 4, 4, 4, 4, 4, 0, 1, 1, None, 0,
          None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a4=None) == -1                   # In
    assert call(a6=None) == -1                   # dW
    assert call(a2=None) == -1                   # GeLU needs U
    assert call(a3=3) == -4
    assert call(a18=0, a19=1) == -3              # fp32 operands, bf16 dIn
    assert call(a18=7) == -3
    assert call(a13=3) == -2                     # ld_u < k
    assert call(a14=3) == -2                     # ld_in < k
    assert call(a16=3) == -2                     # ld_dw < n
    assert call(a8=0) == -2
    # a weight gradient that splits K needs the workspace
    big = dict(a8=4096, a9=256, a10=256, a11=256, a12=256, a13=256, a14=256, a15=256, a16=256)
    assert call(**big) == -5
    assert call(**big, a20=FAKE, a21=64) == -5
    # the workspace query covers both gradients' own needs
    for T, k, n in [(4096, 1536, 768), (4096, 768, 1536), (2048, 6144, 12288), (300, 129, 200)]:
        both = L.tp_linear_bwd_workspace_size(T, k, n, L.TP_BF16)
        assert both >= L.tp_linear_bwd_wgrad_workspace_size(T, k, n, L.TP_BF16)


def test_mlp_bwd_validation(lib):
    """tp_mlp_bwd checks both layers before any launch; its workspace covers
    each layer's own call."""
    f = lib.tp_mlp_bwd
    # dZ X A B U Y dU dB db dXp dA da T h F ld_dz ld_x ld_a ld_b ld_u ld_y ld_du ld_dxp ld_db ld_da
    # acc dt ws bytes stream
    ok = [FAKE] * 6 + [FAKE, FAKE, None, FAKE, FAKE, None, 8, 4, 8, 4, 4, 8, 4, 8, 8, 8, 4, 4, 8,
                       0, 1, None, 0, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a4=None) == -1   # U (GeLU)
    assert call(a5=None) == -1   # Y
    assert call(a10=None) == -1  # dA
    assert call(a26=5) == -3
    assert call(a17=4) == -2     # ld_a < F
    assert call(a24=4) == -2     # ld_da < F
    assert call(a12=0) == -2
    for T, h, F in [(4096, 768, 1536), (6144, 1024, 1024), (2048, 12288, 6144), (300, 129, 200)]:
        both = L.tp_mlp_bwd_workspace_size(T, h, F, L.TP_BF16)
        assert both >= L.tp_linear_bwd_workspace_size(T, F, h, L.TP_BF16)
        assert both >= L.tp_linear_bwd_workspace_size(T, h, F, L.TP_BF16)


def test_attention_validation(lib):
    """The attention entry point rejects bad arguments on the host, before any launch."""
    import ctypes
    buf = ctypes.create_string_buffer(4096 + 64)
    base = (ctypes.addressof(buf) + 63) // 64 * 64
    q = ctypes.c_void_p(base)
    args = dict(batch=1, seq=4, heads=1, hd=64, ld_qkv=192, ld_c=64, causal=1, dt=L.TP_BF16)

    def call(qkv=q, c=q, **kw):
        a = dict(args, **kw)
        return lib.tp_attention_fwd(qkv, c, None, a["batch"], a["seq"], a["heads"], a["hd"],
                                    a["ld_qkv"], a["ld_c"], a["causal"], a["dt"], None)
    assert call(qkv=None) == -1
    assert call(c=None) == -1
    assert call(dt=L.TP_F32) == -3
    assert call(hd=32) == -2
    assert call(seq=0) == -2
    assert call(ld_qkv=191) == -2          # shorter than the row
    assert call(ld_qkv=196) == -2          # not a multiple of 8
    assert call(qkv=ctypes.c_void_p(base + 8)) == -2   # not 16-byte aligned
    assert call(ld_c=66) == -2             # not a multiple of 4


def test_attention_bwd_validation(lib):
    """The attention backward rejects bad arguments on the host, before any launch."""
    import ctypes
    buf = ctypes.create_string_buffer(4096 + 64)
    base = (ctypes.addressof(buf) + 63) // 64 * 64
    q = ctypes.c_void_p(base)
    args = dict(batch=1, seq=4, heads=1, hd=64, ld_qkv=192, ld_c=64, ld_dc=64, ld_dqkv=192,
                causal=1, dt=L.TP_BF16)

    def call(qkv=q, c=q, dc=q, lse=q, delta=q, dqkv=q, **kw):
        a = dict(args, **kw)
        return lib.tp_attention_bwd(qkv, c, dc, lse, delta, dqkv, a["batch"], a["seq"], a["heads"],
                                    a["hd"], a["ld_qkv"], a["ld_c"], a["ld_dc"], a["ld_dqkv"],
                                    a["causal"], a["dt"], None)
    for name in ("qkv", "c", "dc", "lse", "delta", "dqkv"):
        assert call(**{name: None}) == -1, name
    assert call(dt=L.TP_F32) == -3
    assert call(hd=128) == -2
    assert call(heads=0) == -2
    assert call(ld_dqkv=191) == -2         # shorter than the row
    assert call(ld_dc=60) == -2            # shorter than the row
    assert call(ld_c=68) == -2             # not a multiple of 8
    assert call(dc=ctypes.c_void_p(base + 8)) == -2    # not 16-byte aligned
    assert call(dqkv=ctypes.c_void_p(base + 4)) == -2  # not 8-byte aligned
    assert call(delta=ctypes.c_void_p(base + 2)) == -2


def test_dgrad_recompute_validation(lib):
    """The recompute dgrad rejects bad arguments on the host, before any launch."""
    import ctypes
    buf = ctypes.create_string_buffer(4096 + 64)
    q = ctypes.c_void_p((ctypes.addressof(buf) + 63) // 64 * 64)
    args = dict(T=4, k=8, n=8, ld_dout=8, ld_w=8, ld_u=8, ld_din=8, ld_y=8, dt=L.TP_BF16,
                act=L.TP_ACT_GELU_TANH)

    def call(u=q, y=q, **kw):
        a = dict(args, **kw)
        return lib.tp_linear_bwd_dgrad_recompute(q, q, u, a["act"], q, y, a["T"], a["k"], a["n"],
                                                 a["ld_dout"], a["ld_w"], a["ld_u"], a["ld_din"],
                                                 a["ld_y"], a["dt"], None)
    assert call(u=None) == -1
    assert call(y=None) == -1
    assert call(act=L.TP_ACT_NONE) == -4
    assert call(dt=7) == -3
    assert call(ld_y=7) == -2
    assert call(ld_u=7) == -2
    assert call(k=0) == -2


def test_fp8_quantize_multi_validation(lib):
    """The multi-tensor quantiser checks n, its arrays, the workspace and every
    tensor on the host before any launch."""
    import ctypes
    buf = ctypes.create_string_buffer(2 * 4096 + 256)
    p = (ctypes.addressof(buf) + 255) // 256 * 256
    ws = ctypes.c_size_t(0)
    assert lib.tp_fp8_quantize_multi_workspace_size(3, ctypes.byref(ws)) == 0
    assert ws.value == 3 * 4096
    assert lib.tp_fp8_quantize_multi_workspace_size(0, ctypes.byref(ws)) == -2
    assert lib.tp_fp8_quantize_multi_workspace_size(7, ctypes.byref(ws)) == -2
    assert lib.tp_fp8_quantize_multi_workspace_size(2, None) == -1
    vp, i64, i32 = ctypes.c_void_p * 2, ctypes.c_int64 * 2, ctypes.c_int * 2

    def call(n=2, Xs=(p, p), ld_x=(8, 8), fmt=(0, 1), ld_qt=(4, 4), wsb=2 * 4096, rows=True):
        return lib.tp_fp8_quantize_both_multi(
            n, vp(*Xs), i64(4, 4) if rows else None, i64(8, 8), i64(*ld_x),
            i32(L.TP_BF16, L.TP_BF16), i32(*fmt), vp(p, p), i64(8, 8), vp(p, p), i64(*ld_qt),
            vp(p, p), ctypes.c_void_p(p), wsb, None)
    assert call(n=0) == -2 and call(n=7) == -2
    assert call(rows=False) == -1
    assert call(Xs=(p, None)) == -1            # the second tensor's input
    assert call(ld_x=(8, 7)) == -2
    assert call(ld_qt=(4, 3)) == -2            # X^T rows are 4 codes
    assert call(fmt=(0, 2)) == -3
    assert call(wsb=2 * 4096 - 4) == -5        # 4 KiB of maxima per tensor


def test_fp8_validation(lib):
    """The FP8 entry points reject bad arguments on the host, before any launch."""
    import ctypes
    buf = ctypes.create_string_buffer(8192 + 256)
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    q = ctypes.c_void_p(base)
    ws = ctypes.c_size_t(0)
    assert lib.tp_fp8_quantize_workspace_size(4, 4, ctypes.byref(ws)) == 0 and ws.value == 4096
    wsp = ctypes.c_void_p(base)

    def quant(x=q, Q=q, si=q, rows=4, cols=8, ld_x=8, dt=L.TP_BF16, fmt=0, tr=0, ld_q=8,
              wsb=4096):
        return lib.tp_fp8_quantize(x, rows, cols, ld_x, dt, fmt, tr, Q, ld_q, si, wsp, wsb, None)
    assert quant(x=None) == -1 and quant(Q=None) == -1 and quant(si=None) == -1
    assert quant(fmt=2) == -3 and quant(dt=5) == -3
    assert quant(ld_x=7) == -2 and quant(ld_q=7) == -2
    assert quant(tr=1, ld_q=3) == -2          # X^T rows are 4 codes
    assert quant(wsb=4092) == -5

    def col(M=256, N=256, K=256, lda=256, ldb=256, act=L.TP_ACT_GELU_TANH, U=q, bias=None):
        return lib.tp_fp8_column_linear_fwd(q, q, q, q, bias, q, U, M, K, N, lda, ldb, N, act, None)
    assert col(U=None) == -1
    assert col(act=L.TP_ACT_NONE, U=None, bias=q) == -4   # no bias without the activation
    assert col(K=200, lda=256, ldb=256) == -2             # K not a multiple of 128
    assert col(M=200) == -2                                # M not a multiple of 128
    assert col(lda=264) == -2                              # code stride not a multiple of 16

    def dgrad(fmt=1, act=L.TP_ACT_GELU_TANH, out_dt=L.TP_BF16, U=q):
        return lib.tp_fp8_linear_bwd_dgrad(q, q, q, q, fmt, U, act, q, 256, 256, 256, 256, 256,
                                           256, 256, out_dt, None)
    assert dgrad(fmt=3) == -3
    assert dgrad(out_dt=L.TP_F32) == -3                    # the GeLU' epilogue writes bf16
    assert dgrad(U=None) == -1

    def wgrad(T=256, dbias=None, dout=None, wsb=0):
        return lib.tp_fp8_linear_bwd_wgrad(q, q, q, q, 1, q, dout, dbias, T, 256, 256, T, T, 256,
                                           256, None, wsb, None)
    assert wgrad(dbias=q) == -1                            # bias gradient needs the bf16 dOut
    assert wgrad(T=64) == -2
    assert L.tp_fp8_linear_bwd_wgrad_workspace_size(4096, 256, 256) >= 0


def test_gemm_override(lib):
    """The tuning hook forces a tile where the shape allows it, splits only
    weight gradients, changes the workspace query with the plan and resets."""
    try:
        L.tp_set_gemm_override(14, 4)
        assert L.tp_gemm_plan(1024, 384, 4096) == (14, 1, 4096)
        assert L.tp_gemm_plan(1024, 384, 4096, allow_split=True) == (14, 4, 1024)
        assert L.tp_linear_bwd_wgrad_workspace_size(4096, 1024, 384, L.TP_BF16) >= 4 * 1024 * 384 * 4
        # N not a multiple of 192: the planner's own choice
        L.tp_set_gemm_override(0)
        own = L.tp_gemm_plan(1024, 512, 4096, allow_split=True)
        L.tp_set_gemm_override(14, 4)
        assert L.tp_gemm_plan(1024, 512, 4096, allow_split=True) == own
        # split that does not divide K into multiples of 64: one slice
        L.tp_set_gemm_override(10, 3)
        assert L.tp_gemm_plan(512, 512, 1024, allow_split=True) == (10, 1, 1024)
        assert lib.tp_set_gemm_override(7, 1) == -2
        assert lib.tp_set_gemm_override(10, 0) == -2
        assert lib.tp_set_gemm_override(10, 17) == -2
    finally:
        L.tp_set_gemm_override(0)
    assert L.tp_gemm_plan(1024, 512, 4096, allow_split=True) == own


def test_valid_call_without_a_device_reports_hip_error(lib):
    """With no GPU present, a call that passes validation reports TP_ERR_HIP
    (and the hipError_t) instead of crashing. Skipped wherever a device
    exists: the pointers here are host memory."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this case is for hosts without one")
    buf = ctypes.create_string_buffer(4096)
    x = ctypes.c_void_p(ctypes.addressof(buf))
    assert lib.tp_bias_act(x, None, x, 8, 8, 8, 8, 1, 1, 1, None) == -6
    assert L.tp_last_hip_error() != 0
    assert "TP_ERR_HIP" in L.tp_status_string(-6)


def test_gemm_override_is_per_thread(lib):
    """The tuning hook changes the plans of the thread that set it only."""
    import threading
    own = L.tp_gemm_plan(4096, 1536, 768)
    seen = {}
    try:
        L.tp_set_gemm_override(13, 1)
        assert L.tp_gemm_plan(4096, 1536, 768)[0] == 13
        t = threading.Thread(target=lambda: seen.update(plan=L.tp_gemm_plan(4096, 1536, 768)))
        t.start()
        t.join()
    finally:
        L.tp_set_gemm_override(0)
    assert seen["plan"] == own != (13, 1, 768)
    assert L.tp_gemm_plan(4096, 1536, 768) == own


def test_enum_typed_arguments_in_header():
    """dtype, activation and FP8 format arguments carry the header's enum types."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    assert not re.search(r"\bint (dt|out_dt|in_dt|act|fmt|dout_fmt)\b", src)
    assert "tp_dtype dt" in src and "tp_act act" in src and "tp_fp8_format fmt" in src


def test_binding_rejects_mismatched_operands():
    """The torch wrappers check every operand's shape, dtype, layout and device
    before calling the library (which cannot see buffer sizes); nothing is
    launched. CPU tensors of the right shape fail the device check last."""
    import torch
    bf, f32, u8 = torch.bfloat16, torch.float32, torch.uint8
    T, h, F = 64, 32, 48

    def z(*shape, dtype=bf):
        return torch.zeros(*shape, dtype=dtype)

    X, A, a, Y, U = z(T, h), z(h, F), z(F), z(T, F), z(T, F)
    with pytest.raises(ValueError, match="GPU tensor"):
        L.tp_column_linear_fwd(X, A, a, Y, U)
    with pytest.raises(ValueError, match="A_i has shape"):
        L.tp_column_linear_fwd(X, z(F, h), a, Y, U)          # transposed weight
    with pytest.raises(ValueError, match="bias_i has shape"):
        L.tp_column_linear_fwd(X, A, z(h), Y, U)
    with pytest.raises(TypeError, match="Y_i has dtype"):
        L.tp_column_linear_fwd(X, A, a, z(T, F, dtype=f32), U)
    with pytest.raises(ValueError, match="U_i is required"):
        L.tp_column_linear_fwd(X, A, a, Y, None, act="gelu")
    with pytest.raises(ValueError, match="unit stride"):
        L.tp_column_linear_fwd(X, A, a, z(F, T).t(), U)      # column-major view
    B, Zp = z(F, h), z(T, h, dtype=f32)
    with pytest.raises(TypeError, match="Zp_i has dtype"):
        L.tp_row_linear_fwd_partial(Y, B, z(T, h))           # bf16 partial
    with pytest.raises(ValueError, match="B_i has shape"):
        L.tp_row_linear_fwd_partial(Y, z(h, F), Zp)
    with pytest.raises(ValueError, match="dIn has shape"):
        L.tp_linear_bwd_dgrad(z(T, h), B, U, z(T, h), act="gelu")
    with pytest.raises(ValueError, match="dW has shape"):
        L.tp_linear_bwd_wgrad(Y, z(T, h), z(h, F, dtype=f32))
    with pytest.raises(TypeError, match="dW has dtype"):
        L.tp_linear_bwd(z(T, h), B, U, Y, U, z(F, h), act="gelu")
    with pytest.raises(ValueError, match="dXp_i has shape"):
        L.tp_mlp_bwd(z(T, h), X, A, B, U, Y, z(T, F), z(F, h, dtype=f32), None,
                     z(T, F, dtype=f32), z(h, F, dtype=f32), None)
    with pytest.raises(ValueError, match="partials\\[1\\] has shape"):
        L.tp_reduce_partials([Zp, z(T, h + 1, dtype=f32)], None, z(T, h))
    with pytest.raises(TypeError, match="bias has dtype"):
        L.tp_reduce_partials([Zp, Zp], z(h, dtype=f32), z(T, h))
    with pytest.raises(ValueError, match="C has shape"):
        L.tp_attention_fwd(z(128, 3 * 128), z(128, 64), None, 2, 64, 2)
    with pytest.raises(ValueError, match="delta has shape"):
        L.tp_attention_bwd(z(128, 384), z(128, 128), z(128, 128), z(256, dtype=f32),
                           z(255, dtype=f32), z(128, 384), 2, 64, 2)
    with pytest.raises(ValueError, match="Qt has shape"):
        L.tp_fp8_quantize_both(X, z(T, h, dtype=u8), z(T, h, dtype=u8), z(1, dtype=f32),
                               z(4096, dtype=u8))
    with pytest.raises(ValueError, match="Atq has shape"):
        L.tp_fp8_column_linear_fwd(z(T, h, dtype=u8), z(h, F, dtype=u8), z(1, dtype=f32),
                                   z(1, dtype=f32), None, Y, U)
    with pytest.raises(ValueError, match="dOut is required"):
        L.tp_fp8_linear_bwd_wgrad(z(F, T, dtype=u8), z(h, T, dtype=u8), z(1, dtype=f32),
                                  z(1, dtype=f32), z(F, h, dtype=f32), dbias=z(h, dtype=f32))


def test_mlp_step_queries(lib):
    """tp_mlp_step's fused-path and workspace queries (shape-only, host)."""
    bf = L.TP_BF16
    assert L.tp_mlp_step_plan(4096, 768, 1536, 2, bf)           # GPT-2-small, p = 2
    assert L.tp_mlp_step_plan(6144, 1024, 1024, 4, bf)          # the ~350M layer's MLP
    assert not L.tp_mlp_step_plan(680, 768, 1536, 2, bf)        # T not a multiple of 1024
    assert not L.tp_mlp_step_plan(2048, 12288, 6144, 1, bf)     # 175B-class: products too big
    assert not L.tp_mlp_step_plan(4096, 768, 1536, 2, L.TP_F32)
    fused = L.tp_mlp_step_workspace_size(4096, 768, 1536, 2, bf)
    per_product = L.tp_mlp_bwd_workspace_size(4096, 768, 1536, bf)
    assert fused >= per_product and fused % 256 == 0
    # the queue's counters come ahead of the stacked weight gradients' scratch
    for k, n in ((2 * 1536, 768), (768, 2 * 1536)):
        assert fused > L.tp_linear_bwd_wgrad_workspace_size(4096, k, n, bf)
    assert L.tp_mlp_step_workspace_size(680, 768, 1536, 2, bf) >= \
        L.tp_mlp_bwd_workspace_size(680, 768, 1536, bf)
    out = ctypes.c_size_t(0)
    assert lib.tp_mlp_step_workspace_size(4096, 768, 1536, 0, bf, ctypes.byref(out)) == -2
    assert lib.tp_mlp_step_workspace_size(4096, 768, 1536, 17, bf, ctypes.byref(out)) == -2
    assert lib.tp_mlp_step_workspace_size(4096, 768, 1536, 2, 5, ctypes.byref(out)) == -3
    assert lib.tp_mlp_step_workspace_size(4096, 768, 1536, 2, bf, None) == -1
    assert lib.tp_set_wait_limit(0) == 0


def test_mlp_step_validation(lib):
    """tp_mlp_step, its halves and its forward / backward calls reject bad
    arguments before any launch."""
    F_ = FAKE
    for fn, extra in ((lib.tp_mlp_step, ()), (lib.tp_mlp_step_rows, ()),
                      (lib.tp_mlp_step_wgrad, ()), (lib.tp_mlp_step_fwd, ()),
                      (lib.tp_mlp_step_bwd, (0,)), (lib.tp_mlp_step_bwd, (1,))):
        def call(*, X=F_, dX=F_, T=4096, h=768, F=1536, p=2, ld_a=3072, ld_u=3072, dt=1,
                 ws=F_, wsb=1 << 30):
            return fn(X, F_, None, F_, None, F_, F_, F_, F_, F_, F_, F_, None, F_, None, F_, dX,
                      T, h, F, p, 768, ld_a, 768, 768, ld_u, 768, 768, 768, 3072, *extra, dt, ws,
                      wsb, None)
        assert call(X=None) == -1
        assert call(dX=None) == -1
        assert call(T=0) == -2
        assert call(p=0) == -2
        assert call(p=17) == -2
        assert call(ld_a=3071) == -2      # below p * F
        assert call(ld_u=1536) == -2
        assert call(dt=4) == -3
        assert call(ws=None, wsb=0) == -5
        assert call(wsb=1024) == -5


def test_attn_proj_step_queries_and_validation(lib):
    """tp_attn_proj_step's queries and its argument checks, before any launch."""
    bf = L.TP_BF16
    assert L.tp_attn_proj_step_plan(4096, 1024, 1536, 512, 2, bf)    # attention projections
    assert L.tp_attn_proj_step_plan(6144, 1024, 768, 256, 4, bf)     # the ~350M layer's
    assert not L.tp_attn_proj_step_plan(680, 1024, 1536, 512, 2, bf)  # T not a multiple of 1024
    assert not L.tp_attn_proj_step_plan(4096, 1024, 1536, 500, 2, bf)
    assert not L.tp_attn_proj_step_plan(4096, 1024, 1536, 512, 2, L.TP_F32)
    ws = L.tp_attn_proj_step_workspace_size(4096, 1024, 1536, 512, 2, bf)
    assert ws % 256 == 0 and ws >= L.tp_linear_bwd_wgrad_workspace_size(4096, 1024, 3072, bf)
    out = ctypes.c_size_t(0)
    assert lib.tp_attn_proj_step_workspace_size(4096, 1024, 1536, 512, 0, bf,
                                                ctypes.byref(out)) == -2
    assert lib.tp_attn_proj_step_workspace_size(4096, 1024, 1536, 512, 2, 9,
                                                ctypes.byref(out)) == -3
    assert lib.tp_attn_proj_step_workspace_size(4096, 1024, 1536, 512, 2, bf, None) == -1
    F_ = FAKE

    def call(*, stages=31, X=F_, C=F_, dQKV=F_, T=4096, p=2, ld_w=3072, dt=1, ws=F_,
             wsb=1 << 30):
        return lib.tp_attn_proj_step(X, F_, F_, C, F_, dQKV, F_, F_, F_, F_, F_, F_, F_, F_, T,
                                     1024, 1536, 512, p, 1024, ld_w, 1024, 1024, 1024, 3072, 3072,
                                     1024, 1024, 1024, 1024, 3072, stages, dt, ws, wsb, None)
    assert call(stages=0) == -2
    assert call(stages=32) == -2
    assert call(X=None) == -1                 # stage 1 reads X
    # dC alone does not read X: that call passes the pointer checks and stops
    # at the (too small) workspace, so nothing is launched
    assert call(stages=4, X=None, wsb=1024) == -5
    assert call(stages=2, C=None) == -1
    assert call(stages=8, dQKV=None) == -1
    assert call(T=0) == -2
    assert call(p=17) == -2
    assert call(ld_w=3071) == -2
    assert call(dt=4) == -3
    assert call(ws=None, wsb=0) == -5
    assert call(wsb=1024) == -5


def test_noalloc_wgrad_rejects_shape_beyond_scratch(lib):
    # the size check runs before any HIP call, so this needs no GPU; the
    # pointers are never dereferenced
    T, k, n = 1 << 20, 256, 1024
    assert L.tp_linear_bwd_wgrad_workspace_size(T, k, n, L.TP_BF16) > L.TP_NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    st = lib.tp_linear_bwd_wgrad_noalloc(fake, fake, fake, None, T, k, n, k, n, n, 0,
                                         L.TP_BF16, None)
    assert L.STATUS[st] == "TP_ERR_SCRATCH"
    assert L.tp_status_string(st).startswith("TP_ERR_SCRATCH")
    assert lib.tp_linear_bwd_wgrad_noalloc(None, fake, fake, None, 5, 5, 5, 5, 5, 5, 0,
                                           L.TP_BF16, None) == -1
    assert lib.tp_linear_bwd_wgrad_noalloc(fake, fake, fake, None, 5, 5, 5, 4, 5, 5, 0,
                                           L.TP_BF16, None) == -2
    assert lib.tp_linear_bwd_wgrad_noalloc(fake, fake, fake, None, 5, 5, 5, 5, 5, 5, 0,
                                           9, None) == -3
    with open(HEADER) as f:
        assert "#define TP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in f.read()
    assert L.TP_NOALLOC_SCRATCH_BYTES == 32 << 20


def test_fp8_amax_entry_points_reject_bad_arguments(lib):
    fake = 1 << 20
    out = ctypes.c_int64(0)
    assert lib.tp_fp8_amax_slots(4096, 1536, 768, ctypes.byref(out)) == 0 and out.value > 0
    assert out.value % 4 == 0
    assert lib.tp_fp8_amax_slots(100, 1536, 768, ctypes.byref(out)) == -2   # no FP8 tile fits
    assert lib.tp_fp8_amax_slots(4096, 1536, 768, None) == -1
    args = (fake, fake, fake, fake, None, fake, fake, 4096, 768, 1536, 768, 768, 1536)
    assert lib.tp_fp8_column_linear_fwd_amax(*args, None, None) == -1
    assert lib.tp_fp8_column_linear_fwd_amax(fake, fake, fake, fake, None, fake, fake, 100, 768,
                                             1536, 768, 768, 1536, fake, None) == -2
    assert lib.tp_fp8_linear_bwd_dgrad_amax(fake, fake, fake, fake, 1, fake, fake, 4096, 1536,
                                            768, 768, 768, 1536, 1536, None, None) == -1
    assert lib.tp_fp8_quantize_both_from_amax(fake, 64, 64, 64, L.TP_BF16, 0, fake, 64, fake, 64,
                                              fake, None, 16, None) == -1
    assert lib.tp_fp8_quantize_both_from_amax(fake, 64, 64, 64, L.TP_BF16, 0, fake, 64, fake, 64,
                                              fake, fake, 0, None) == -2
