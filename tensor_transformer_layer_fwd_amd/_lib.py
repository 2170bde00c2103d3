"""ctypes binding of libtpmlp.so (include/tp_mlp.h). Argument marshalling only:
every step of the shard runs in the library's HIP kernels.

Two layers:
  - ``lib()`` returns the loaded ``ctypes.CDLL`` with typed signatures;
  - the ``tp_*`` functions below take torch tensors that already live on the
    GPU, derive sizes and row strides from them, call the entry point of the
    same name on the current torch stream and raise ``TPError`` on a non-zero
    status.
There is no fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpmlp.so")

TP_OK = 0
TP_F32, TP_BF16 = 0, 1
TP_ACT_NONE, TP_ACT_GELU_TANH = 0, 1
STATUS = {0: "TP_OK", -1: "TP_ERR_NULL", -2: "TP_ERR_SHAPE", -3: "TP_ERR_DTYPE",
          -4: "TP_ERR_ACT", -5: "TP_ERR_WORKSPACE", -6: "TP_ERR_HIP",
          -7: "TP_ERR_SCRATCH"}
TP_NOALLOC_SCRATCH_BYTES = 32 << 20

# Every function declared in include/tp_mlp.h, with its ctypes signature.
_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "tp_column_linear_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                    _int, _int, _vp]),
    "tp_row_linear_fwd_partial": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _int,
                                         _vp]),
    "tp_linear_bwd_dgrad": (_int, [_vp, _vp, _vp, _int, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                   _i64, _int, _int, _vp]),
    "tp_linear_bwd_wgrad": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _int,
                                   _int, _vp, _sz, _vp]),
    "tp_linear_bwd_wgrad_noalloc": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                           _i64, _int, _int, _vp]),
    "tp_linear_bwd_wgrad_workspace_size": (_int, [_i64, _i64, _i64, _int,
                                                  ctypes.POINTER(ctypes.c_size_t)]),
    "tp_linear_bwd": (_int, [_vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                             _i64, _i64, _i64, _i64, _i64, _int, _int, _int, _vp, _sz, _vp]),
    "tp_linear_bwd_workspace_size": (_int, [_i64, _i64, _i64, _int,
                                            ctypes.POINTER(ctypes.c_size_t)]),
    "tp_linear_bwd_plan": (_int, [_i64, _i64, _i64, ctypes.POINTER(ctypes.c_int),
                                  ctypes.POINTER(ctypes.c_int)]),
    "tp_mlp_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                          _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _int,
                          _int, _vp, _sz, _vp]),
    "tp_mlp_bwd_workspace_size": (_int, [_i64, _i64, _i64, _int,
                                         ctypes.POINTER(ctypes.c_size_t)]),
    "tp_mlp_step": (_int, [_vp] * 17 + [_i64, _i64, _i64, _int] + [_i64] * 9 +
                    [_int, _vp, _sz, _vp]),
    "tp_mlp_step_rows": (_int, [_vp] * 17 + [_i64, _i64, _i64, _int] + [_i64] * 9 +
                         [_int, _vp, _sz, _vp]),
    "tp_mlp_step_wgrad": (_int, [_vp] * 17 + [_i64, _i64, _i64, _int] + [_i64] * 9 +
                          [_int, _vp, _sz, _vp]),
    "tp_mlp_step_fwd": (_int, [_vp] * 17 + [_i64, _i64, _i64, _int] + [_i64] * 9 +
                        [_int, _vp, _sz, _vp]),
    "tp_mlp_step_bwd": (_int, [_vp] * 17 + [_i64, _i64, _i64, _int] + [_i64] * 9 +
                        [_int, _int, _vp, _sz, _vp]),
    "tp_mlp_step_workspace_size": (_int, [_i64, _i64, _i64, _int, _int,
                                          ctypes.POINTER(ctypes.c_size_t)]),
    "tp_mlp_step_plan": (_int, [_i64, _i64, _i64, _int, _int, ctypes.POINTER(ctypes.c_int)]),
    "tp_attn_proj_step": (_int, [_vp] * 14 + [_i64, _i64, _i64, _i64, _int] + [_i64] * 12 +
                          [_int, _int, _vp, _sz, _vp]),
    "tp_attn_proj_step_workspace_size": (_int, [_i64, _i64, _i64, _i64, _int, _int,
                                                ctypes.POINTER(ctypes.c_size_t)]),
    "tp_attn_proj_step_plan": (_int, [_i64, _i64, _i64, _i64, _int, _int,
                                      ctypes.POINTER(ctypes.c_int)]),
    "tp_set_wait_limit": (_int, [_i64]),
    "tp_reduce_partials": (_int, [ctypes.POINTER(ctypes.c_void_p), _int, _vp, _vp, _i64, _i64, _i64,
                                  _i64, _int, _vp]),
    "tp_bias_act": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _int, _int, _vp]),
    "tp_gemm_plan": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(ctypes.c_int),
                            ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int64)]),
    "tp_attention_fwd": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _int, _int,
                                _vp]),
    "tp_linear_bwd_dgrad_recompute": (_int, [_vp, _vp, _vp, _int, _vp, _vp, _i64, _i64, _i64,
                                             _i64, _i64, _i64, _i64, _i64, _int, _vp]),
    "tp_fp8_quantize_workspace_size": (_int, [_i64, _i64, ctypes.POINTER(ctypes.c_size_t)]),
    "tp_fp8_quantize": (_int, [_vp, _i64, _i64, _i64, _int, _int, _int, _vp, _i64, _vp, _vp,
                               ctypes.c_size_t, _vp]),
    "tp_fp8_quantize_both": (_int, [_vp, _i64, _i64, _i64, _int, _int, _vp, _i64, _vp, _i64,
                                    _vp, _vp, ctypes.c_size_t, _vp]),
    "tp_fp8_quantize_both_multi": (_int, [_int, ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                          ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_void_p), _vp, _sz, _vp]),
    "tp_fp8_quantize_multi_workspace_size": (_int, [_int, ctypes.POINTER(ctypes.c_size_t)]),
    "tp_fp8_column_linear_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                        _i64, _i64, _i64, _int, _vp]),
    "tp_fp8_column_linear_fwd_amax": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                             _i64, _i64, _i64, _i64, _vp, _vp]),
    "tp_fp8_amax_slots": (_int, [_i64, _i64, _i64, ctypes.POINTER(ctypes.c_int64)]),
    "tp_fp8_quantize_both_from_amax": (_int, [_vp, _i64, _i64, _i64, _int, _int, _vp, _i64, _vp,
                                              _i64, _vp, _vp, _i64, _vp]),
    "tp_fp8_linear_bwd_dgrad_amax": (_int, [_vp, _vp, _vp, _vp, _int, _vp, _vp, _i64, _i64, _i64,
                                            _i64, _i64, _i64, _i64, _vp, _vp]),
    "tp_fp8_row_linear_fwd_partial": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                             _i64, _i64, _vp]),
    "tp_fp8_linear_bwd_dgrad": (_int, [_vp, _vp, _vp, _vp, _int, _vp, _int, _vp, _i64, _i64,
                                       _i64, _i64, _i64, _i64, _i64, _int, _vp]),
    "tp_fp8_linear_bwd_wgrad_workspace_size": (_int, [_i64, _i64, _i64,
                                                      ctypes.POINTER(ctypes.c_size_t)]),
    "tp_fp8_linear_bwd_wgrad": (_int, [_vp, _vp, _vp, _vp, _int, _vp, _vp, _vp, _i64, _i64,
                                       _i64, _i64, _i64, _i64, _i64, _vp, ctypes.c_size_t, _vp]),
    "tp_attention_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                _i64, _i64, _int, _int, _vp]),
    "tp_attention_fwd_shards": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                       _int, _int, _vp]),
    "tp_attention_bwd_shards": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                       _i64, _i64, _i64, _i64, _int, _int, _vp]),
    "tp_set_gemm_override": (_int, [_int, _int]),
    "tp_status_string": (ctypes.c_char_p, [_int]),
    "tp_last_hip_error": (_int, []),
}

_LIB = None


class TPError(RuntimeError):
    def __init__(self, fn: str, status: int):
        detail = ""
        if status == -6:
            detail = f" (hipError_t {lib().tp_last_hip_error()})"
        super().__init__(f"{fn} returned {status} {STATUS.get(status, '?')}{detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libtpmlp.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        # torch ships its own HIP runtime (same SONAME as the system one); load
        # it first so that this library binds to it and shares torch's streams
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m tensor_transformer_layer_fwd_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(fn: str, status: int) -> None:
    if status != TP_OK:
        raise TPError(fn, status)


# --------------------------------------------------------------------------- #
# torch-tensor conveniences (device memory and streams come from torch)       #
# --------------------------------------------------------------------------- #
def _dt(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ld(t) -> int:
    """Row stride of a 2-D row-major view (unit stride along columns)."""
    if t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1):
        raise ValueError("expected a 2-D tensor with unit column stride")
    return int(t.stride(0)) if t.shape[0] > 1 else int(max(t.stride(0), t.shape[1]))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _act(act) -> int:
    if act in (None, "none", TP_ACT_NONE):
        return TP_ACT_NONE
    if act in ("gelu", "gelu_tanh", TP_ACT_GELU_TANH):
        return TP_ACT_GELU_TANH
    raise ValueError(f"unknown activation {act!r}")


def _torch_dtypes(*names):
    import torch
    m = {"bf16": torch.bfloat16, "f32": torch.float32, "u8": torch.uint8}
    return tuple(m[n] for n in names)


class _Operands:
    """The checks every wrapper runs on its operands before the library sees a
    pointer: the C interface cannot see buffer sizes, so a tensor of the wrong
    shape, dtype or layout would make the kernels read or write out of bounds.
    Shapes and dtypes are checked first (ValueError / TypeError), then that
    every operand is a GPU tensor on one device, the device of the stream."""

    def __init__(self, fn: str):
        self.fn = fn
        self.seen = []

    def __call__(self, name, t, shape, dtypes, optional=False):
        import torch
        if t is None:
            if optional:
                return self
            raise ValueError(f"{self.fn}: {name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.fn}: {name} must be a torch.Tensor, not {type(t).__name__}")
        if tuple(t.shape) != tuple(int(d) for d in shape):
            raise ValueError(f"{self.fn}: {name} has shape {tuple(t.shape)}, "
                             f"expected {tuple(int(d) for d in shape)}")
        if dtypes is not None and t.dtype not in dtypes:
            raise TypeError(f"{self.fn}: {name} has dtype {t.dtype}, expected one of "
                            f"{[str(d) for d in dtypes]}")
        if t.dim() == 2:
            if t.stride(1) != 1 and t.shape[1] > 1:
                raise ValueError(f"{self.fn}: {name} needs unit stride along its rows")
        elif t.dim() == 1:
            if t.stride(0) != 1 and t.shape[0] > 1:
                raise ValueError(f"{self.fn}: {name} must be contiguous")
        self.seen.append((name, t))
        return self

    def done(self, stream=None):
        import torch
        devs = set()
        for name, t in self.seen:
            if not t.is_cuda:
                raise ValueError(f"{self.fn}: {name} is on {t.device}; every operand must be a "
                                 "GPU tensor")
            devs.add(t.device)
        if len(devs) > 1:
            raise ValueError(f"{self.fn}: operands on more than one device: {sorted(map(str, devs))}")
        if devs:
            (dev,) = devs
            sdev = (torch.cuda.current_stream() if stream is None else stream).device
            if sdev != dev:
                raise ValueError(f"{self.fn}: operands on {dev}, stream on {sdev}")


def _ws_bytes(workspace) -> int:
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def _check_ws(chk, workspace):
    """A workspace is any contiguous GPU tensor; the library checks its size."""
    if workspace is not None:
        chk("workspace", workspace, (workspace.numel(),) if workspace.dim() == 1 else workspace.shape,
            None)
        if not workspace.is_contiguous():
            raise ValueError(f"{chk.fn}: workspace must be contiguous")


def tp_column_linear_fwd(X, A_i, bias_i, Y_i, U_i=None, act="gelu", stream=None):
    chk = _Operands("tp_column_linear_fwd")
    chk("X", X, _shape2(X), _torch_dtypes("bf16", "f32"))
    T, h = X.shape
    dts = (X.dtype,)
    chk("A_i", A_i, (h, _shape2(A_i)[1]), dts)
    n = A_i.shape[1]
    chk("bias_i", bias_i, (n,), dts, optional=True)
    chk("Y_i", Y_i, (T, n), dts)
    chk("U_i", U_i, (T, n), dts, optional=_act(act) == TP_ACT_NONE)
    chk.done(stream)
    if U_i is not None and _ld(U_i) != _ld(Y_i):
        raise ValueError("U_i and Y_i must share a row stride")
    _check("tp_column_linear_fwd", lib().tp_column_linear_fwd(
        _ptr(X), _ptr(A_i), _ptr(bias_i), _ptr(Y_i), _ptr(U_i), T, h, n, _ld(X), _ld(A_i),
        _ld(Y_i), _dt(X), _act(act), _stream(stream)))


def _shape2(t):
    """(rows, cols) of a 2-D tensor, or (-1, -1) so that the shape check fails."""
    return tuple(t.shape) if t is not None and hasattr(t, "dim") and t.dim() == 2 else (-1, -1)


def tp_row_linear_fwd_partial(Y_i, B_i, Zp_i, stream=None):
    chk = _Operands("tp_row_linear_fwd_partial")
    chk("Y_i", Y_i, _shape2(Y_i), _torch_dtypes("bf16", "f32"))
    T, k = Y_i.shape
    chk("B_i", B_i, (k, _shape2(B_i)[1]), (Y_i.dtype,))
    h = B_i.shape[1]
    chk("Zp_i", Zp_i, (T, h), _torch_dtypes("f32")).done(stream)
    _check("tp_row_linear_fwd_partial", lib().tp_row_linear_fwd_partial(
        _ptr(Y_i), _ptr(B_i), _ptr(Zp_i), T, k, h, _ld(Y_i), _ld(B_i), _ld(Zp_i), _dt(Y_i),
        _stream(stream)))


def _out_dtypes(dt):
    """Output dtypes a product of operand dtype dt may write: its own, or fp32."""
    import torch
    return (dt, torch.float32)


def tp_linear_bwd_dgrad(dOut, W, U, dIn, act="none", stream=None):
    chk = _Operands("tp_linear_bwd_dgrad")
    chk("dOut", dOut, _shape2(dOut), _torch_dtypes("bf16", "f32"))
    T, n = dOut.shape
    chk("W", W, (_shape2(W)[0], n), (dOut.dtype,))
    k = W.shape[0]
    chk("U", U, (T, k), (dOut.dtype,), optional=_act(act) == TP_ACT_NONE)
    chk("dIn", dIn, (T, k), _out_dtypes(dOut.dtype)).done(stream)
    ld_u = _ld(U) if U is not None else k
    _check("tp_linear_bwd_dgrad", lib().tp_linear_bwd_dgrad(
        _ptr(dOut), _ptr(W), _ptr(U), _act(act), _ptr(dIn), T, k, n, _ld(dOut), _ld(W), ld_u,
        _ld(dIn), _dt(dOut), _dt(dIn), _stream(stream)))


def tp_linear_bwd_dgrad_recompute(dOut, W, U, dIn, Y, act="gelu", stream=None):
    """dIn = (dOut W^T) * act'(U) and Y = act(U) recomputed from the saved U."""
    chk = _Operands("tp_linear_bwd_dgrad_recompute")
    chk("dOut", dOut, _shape2(dOut), _torch_dtypes("bf16", "f32"))
    T, n = dOut.shape
    dts = (dOut.dtype,)
    chk("W", W, (_shape2(W)[0], n), dts)
    k = W.shape[0]
    chk("U", U, (T, k), dts)("dIn", dIn, (T, k), dts)("Y", Y, (T, k), dts).done(stream)
    _check("tp_linear_bwd_dgrad_recompute", lib().tp_linear_bwd_dgrad_recompute(
        _ptr(dOut), _ptr(W), _ptr(U), _act(act), _ptr(dIn), _ptr(Y), T, k, n, _ld(dOut), _ld(W),
        _ld(U), _ld(dIn), _ld(Y), _dt(dOut), _stream(stream)))


def tp_linear_bwd_wgrad_workspace_size(T: int, k: int, n: int, dt: int) -> int:
    out = ctypes.c_size_t(0)
    _check("tp_linear_bwd_wgrad_workspace_size",
           lib().tp_linear_bwd_wgrad_workspace_size(T, k, n, dt, ctypes.byref(out)))
    return int(out.value)


def tp_linear_bwd_wgrad(In, dOut, dW, dbias=None, accumulate=False, workspace=None,
                        stream=None):
    chk = _Operands("tp_linear_bwd_wgrad")
    chk("In", In, _shape2(In), _torch_dtypes("bf16", "f32"))
    T, k = In.shape
    chk("dOut", dOut, (T, _shape2(dOut)[1]), (In.dtype,))
    n = dOut.shape[1]
    f32 = _torch_dtypes("f32")
    chk("dW", dW, (k, n), f32)("dbias", dbias, (n,), f32, optional=True)
    _check_ws(chk, workspace)
    chk.done(stream)
    _check("tp_linear_bwd_wgrad", lib().tp_linear_bwd_wgrad(
        _ptr(In), _ptr(dOut), _ptr(dW), _ptr(dbias), T, k, n, _ld(In), _ld(dOut), _ld(dW),
        int(bool(accumulate)), _dt(In), _ptr(workspace), _ws_bytes(workspace), _stream(stream)))


def tp_linear_bwd_wgrad_noalloc(In, dOut, dW, dbias=None, accumulate=False, stream=None):
    """tp_linear_bwd_wgrad on the library's static per-GPU scratch array: no
    workspace argument, nothing allocated. Calls that may overlap on one GPU
    race on that array."""
    chk = _Operands("tp_linear_bwd_wgrad_noalloc")
    chk("In", In, _shape2(In), _torch_dtypes("bf16", "f32"))
    T, k = In.shape
    chk("dOut", dOut, (T, _shape2(dOut)[1]), (In.dtype,))
    n = dOut.shape[1]
    f32 = _torch_dtypes("f32")
    chk("dW", dW, (k, n), f32)("dbias", dbias, (n,), f32, optional=True)
    chk.done(stream)
    _check("tp_linear_bwd_wgrad_noalloc", lib().tp_linear_bwd_wgrad_noalloc(
        _ptr(In), _ptr(dOut), _ptr(dW), _ptr(dbias), T, k, n, _ld(In), _ld(dOut), _ld(dW),
        int(bool(accumulate)), _dt(In), _stream(stream)))


def tp_linear_bwd_workspace_size(T: int, k: int, n: int, dt: int) -> int:
    out = ctypes.c_size_t(0)
    _check("tp_linear_bwd_workspace_size",
           lib().tp_linear_bwd_workspace_size(T, k, n, dt, ctypes.byref(out)))
    return int(out.value)


def tp_linear_bwd_plan(T: int, k: int, n: int):
    """(pairing, K slices) of tp_linear_bwd for a bf16 layer: pairing 0 runs
    the two products as separate calls, 1..3 in one paired launch."""
    pr, sk = ctypes.c_int(0), ctypes.c_int(0)
    _check("tp_linear_bwd_plan", lib().tp_linear_bwd_plan(T, k, n, ctypes.byref(pr),
                                                           ctypes.byref(sk)))
    return int(pr.value), int(sk.value)


def tp_linear_bwd(dOut, W, U, In, dIn, dW, dbias=None, act="none", accumulate=False,
                  workspace=None, stream=None):
    """Both gradients of one linear layer: dIn = (dOut W^T) [* act'(U)] and
    dW (+)= In^T dOut, dbias (+)= column sums of dOut."""
    chk = _Operands("tp_linear_bwd")
    chk("dOut", dOut, _shape2(dOut), _torch_dtypes("bf16", "f32"))
    T, n = dOut.shape
    dts = (dOut.dtype,)
    chk("W", W, (_shape2(W)[0], n), dts)
    k = W.shape[0]
    f32 = _torch_dtypes("f32")
    chk("U", U, (T, k), dts, optional=_act(act) == TP_ACT_NONE)
    chk("In", In, (T, k), dts)("dIn", dIn, (T, k), _out_dtypes(dOut.dtype))
    chk("dW", dW, (k, n), f32)("dbias", dbias, (n,), f32, optional=True)
    _check_ws(chk, workspace)
    chk.done(stream)
    ld_u = _ld(U) if U is not None else k
    _check("tp_linear_bwd", lib().tp_linear_bwd(
        _ptr(dOut), _ptr(W), _ptr(U), _act(act), _ptr(In), _ptr(dIn), _ptr(dW), _ptr(dbias),
        T, k, n, _ld(dOut), _ld(W), ld_u, _ld(In), _ld(dIn), _ld(dW), int(bool(accumulate)),
        _dt(dOut), _dt(dIn), _ptr(workspace), _ws_bytes(workspace), _stream(stream)))


def tp_mlp_bwd_workspace_size(T: int, h: int, F: int, dt: int) -> int:
    out = ctypes.c_size_t(0)
    _check("tp_mlp_bwd_workspace_size",
           lib().tp_mlp_bwd_workspace_size(T, h, F, dt, ctypes.byref(out)))
    return int(out.value)


def tp_mlp_bwd(dZ, X, A_i, B_i, U_i, Y_i, dU_i, dB_i, db, dXp_i, dA_i, da_i, accumulate=False,
               workspace=None, stream=None):
    """The backward of one shard's MLP block: fc2's gradients with the GeLU
    derivative, then fc1's, dXp_i the shard's fp32 dX partial."""
    chk = _Operands("tp_mlp_bwd")
    chk("dZ", dZ, _shape2(dZ), _torch_dtypes("bf16", "f32"))
    T, h = dZ.shape
    dts, f32 = (dZ.dtype,), _torch_dtypes("f32")
    chk("B_i", B_i, (_shape2(B_i)[0], h), dts)
    F = B_i.shape[0]
    chk("X", X, (T, h), dts)("A_i", A_i, (h, F), dts)("U_i", U_i, (T, F), dts)
    chk("Y_i", Y_i, (T, F), dts)("dU_i", dU_i, (T, F), dts)("dB_i", dB_i, (F, h), f32)
    chk("db", db, (h,), f32, optional=True)("dXp_i", dXp_i, (T, h), f32)
    chk("dA_i", dA_i, (h, F), f32)("da_i", da_i, (F,), f32, optional=True)
    _check_ws(chk, workspace)
    chk.done(stream)
    _check("tp_mlp_bwd", lib().tp_mlp_bwd(
        _ptr(dZ), _ptr(X), _ptr(A_i), _ptr(B_i), _ptr(U_i), _ptr(Y_i), _ptr(dU_i), _ptr(dB_i),
        _ptr(db), _ptr(dXp_i), _ptr(dA_i), _ptr(da_i), T, h, F, _ld(dZ), _ld(X), _ld(A_i),
        _ld(B_i), _ld(U_i), _ld(Y_i), _ld(dU_i), _ld(dXp_i), _ld(dB_i), _ld(dA_i),
        int(bool(accumulate)), _dt(dZ), _ptr(workspace), _ws_bytes(workspace), _stream(stream)))


def tp_mlp_step_workspace_size(T: int, h: int, F: int, p: int, dt: int) -> int:
    out = ctypes.c_size_t(0)
    _check("tp_mlp_step_workspace_size",
           lib().tp_mlp_step_workspace_size(T, h, F, p, dt, ctypes.byref(out)))
    return int(out.value)


def tp_mlp_step_plan(T: int, h: int, F: int, p: int, dt: int) -> bool:
    """Whether tp_mlp_step runs these shapes fused: the persistent launch, then
    the two stacked weight-gradient products."""
    f = ctypes.c_int(0)
    _check("tp_mlp_step_plan", lib().tp_mlp_step_plan(T, h, F, p, dt, ctypes.byref(f)))
    return bool(f.value)


def tp_attn_proj_step_workspace_size(T: int, h: int, Q: int, O: int, p: int, dt: int) -> int:
    out = ctypes.c_size_t(0)
    _check("tp_attn_proj_step_workspace_size",
           lib().tp_attn_proj_step_workspace_size(T, h, Q, O, p, dt, ctypes.byref(out)))
    return int(out.value)


def tp_attn_proj_step_plan(T: int, h: int, Q: int, O: int, p: int, dt: int) -> bool:
    """Whether tp_attn_proj_step runs these shapes fused: the persistent launch,
    then the two stacked weight-gradient products."""
    f = ctypes.c_int(0)
    _check("tp_attn_proj_step_plan",
           lib().tp_attn_proj_step_plan(T, h, Q, O, p, dt, ctypes.byref(f)))
    return bool(f.value)


ATTN_PROJ_STAGES = {"qkv": 1, "out": 2, "dc": 4, "dx": 8, "wgrad": 16}


def tp_attn_proj_step(X, W, Ow, C, dZa, dQKV, QKV, Zpa, Za, dC, dOw, dW, dXqp, dXq, workspace,
                      stages=31, stream=None):
    """The attention projections of all p shards (layouts in include/tp_mlp.h):
    W [h, p*Q], Ow [p*O, h]; C, dC [T, p*O]; QKV, dQKV [T, p*Q]; Zpa, dXqp fp32
    [p, T, h]; dOw fp32 [p*O, h]; dW fp32 [h, p*Q]. stages: a sum of
    ATTN_PROJ_STAGES (an int, or an iterable of their names); the tensors a
    stage does not touch may be None."""
    if not isinstance(stages, int):
        stages = sum(ATTN_PROJ_STAGES[n] for n in stages)
    chk = _Operands("tp_attn_proj_step")
    chk("X", X, _shape2(X), _torch_dtypes("bf16", "f32"))
    T, h = X.shape
    dts, f32 = (X.dtype,), _torch_dtypes("f32")
    if Zpa is not None and Zpa.dim() == 3:
        p = Zpa.shape[0]
    elif dXqp is not None and dXqp.dim() == 3:
        p = dXqp.shape[0]
    else:
        raise ValueError("tp_attn_proj_step: Zpa or dXqp must be a [p, T, h] tensor")
    chk("W", W, (h, _shape2(W)[1]), dts)("Ow", Ow, (_shape2(Ow)[0], h), dts)
    pQ, pO = W.shape[1], Ow.shape[0]
    if pQ % p or pO % p:
        raise ValueError(f"tp_attn_proj_step: W's {pQ} columns or Ow's {pO} rows do not split "
                         f"into {p} shards")
    Q, O = pQ // p, pO // p
    opt = True
    chk("C", C, (T, pO), dts, optional=opt)("dZa", dZa, (T, h), dts, optional=opt)
    chk("dQKV", dQKV, (T, pQ), dts, optional=opt)("QKV", QKV, (T, pQ), dts, optional=opt)
    chk("Za", Za, (T, h), dts, optional=opt)("dC", dC, (T, pO), dts, optional=opt)
    chk("dXq", dXq, (T, h), dts, optional=opt)
    for name, t in (("Zpa", Zpa), ("dXqp", dXqp)):
        chk(name, t, (p, T, h), f32, optional=opt)
        if t is not None and not t.is_contiguous():
            raise ValueError(f"tp_attn_proj_step: {name} must be contiguous [p, T, h]")
    chk("dOw", dOw, (pO, h), f32, optional=opt)("dW", dW, (h, pQ), f32, optional=opt)
    _check_ws(chk, workspace)
    chk.done(stream)

    def ld(t, w):
        return _ld(t) if t is not None else w
    _check("tp_attn_proj_step", lib().tp_attn_proj_step(
        _ptr(X), _ptr(W), _ptr(Ow), _ptr(C), _ptr(dZa), _ptr(dQKV), _ptr(QKV), _ptr(Zpa),
        _ptr(Za), _ptr(dC), _ptr(dOw), _ptr(dW), _ptr(dXqp), _ptr(dXq), T, h, Q, O, p, _ld(X),
        _ld(W), _ld(Ow), ld(C, pO), ld(dZa, h), ld(dQKV, pQ), ld(QKV, pQ), ld(dC, pO), ld(Za, h),
        ld(dXq, h), ld(dOw, h), ld(dW, pQ), int(stages), _dt(X), _ptr(workspace),
        _ws_bytes(workspace), _stream(stream)))


def tp_set_wait_limit(polls: int = 0) -> None:
    """Test hook: polls before a dependency wait of tp_mlp_step gives up (0:
    the default; negative: at the first unmet check), for this thread."""
    _check("tp_set_wait_limit", lib().tp_set_wait_limit(int(polls)))


def tp_mlp_step(X, A, a, B, b, dZ, U, Y, Zp, Z, dU, dB, db, dA, da, dXp, dX, workspace,
                stream=None, part="step", recompute=False):
    """The MLP step of all p shards (layouts in include/tp_mlp.h): U, Y, dU
    [T, p*F]; Zp, dXp fp32 [p, T, h]; dB fp32 [p*F, h]; dA fp32 [h, p*F].
    part "rows" or "wgrad" runs tp_mlp_step_rows / tp_mlp_step_wgrad, "fwd" or
    "bwd" tp_mlp_step_fwd / tp_mlp_step_bwd (recompute: the backward rebuilds
    Y from U)."""
    fn = {"step": "tp_mlp_step", "rows": "tp_mlp_step_rows", "wgrad": "tp_mlp_step_wgrad",
          "fwd": "tp_mlp_step_fwd", "bwd": "tp_mlp_step_bwd"}[part]
    if recompute and part != "bwd":
        raise ValueError("tp_mlp_step: recompute applies to part 'bwd'")
    chk = _Operands(fn)
    chk("X", X, _shape2(X), _torch_dtypes("bf16", "f32"))
    T, h = X.shape
    dts, f32 = (X.dtype,), _torch_dtypes("f32")
    if Zp is None or Zp.dim() != 3:
        raise ValueError("tp_mlp_step: Zp must be a [p, T, h] tensor")
    p = Zp.shape[0]
    chk("A", A, (h, _shape2(A)[1]), dts)
    pF = A.shape[1]
    if pF % p:
        raise ValueError(f"tp_mlp_step: A's {pF} columns do not split into {p} shards")
    F = pF // p
    chk("a", a, (pF,), dts, optional=True)("B", B, (pF, h), dts)("b", b, (h,), dts, optional=True)
    chk("dZ", dZ, (T, h), dts)("U", U, (T, pF), dts)("Y", Y, (T, pF), dts)
    chk("dU", dU, (T, pF), dts)("Z", Z, (T, h), dts)("dX", dX, (T, h), dts)
    for name, t in (("Zp", Zp), ("dXp", dXp)):
        chk(name, t, (p, T, h), f32)
        if not t.is_contiguous():
            raise ValueError(f"tp_mlp_step: {name} must be contiguous [p, T, h]")
    chk("dB", dB, (pF, h), f32)("db", db, (h,), f32, optional=True)
    chk("dA", dA, (h, pF), f32)("da", da, (pF,), f32, optional=True)
    _check_ws(chk, workspace)
    chk.done(stream)
    if _ld(U) != _ld(Y) or _ld(U) != _ld(dU):
        raise ValueError("tp_mlp_step: U, Y and dU must share a row stride")
    _check(fn, getattr(lib(), fn)(
        _ptr(X), _ptr(A), _ptr(a), _ptr(B), _ptr(b), _ptr(dZ), _ptr(U), _ptr(Y), _ptr(Zp),
        _ptr(Z), _ptr(dU), _ptr(dB), _ptr(db), _ptr(dA), _ptr(da), _ptr(dXp), _ptr(dX),
        T, h, F, p, _ld(X), _ld(A), _ld(B), _ld(dZ), _ld(U), _ld(Z), _ld(dX), _ld(dB), _ld(dA),
        *([int(bool(recompute))] if part == "bwd" else []),
        _dt(X), _ptr(workspace), _ws_bytes(workspace), _stream(stream)))


def tp_reduce_partials(partials, bias, out, stream=None):
    chk = _Operands("tp_reduce_partials")
    if not partials:
        raise ValueError("tp_reduce_partials: no partials")
    p = len(partials)
    chk("partials[0]", partials[0], _shape2(partials[0]), _torch_dtypes("f32"))
    T, h = partials[0].shape
    ld_p = _ld(partials[0])
    for i, P in enumerate(partials[1:], 1):
        chk(f"partials[{i}]", P, (T, h), _torch_dtypes("f32"))
        if _ld(P) != ld_p:
            raise ValueError("partials must share shape and row stride")
    chk("out", out, (T, h), _torch_dtypes("bf16", "f32"))
    chk("bias", bias, (h,), (out.dtype,), optional=True).done(stream)
    arr = (ctypes.c_void_p * p)(*[P.data_ptr() for P in partials])
    _check("tp_reduce_partials", lib().tp_reduce_partials(
        arr, p, _ptr(bias), _ptr(out), T, h, ld_p, _ld(out), _dt(out), _stream(stream)))


def tp_bias_act(U, bias, Y, act="gelu", stream=None):
    chk = _Operands("tp_bias_act")
    chk("U", U, _shape2(U), _torch_dtypes("bf16", "f32"))
    T, n = U.shape
    chk("bias", bias, (n,), (U.dtype,), optional=True)
    chk("Y", Y, (T, n), _torch_dtypes("bf16", "f32")).done(stream)
    _check("tp_bias_act", lib().tp_bias_act(
        _ptr(U), _ptr(bias), _ptr(Y), T, n, _ld(U), _ld(Y), _dt(U), _dt(Y), _act(act),
        _stream(stream)))


def tp_gemm_plan(M: int, N: int, K: int, allow_split: bool = False):
    """(tile id, K slices, K per slice) the library uses for a bf16 product."""
    t, sk, kc = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int64(0)
    _check("tp_gemm_plan", lib().tp_gemm_plan(M, N, K, int(bool(allow_split)), ctypes.byref(t),
                                               ctypes.byref(sk), ctypes.byref(kc)))
    return int(t.value), int(sk.value), int(kc.value)


def tp_attention_fwd(QKV, C, lse, batch: int, seq: int, heads: int, causal: bool = True,
                     stream=None, shards: int = 1):
    """Attention core of one shard: QKV [batch*seq, 3*heads*64] bf16 -> C
    [batch*seq, heads*64] bf16 and lse [batch, heads, seq] fp32 (or None).
    shards > 1: that many shards of `heads` heads side by side in one launch
    (tp_attention_fwd_shards): QKV [.., shards*3*heads*64], C [.., shards*heads*64],
    lse [batch, shards*heads, seq]."""
    fn = "tp_attention_fwd" if shards == 1 else "tp_attention_fwd_shards"
    chk = _Operands(fn)
    H = heads * shards
    T, hd, bf = batch * seq, H * 64, _torch_dtypes("bf16")
    chk("QKV", QKV, (T, 3 * hd), bf)("C", C, (T, hd), bf)
    if lse is not None:
        chk("lse", lse, (batch * H * seq,) if lse.dim() == 1 else (batch, H, seq),
            _torch_dtypes("f32"))
        if not lse.is_contiguous():
            raise ValueError(f"{fn}: lse must be contiguous")
    chk.done(stream)
    extra = [] if shards == 1 else [shards]
    _check(fn, getattr(lib(), fn)(
        _ptr(QKV), _ptr(C), _ptr(lse), batch, seq, heads, *extra, 64, _ld(QKV), _ld(C),
        int(bool(causal)), _dt(QKV), _stream(stream)))


def tp_attention_bwd(QKV, C, dC, lse, delta, dQKV, batch: int, seq: int, heads: int,
                     causal: bool = True, stream=None, shards: int = 1):
    """Backward of tp_attention_fwd: dQKV (laid out like QKV) from dC, the
    forward's C and lse; delta [batch, heads, seq] fp32 is a workspace.
    shards as tp_attention_fwd (delta [batch, shards*heads, seq])."""
    fn = "tp_attention_bwd" if shards == 1 else "tp_attention_bwd_shards"
    chk = _Operands(fn)
    H = heads * shards
    T, hd, bf, f32 = batch * seq, H * 64, _torch_dtypes("bf16"), _torch_dtypes("f32")
    chk("QKV", QKV, (T, 3 * hd), bf)("C", C, (T, hd), bf)("dC", dC, (T, hd), bf)
    chk("dQKV", dQKV, (T, 3 * hd), bf)
    for name, t in (("lse", lse), ("delta", delta)):
        chk(name, t, (batch * H * seq,) if t is not None and t.dim() == 1
            else (batch, H, seq), f32)
        if not t.is_contiguous():
            raise ValueError(f"{fn}: {name} must be contiguous")
    chk.done(stream)
    extra = [] if shards == 1 else [shards]
    _check(fn, getattr(lib(), fn)(
        _ptr(QKV), _ptr(C), _ptr(dC), _ptr(lse), _ptr(delta), _ptr(dQKV), batch, seq, heads,
        *extra, 64, _ld(QKV), _ld(C), _ld(dC), _ld(dQKV), int(bool(causal)), _dt(QKV),
        _stream(stream)))


TP_FP8_E4M3, TP_FP8_E5M2 = 0, 1


def _fmt(fmt) -> int:
    return {"e4m3": TP_FP8_E4M3, "e5m2": TP_FP8_E5M2, 0: 0, 1: 1}[fmt]


def tp_fp8_quantize_workspace_size(rows: int, cols: int) -> int:
    out = ctypes.c_size_t(0)
    _check("tp_fp8_quantize_workspace_size",
           lib().tp_fp8_quantize_workspace_size(rows, cols, ctypes.byref(out)))
    return int(out.value)


def tp_fp8_quantize(X, Q, scale_inv, workspace, fmt="e4m3", transpose=False, stream=None):
    """Codes of X (or X^T) into the uint8 tensor Q; scale_inv (fp32 [1]) = 1/s."""
    chk = _Operands("tp_fp8_quantize")
    chk("X", X, _shape2(X), _torch_dtypes("bf16", "f32"))
    rows, cols = X.shape
    chk("Q", Q, (cols, rows) if transpose else (rows, cols), _torch_dtypes("u8"))
    chk("scale_inv", scale_inv, (1,), _torch_dtypes("f32"))
    if workspace is None:
        raise ValueError("tp_fp8_quantize: workspace is required")
    _check_ws(chk, workspace)
    chk.done(stream)
    _check("tp_fp8_quantize", lib().tp_fp8_quantize(
        _ptr(X), rows, cols, _ld(X), _dt(X), _fmt(fmt), int(bool(transpose)), _ptr(Q), _ld(Q),
        _ptr(scale_inv), _ptr(workspace), _ws_bytes(workspace), _stream(stream)))


def tp_fp8_quantize_both(X, Q, Qt, scale_inv, workspace, fmt="e4m3", stream=None):
    """Codes of X into Q and of X^T into Qt from one read; scale_inv = 1/s."""
    chk = _Operands("tp_fp8_quantize_both")
    chk("X", X, _shape2(X), _torch_dtypes("bf16", "f32"))
    rows, cols = X.shape
    u8 = _torch_dtypes("u8")
    chk("Q", Q, (rows, cols), u8)("Qt", Qt, (cols, rows), u8)
    chk("scale_inv", scale_inv, (1,), _torch_dtypes("f32"))
    if workspace is None:
        raise ValueError("tp_fp8_quantize_both: workspace is required")
    _check_ws(chk, workspace)
    chk.done(stream)
    _check("tp_fp8_quantize_both", lib().tp_fp8_quantize_both(
        _ptr(X), rows, cols, _ld(X), _dt(X), _fmt(fmt), _ptr(Q), _ld(Q), _ptr(Qt), _ld(Qt),
        _ptr(scale_inv), _ptr(workspace), _ws_bytes(workspace), _stream(stream)))


def tp_fp8_quantize_multi_workspace_size(n: int) -> int:
    out = ctypes.c_size_t(0)
    _check("tp_fp8_quantize_multi_workspace_size",
           lib().tp_fp8_quantize_multi_workspace_size(n, ctypes.byref(out)))
    return int(out.value)


def tp_fp8_quantize_both_multi(items, workspace, stream=None):
    """tp_fp8_quantize_both for each (X, Q, Qt, scale_inv, fmt) of `items` (at
    most 6) in two launches in all."""
    chk = _Operands("tp_fp8_quantize_both_multi")
    n = len(items)
    u8 = _torch_dtypes("u8")
    for j, (x, q, qt, si, _) in enumerate(items):
        chk(f"X[{j}]", x, _shape2(x), _torch_dtypes("bf16", "f32"))
        chk(f"Q[{j}]", q, tuple(x.shape), u8)(f"Qt[{j}]", qt, tuple(x.shape)[::-1], u8)
        chk(f"scale_inv[{j}]", si, (1,), _torch_dtypes("f32"))
    if workspace is None:
        raise ValueError("tp_fp8_quantize_both_multi: workspace is required")
    _check_ws(chk, workspace)
    chk.done(stream)
    vp = ctypes.c_void_p * n
    i64 = ctypes.c_int64 * n
    i32 = ctypes.c_int * n
    X = vp(*[x.data_ptr() for x, *_ in items])
    rows = i64(*[x.shape[0] for x, *_ in items])
    cols = i64(*[x.shape[1] for x, *_ in items])
    ld_x = i64(*[_ld(x) for x, *_ in items])
    dt = i32(*[_dt(x) for x, *_ in items])
    fmt = i32(*[_fmt(f) for *_, f in items])
    Q = vp(*[q.data_ptr() for _, q, *_ in items])
    ld_q = i64(*[_ld(q) for _, q, *_ in items])
    Qt = vp(*[qt.data_ptr() for _, _, qt, *_ in items])
    ld_qt = i64(*[_ld(qt) for _, _, qt, *_ in items])
    si = vp(*[s.data_ptr() for _, _, _, s, _ in items])
    _check("tp_fp8_quantize_both_multi", lib().tp_fp8_quantize_both_multi(
        n, X, rows, cols, ld_x, dt, fmt, Q, ld_q, Qt, ld_qt, si, _ptr(workspace),
        _ws_bytes(workspace), _stream(stream)))


def tp_fp8_amax_slots(M: int, N: int, K: int) -> int:
    """Floats of amax slots the _amax FP8 products write for an M x N output."""
    out = ctypes.c_int64(0)
    _check("tp_fp8_amax_slots", lib().tp_fp8_amax_slots(M, N, K, ctypes.byref(out)))
    return int(out.value)


def tp_fp8_quantize_both_from_amax(X, Q, Qt, scale_inv, amax, n_amax, fmt="e4m3", stream=None):
    """tp_fp8_quantize_both with the maxima of |X| given (n_amax amax slots of
    the product that wrote X): one launch."""
    chk = _Operands("tp_fp8_quantize_both_from_amax")
    chk("X", X, _shape2(X), _torch_dtypes("bf16", "f32"))
    rows, cols = X.shape
    u8, f32 = _torch_dtypes("u8"), _torch_dtypes("f32")
    chk("Q", Q, (rows, cols), u8)("Qt", Qt, (cols, rows), u8)
    chk("scale_inv", scale_inv, (1,), f32)
    if amax is None or amax.dim() != 1 or amax.numel() < n_amax:
        raise ValueError(f"tp_fp8_quantize_both_from_amax: amax must hold {n_amax} floats")
    chk("amax", amax, (amax.numel(),), f32).done(stream)
    _check("tp_fp8_quantize_both_from_amax", lib().tp_fp8_quantize_both_from_amax(
        _ptr(X), rows, cols, _ld(X), _dt(X), _fmt(fmt), _ptr(Q), _ld(Q), _ptr(Qt), _ld(Qt),
        _ptr(scale_inv), _ptr(amax), int(n_amax), _stream(stream)))


def tp_fp8_column_linear_fwd(Xq, Atq, x_si, a_si, bias, Y, U, act="gelu", amax=None,
                             stream=None):
    """With amax (act "gelu" only): also the amax slots of |Y| (tp_fp8_amax_slots floats)."""
    chk = _Operands("tp_fp8_column_linear_fwd")
    u8, f32, bf = _torch_dtypes("u8"), _torch_dtypes("f32"), _torch_dtypes("bf16")
    chk("Xq", Xq, _shape2(Xq), u8)
    T, h = Xq.shape
    chk("Atq", Atq, (_shape2(Atq)[0], h), u8)
    n = Atq.shape[0]
    chk("x_scale_inv", x_si, (1,), f32)("a_scale_inv", a_si, (1,), f32)
    none = _act(act) == TP_ACT_NONE
    chk("bias", bias, (n,), bf, optional=True)("Y", Y, (T, n), bf)
    chk("U", U, (T, n), bf, optional=none)
    if amax is not None:
        if none:
            raise ValueError("tp_fp8_column_linear_fwd: amax needs act 'gelu'")
        chk("amax", amax, (tp_fp8_amax_slots(T, n, h),), f32).done(stream)
        _check("tp_fp8_column_linear_fwd_amax", lib().tp_fp8_column_linear_fwd_amax(
            _ptr(Xq), _ptr(Atq), _ptr(x_si), _ptr(a_si), _ptr(bias), _ptr(Y), _ptr(U), T, h, n,
            _ld(Xq), _ld(Atq), _ld(Y), _ptr(amax), _stream(stream)))
        return
    chk.done(stream)
    _check("tp_fp8_column_linear_fwd", lib().tp_fp8_column_linear_fwd(
        _ptr(Xq), _ptr(Atq), _ptr(x_si), _ptr(a_si), _ptr(bias), _ptr(Y), _ptr(U), T, h, n,
        _ld(Xq), _ld(Atq), _ld(Y), _act(act), _stream(stream)))


def tp_fp8_row_linear_fwd_partial(Yq, Btq, y_si, b_si, Zp, stream=None):
    chk = _Operands("tp_fp8_row_linear_fwd_partial")
    u8, f32 = _torch_dtypes("u8"), _torch_dtypes("f32")
    chk("Yq", Yq, _shape2(Yq), u8)
    T, k = Yq.shape
    chk("Btq", Btq, (_shape2(Btq)[0], k), u8)
    h = Btq.shape[0]
    chk("y_scale_inv", y_si, (1,), f32)("b_scale_inv", b_si, (1,), f32)
    chk("Zp", Zp, (T, h), f32).done(stream)
    _check("tp_fp8_row_linear_fwd_partial", lib().tp_fp8_row_linear_fwd_partial(
        _ptr(Yq), _ptr(Btq), _ptr(y_si), _ptr(b_si), _ptr(Zp), T, k, h, _ld(Yq), _ld(Btq),
        _ld(Zp), _stream(stream)))


def tp_fp8_linear_bwd_dgrad(dOutq, Wq, d_si, w_si, dIn, U=None, act="none", dout_fmt="e5m2",
                            amax=None, stream=None):
    """With amax (act "gelu", bf16 dIn only): also the amax slots of |dIn|."""
    chk = _Operands("tp_fp8_linear_bwd_dgrad")
    u8, f32, bf = _torch_dtypes("u8"), _torch_dtypes("f32"), _torch_dtypes("bf16")
    chk("dOutq", dOutq, _shape2(dOutq), u8)
    T, n = dOutq.shape
    chk("Wq", Wq, (_shape2(Wq)[0], n), u8)
    k = Wq.shape[0]
    chk("dout_scale_inv", d_si, (1,), f32)("w_scale_inv", w_si, (1,), f32)
    chk("U", U, (T, k), bf, optional=_act(act) == TP_ACT_NONE)
    chk("dIn", dIn, (T, k), _torch_dtypes("bf16", "f32"))
    ld_u = _ld(U) if U is not None else k
    if amax is not None:
        if _act(act) != TP_ACT_GELU_TANH or dIn.dtype != _torch_dtypes("bf16")[0]:
            raise ValueError("tp_fp8_linear_bwd_dgrad: amax needs act 'gelu' and a bf16 dIn")
        chk("amax", amax, (tp_fp8_amax_slots(T, k, n),), f32).done(stream)
        _check("tp_fp8_linear_bwd_dgrad_amax", lib().tp_fp8_linear_bwd_dgrad_amax(
            _ptr(dOutq), _ptr(Wq), _ptr(d_si), _ptr(w_si), _fmt(dout_fmt), _ptr(U), _ptr(dIn), T,
            k, n, _ld(dOutq), _ld(Wq), ld_u, _ld(dIn), _ptr(amax), _stream(stream)))
        return
    chk.done(stream)
    _check("tp_fp8_linear_bwd_dgrad", lib().tp_fp8_linear_bwd_dgrad(
        _ptr(dOutq), _ptr(Wq), _ptr(d_si), _ptr(w_si), _fmt(dout_fmt), _ptr(U), _act(act),
        _ptr(dIn), T, k, n, _ld(dOutq), _ld(Wq), ld_u, _ld(dIn), _dt(dIn), _stream(stream)))


def tp_fp8_linear_bwd_wgrad_workspace_size(T: int, k: int, n: int) -> int:
    out = ctypes.c_size_t(0)
    _check("tp_fp8_linear_bwd_wgrad_workspace_size",
           lib().tp_fp8_linear_bwd_wgrad_workspace_size(T, k, n, ctypes.byref(out)))
    return int(out.value)


def tp_fp8_linear_bwd_wgrad(Intq, dOuttq, in_si, d_si, dW, dOut=None, dbias=None,
                            dout_fmt="e5m2", workspace=None, stream=None):
    chk = _Operands("tp_fp8_linear_bwd_wgrad")
    u8, f32 = _torch_dtypes("u8"), _torch_dtypes("f32")
    chk("Intq", Intq, _shape2(Intq), u8)
    k, T = Intq.shape
    chk("dOuttq", dOuttq, (_shape2(dOuttq)[0], T), u8)
    n = dOuttq.shape[0]
    chk("in_scale_inv", in_si, (1,), f32)("dout_scale_inv", d_si, (1,), f32)
    chk("dW", dW, (k, n), f32)("dbias", dbias, (n,), f32, optional=True)
    chk("dOut", dOut, (T, n), _torch_dtypes("bf16"), optional=dbias is None)
    _check_ws(chk, workspace)
    chk.done(stream)
    _check("tp_fp8_linear_bwd_wgrad", lib().tp_fp8_linear_bwd_wgrad(
        _ptr(Intq), _ptr(dOuttq), _ptr(in_si), _ptr(d_si), _fmt(dout_fmt), _ptr(dW), _ptr(dOut),
        _ptr(dbias), T, k, n, _ld(Intq), _ld(dOuttq), _ld(dW),
        _ld(dOut) if dOut is not None else n, _ptr(workspace), _ws_bytes(workspace),
        _stream(stream)))


def tp_set_gemm_override(tile: int = 0, splitk: int = 1) -> None:
    """Force a pipelined tile (and K slices for weight gradients) on every later
    bf16 product whose shape it supports; tile 0 restores the library's choice."""
    _check("tp_set_gemm_override", lib().tp_set_gemm_override(int(tile), int(splitk)))


def tp_status_string(status: int) -> str:
    return lib().tp_status_string(status).decode()


def tp_last_hip_error() -> int:
    return int(lib().tp_last_hip_error())
