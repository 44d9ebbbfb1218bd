"""Python binding of libbi.so, the deterministic batch-invariant GEMM library.

Argument marshalling only: every function forwards to the C entry point of the
same name declared in include/bi.h and returns its integer status.  Pointers
may be given as integers (device addresses) or as objects with ``data_ptr()``
(e.g. torch tensors); streams as integer ``hipStream_t`` handles or objects
with a ``cuda_stream`` attribute (torch streams); ``None`` means NULL / the null
stream.  No computation happens in Python and there is no fallback: if the
library is not built, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbi.so")
# the same kernels with the tile-forcing values of tc (tc = 16 + tile id, plus
# 4096 for the fp8 fast path on that tile): tile-identity tests and tile tuning
LIB_TESTING_PATH = os.path.join(HERE, "libbi_testing.so")

BI_F32, BI_BF16, BI_F16 = 0, 1, 2
BI_FP8_E4M3, BI_FP8_E5M2 = 3, 4
BI_OK = 0
BI_STATIC_SCRATCH_BYTES = 64 << 20
TC_SCALAR, TC_AUTO, TC_MFMA, TC_FP8_FAST = 0, 1, 2, 3
STATUS = {0: "BI_OK", -1: "BI_ERR_NULL", -2: "BI_ERR_DTYPE", -3: "BI_ERR_SHAPE",
          -4: "BI_ERR_TOO_LARGE", -5: "BI_ERR_WORKSPACE", -6: "BI_ERR_HIP",
          -7: "BI_ERR_UNSUPPORTED"}
OP_FWD, OP_DX, OP_DW, OP_FP8, OP_GFWD, OP_GDIN, OP_GDW = range(7)

_lib = None
_lib_testing = None


class BIError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}" if what else status_string(status))


def load() -> ctypes.CDLL:
    """Load libbi.so (built by ``build.build()``); raise if it is missing."""
    global _lib
    if _lib is None:
        _lib = _bind(LIB_PATH)
    return _lib


class testing_build:
    """Context manager: the entry points of this module call libbi_testing.so
    (tile-forcing tc values accepted) instead of libbi.so while it is open."""

    def __enter__(self):
        global _lib, _lib_testing
        if _lib_testing is None:
            _lib_testing = _bind(LIB_TESTING_PATH)
        self._saved = load()
        _lib = _lib_testing
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def _bind(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run deterministic_invariant_gemm_amd."
                           "build.build() (hipcc, gfx950) first")
    L = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.bi_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, i32]
    L.bi_backward_dx.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, i32]
    L.bi_backward_dw_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    L.bi_backward_dw_workspace_bytes.restype = sz
    L.bi_backward_dw.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, sz, vp, i32]
    L.bi_fp8_mm.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, i32]
    L.bi_linear_backward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp, i32]
    L.bi_linear_backward.restype = i32
    L.bi_linear_backward_static.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i32]
    L.bi_linear_backward_static.restype = i32
    L.bi_bias_grad_workspace_bytes.argtypes = [i64, i64, i32]
    L.bi_bias_grad_workspace_bytes.restype = sz
    L.bi_bias_grad.argtypes = [vp, vp, i64, i64, i32, vp, sz, vp]
    L.bi_bias_grad.restype = i32
    L.bi_grouped_nt.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp, i32]
    L.bi_grouped_nt_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32,
                                         vp, i32]
    L.bi_fp8_quantize.argtypes = [vp, vp, vp, vp, i64, i32, vp]
    L.bi_fp8_transpose_quantize.argtypes = [vp, vp, vp, vp, i64, i64, i32, vp]
    L.bi_fp8_linear_workspace_bytes.argtypes = [i64, i64, i64]
    L.bi_fp8_linear_workspace_bytes.restype = sz
    L.bi_fp8_linear_forward.argtypes = [vp] * 10 + [i64] * 3 + [vp, sz, vp, i32]
    L.bi_fp8_linear_backward.argtypes = [vp] * 12 + [i64] * 3 + [vp, sz, vp, i32]
    for f in ("bi_fp8_quantize", "bi_fp8_transpose_quantize", "bi_fp8_linear_forward",
              "bi_fp8_linear_backward"):
        getattr(L, f).restype = i32
    L.bi_status_string.argtypes = [i32]
    L.bi_status_string.restype = ctypes.c_char_p
    L.bi_plan.argtypes = [i32, i32, i32, i64, i64, ctypes.POINTER(i64)]
    L.bi_plan_batch.argtypes = [i32, i32, i32, i64, i64, i64, i64]
    for f in ("bi_forward", "bi_backward_dx", "bi_backward_dw", "bi_fp8_mm", "bi_grouped_nt",
              "bi_grouped_nt_backward", "bi_plan", "bi_plan_batch"):
        getattr(L, f).restype = i32
    return L


def _p(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _s(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def status_string(status: int) -> str:
    try:
        return load().bi_status_string(int(status)).decode()
    except RuntimeError:
        return STATUS.get(int(status), f"unknown status {status}")


def check(status: int, what: str = "") -> None:
    if status != BI_OK:
        raise BIError(status, what)


def bi_forward(y, x, w, bias, m, k, n, dtype, stream=None, tc=1) -> int:
    return load().bi_forward(_p(y), _p(x), _p(w), _p(bias), m, k, n, dtype, _s(stream), tc)


def bi_backward_dx(dx, dy, w, m, k, n, dtype, stream=None, tc=1) -> int:
    return load().bi_backward_dx(_p(dx), _p(dy), _p(w), m, k, n, dtype, _s(stream), tc)


def bi_backward_dw_workspace_bytes(m, k, n, dtype, tc=1) -> int:
    return load().bi_backward_dw_workspace_bytes(m, k, n, dtype, tc)


def bi_backward_dw(dw, x, dy, m, k, n, dtype, workspace, workspace_bytes, stream=None,
                   tc=1) -> int:
    return load().bi_backward_dw(_p(dw), _p(x), _p(dy), m, k, n, dtype, _p(workspace),
                                 workspace_bytes, _s(stream), tc)


def bi_linear_backward(dx, dw, dy, x, w, m, k, n, dtype, workspace, workspace_bytes, stream=None,
                       tc=1) -> int:
    return load().bi_linear_backward(_p(dx), _p(dw), _p(dy), _p(x), _p(w), m, k, n, dtype,
                                     _p(workspace), workspace_bytes, _s(stream), tc)


def bi_linear_backward_static(dx, dw, dy, x, w, m, k, n, dtype, stream=None, tc=1) -> int:
    return load().bi_linear_backward_static(_p(dx), _p(dw), _p(dy), _p(x), _p(w), m, k, n, dtype,
                                            _s(stream), tc)


def bi_bias_grad_workspace_bytes(m, n, dtype) -> int:
    return load().bi_bias_grad_workspace_bytes(m, n, dtype)


def bi_bias_grad(db, dy, m, n, dtype, workspace, workspace_bytes, stream=None) -> int:
    return load().bi_bias_grad(_p(db), _p(dy), m, n, dtype, _p(workspace), workspace_bytes,
                               _s(stream))


def bi_fp8_mm(y, a, bt, a_dequant, b_dequant, m, k, n, stream=None, tc=1) -> int:
    return load().bi_fp8_mm(_p(y), _p(a), _p(bt), _p(a_dequant), _p(b_dequant), m, k, n,
                            _s(stream), tc)


def bi_fp8_quantize(dst, src, scale_inv, amax, n, fmt, stream=None) -> int:
    return load().bi_fp8_quantize(_p(dst), _p(src), _p(scale_inv), _p(amax), n, fmt, _s(stream))


def bi_fp8_transpose_quantize(dst, src, scale_inv, amax, rows, cols, fmt, stream=None) -> int:
    return load().bi_fp8_transpose_quantize(_p(dst), _p(src), _p(scale_inv), _p(amax), rows,
                                            cols, fmt, _s(stream))


def bi_fp8_linear_workspace_bytes(m, k, n) -> int:
    return load().bi_fp8_linear_workspace_bytes(m, k, n)


def bi_fp8_linear_forward(y, x, w, bias, sx, sw, sx_inv, sw_inv, amax_x, amax_w, m, k, n,
                          workspace, workspace_bytes, stream=None, tc=1) -> int:
    return load().bi_fp8_linear_forward(_p(y), _p(x), _p(w), _p(bias), _p(sx), _p(sw),
                                        _p(sx_inv), _p(sw_inv), _p(amax_x), _p(amax_w), m, k, n,
                                        _p(workspace), workspace_bytes, _s(stream), tc)


def bi_fp8_linear_backward(dx, dw, g, x, w, sg, sw, sx, sg_inv, sw_inv, sx_inv, amax_g, m, k, n,
                           workspace, workspace_bytes, stream=None, tc=1) -> int:
    return load().bi_fp8_linear_backward(_p(dx), _p(dw), _p(g), _p(x), _p(w), _p(sg), _p(sw),
                                         _p(sx), _p(sg_inv), _p(sw_inv), _p(sx_inv), _p(amax_g),
                                         m, k, n, _p(workspace), workspace_bytes, _s(stream), tc)


def bi_grouped_nt(y, inp, weights, row_experts, offsets, m, k, n, e, dtype, stream=None,
                  tc=1) -> int:
    return load().bi_grouped_nt(_p(y), _p(inp), _p(weights), _p(row_experts), _p(offsets),
                                m, k, n, e, dtype, _s(stream), tc)


def bi_grouped_nt_backward(dinput, dweights, inp, weights, grad_out, row_experts, offsets,
                           m, k, n, e, dtype, stream=None, tc=1) -> int:
    return load().bi_grouped_nt_backward(_p(dinput), _p(dweights), _p(inp), _p(weights),
                                         _p(grad_out), _p(row_experts), _p(offsets), m, k, n,
                                         e, dtype, _s(stream), tc)


def bi_plan(op, dtype, tc, k, n):
    """(tier/tile id, dW chunk rows) the dispatcher picks for these arguments."""
    chunk = ctypes.c_int64(0)
    r = load().bi_plan(op, dtype, tc, k, n, ctypes.byref(chunk))
    return r, chunk.value


def bi_plan_batch(op, dtype, tc, m, k, n, e=0):
    """Tile id a call with batch m (e experts for the grouped forward) launches
    on aligned operands (0: scalar tier)."""
    return load().bi_plan_batch(op, dtype, tc, m, k, n, e)


def bi_status_string(status: int) -> str:
    return status_string(status)
