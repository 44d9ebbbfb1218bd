"""CPU oracle for the deterministic GEMM library (test infrastructure only).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
import this package.  The product library never loads it, and it shares no code
with the HIP path.  The arithmetic lives in ``oracle.c`` (plain C, f64
accumulation, one round-to-nearest-even at the end); this module only marshals
numpy arrays into it with ctypes.

Dtype codes: 0 = f32, 1 = bf16, 2 = f16 (storage as uint32 / uint16 bit
patterns); fp8 formats 3 = e4m3fn, 4 = e5m2 (codes are uint8).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC_PATH = os.path.join(HERE, "oracle.c")

F32, BF16, F16, E4M3, E5M2 = 0, 1, 2, 3, 4
STORAGE = {F32: np.uint32, BF16: np.uint16, F16: np.uint16}


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU involved)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-pthread", SRC_PATH,
           "-o", LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        # ORACLE_LIB lets the mutation test load a deliberately broken copy
        path = os.environ.get("ORACLE_LIB", LIB_PATH)
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_decode_bf16.argtypes = [ctypes.c_uint16]
        L.orc_decode_bf16.restype = ctypes.c_double
        L.orc_decode_f16.argtypes = [ctypes.c_uint16]
        L.orc_decode_f16.restype = ctypes.c_double
        L.orc_decode_e4m3.argtypes = [ctypes.c_uint8]
        L.orc_decode_e4m3.restype = ctypes.c_double
        L.orc_decode_f32_bits.argtypes = [ctypes.c_uint32]
        L.orc_decode_f32_bits.restype = ctypes.c_double
        L.orc_rne_bf16.argtypes = [ctypes.c_double]
        L.orc_rne_bf16.restype = ctypes.c_uint16
        L.orc_rne_f16.argtypes = [ctypes.c_double]
        L.orc_rne_f16.restype = ctypes.c_uint16
        L.orc_rne_f32.argtypes = [ctypes.c_double]
        L.orc_rne_f32.restype = ctypes.c_uint32
        L.orc_rne_e4m3_sat.argtypes = [ctypes.c_double]
        L.orc_rne_e4m3_sat.restype = ctypes.c_uint8
        L.orc_decode_e5m2.argtypes = [ctypes.c_uint8]
        L.orc_decode_e5m2.restype = ctypes.c_double
        L.orc_rne_e5m2_sat.argtypes = [ctypes.c_double]
        L.orc_rne_e5m2_sat.restype = ctypes.c_uint8
        f32 = ctypes.c_float
        L.orc_fp8_quantize.argtypes = [i32, vp, f32, i64, vp, vp]
        L.orc_fp8_transpose_quantize.argtypes = [i32, vp, f32, i64, i64, vp, vp]
        L.orc_fp8_linear_forward.argtypes = [vp, vp, vp, f32, f32, f32, f32, i64, i64, i64, vp,
                                             i64, vp, vp, vp, vp, vp, vp, i32]
        L.orc_fp8_linear_backward.argtypes = [i32, vp, vp, vp, f32, f32, f32, f32, f32, f32,
                                              i64, i64, i64, vp, i64, vp, vp, vp, vp, vp, i32]
        common = [i64, i64, i64, vp, i64, vp, vp, vp, i32]
        L.orc_linear_forward.argtypes = [i32, vp, vp, vp] + common
        L.orc_linear_dx.argtypes = [i32, vp, vp] + common
        L.orc_linear_dw.argtypes = [i32, vp, vp] + common
        L.orc_fp8_mm.argtypes = [vp, vp, ctypes.c_float, ctypes.c_float, i64, i64, i64, vp, i64,
                                 vp, vp, vp, vp, i32]
        gcommon = [vp, i64, i64, i64, i64, vp, i64, vp, vp, vp, i32]
        L.orc_grouped_fwd.argtypes = [i32, vp, vp] + gcommon
        L.orc_grouped_dinput.argtypes = [i32, vp, vp] + gcommon
        L.orc_grouped_dweights.argtypes = [i32, vp, vp] + gcommon
        L.orc_bias_grad.argtypes = [i32, vp, i64, i64, vp, vp, vp]
        L.orc_bias_grad.restype = i32
        for f in ("orc_linear_forward", "orc_linear_dx", "orc_linear_dw", "orc_fp8_mm",
                  "orc_grouped_fwd", "orc_grouped_dinput", "orc_grouped_dweights",
                  "orc_fp8_quantize", "orc_fp8_transpose_quantize", "orc_fp8_linear_forward",
                  "orc_fp8_linear_backward"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _rows_arg(rows, total):
    if rows is None:
        return None, total
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < total))
    return r, r.size


class Result:
    """Rounded output bits plus the exact pre-rounding value S and the
    absolute-product scale A for every computed element (fp8 results also
    carry .g: the sum over 8-index groups of the largest |product|)."""

    def __init__(self, out, s, a):
        self.out, self.s, self.a = out, s, a
        self.g = None


def _alloc(nrows, ncols, dt):
    out = np.zeros((nrows, ncols), dtype=STORAGE[dt])
    s = np.zeros((nrows, ncols), dtype=np.float64)
    a = np.zeros((nrows, ncols), dtype=np.float64)
    return out, s, a


def linear_forward(dt, x, w, bias, m, k, n, rows=None, threads=None):
    """Y = RNE_T(X W + b) for the selected rows of M.  x: [m,k], w: [k,n]
    (weight stored [in,out]), bias: [n] or None; arrays hold bit patterns."""
    st = STORAGE[dt]
    x, w = _c(x, st), _c(w, st)
    bias = None if bias is None else _c(bias, st)
    r, nr = _rows_arg(rows, m)
    out, s, a = _alloc(nr, n, dt)
    rc = lib().orc_linear_forward(dt, _ptr(x), _ptr(w), _ptr(bias), m, k, n, _ptr(r), nr,
                                  _ptr(out), _ptr(s), _ptr(a), threads or default_threads())
    assert rc == 0
    return Result(out, s, a)


def linear_dx(dt, dy, w, m, k, n, rows=None, threads=None):
    """dX = RNE_T(dY W^T) for the selected rows of M.  dy: [m,n], w: [k,n]."""
    st = STORAGE[dt]
    dy, w = _c(dy, st), _c(w, st)
    r, nr = _rows_arg(rows, m)
    out, s, a = _alloc(nr, k, dt)
    rc = lib().orc_linear_dx(dt, _ptr(dy), _ptr(w), m, k, n, _ptr(r), nr, _ptr(out), _ptr(s),
                             _ptr(a), threads or default_threads())
    assert rc == 0
    return Result(out, s, a)


def linear_dw(dt, x, dy, m, k, n, rows=None, threads=None):
    """dW = RNE_T(X^T dY) for the selected rows of K.  x: [m,k], dy: [m,n]."""
    st = STORAGE[dt]
    x, dy = _c(x, st), _c(dy, st)
    r, nr = _rows_arg(rows, k)
    out, s, a = _alloc(nr, n, dt)
    rc = lib().orc_linear_dw(dt, _ptr(x), _ptr(dy), m, k, n, _ptr(r), nr, _ptr(out), _ptr(s),
                             _ptr(a), threads or default_threads())
    assert rc == 0
    return Result(out, s, a)


def fp8_mm(a8, bt8, da, db, m, k, n, rows=None, threads=None):
    """Y = RNE_bf16((A8 B8^T) * da * db); a8: [m,k] e4m3fn codes, bt8: [n,k]."""
    a8, bt8 = _c(a8, np.uint8), _c(bt8, np.uint8)
    r, nr = _rows_arg(rows, m)
    out = np.zeros((nr, n), dtype=np.uint16)
    s = np.zeros((nr, n), dtype=np.float64)
    a = np.zeros((nr, n), dtype=np.float64)
    g = np.zeros((nr, n), dtype=np.float64)
    rc = lib().orc_fp8_mm(_ptr(a8), _ptr(bt8), float(np.float32(da)), float(np.float32(db)),
                          m, k, n, _ptr(r), nr, _ptr(out), _ptr(s), _ptr(a), _ptr(g),
                          threads or default_threads())
    assert rc == 0
    res = Result(out, s, a)
    res.g = g
    return res


def bias_grad(dt, dy, m, n):
    """db = RNE_T(column sums of dY); dy: [m, n] bit patterns."""
    dy = _c(dy, STORAGE[dt])
    out, s, a = _alloc(1, n, dt)
    rc = lib().orc_bias_grad(dt, _ptr(dy), m, n, _ptr(out), _ptr(s), _ptr(a))
    assert rc == 0
    return Result(out[0], s[0], a[0])


def fp8_quantize(fmt, src, scale_inv):
    """(codes, amax): codes[i] = FP8(f32(src[i]) * scale_inv) (RNE, saturating),
    amax = max |src| over the unscaled bf16 source.  src: uint16 bf16 bits (any
    shape); fmt: E4M3 or E5M2; scale_inv: an f32 value."""
    src = np.ascontiguousarray(src, dtype=np.uint16)
    dst = np.zeros(src.shape, dtype=np.uint8)
    amax = ctypes.c_float(0.0)
    rc = lib().orc_fp8_quantize(fmt, _ptr(src), float(np.float32(scale_inv)), src.size,
                                _ptr(dst), ctypes.byref(amax))
    assert rc == 0
    return dst, amax.value


def fp8_transpose_quantize(fmt, src, scale_inv, rows, cols):
    """(codes [cols, rows], amax) for src [rows, cols] bf16 bits."""
    src = np.ascontiguousarray(src, dtype=np.uint16).reshape(rows, cols)
    dst = np.zeros((cols, rows), dtype=np.uint8)
    amax = ctypes.c_float(0.0)
    rc = lib().orc_fp8_transpose_quantize(fmt, _ptr(src), float(np.float32(scale_inv)), rows,
                                          cols, _ptr(dst), ctypes.byref(amax))
    assert rc == 0
    return dst, amax.value


def fp8_linear_forward(x, w, bias, sx, sw, sx_inv, sw_inv, m, k, n, rows=None, threads=None):
    """Y = RNE_bf16((q(x) q(w)^T) * sx * sw + b); x: [m,k], w: [n,k], bias: [n]
    or None (bf16 bits).  Returns a Result with .amax_x and .amax_w."""
    x, w = _c(x, np.uint16), _c(w, np.uint16)
    bias = None if bias is None else _c(bias, np.uint16)
    r, nr = _rows_arg(rows, m)
    out, s, a = _alloc(nr, n, BF16)
    g = np.zeros_like(s)
    ax, aw = ctypes.c_float(0.0), ctypes.c_float(0.0)
    f = lambda v: float(np.float32(v))
    rc = lib().orc_fp8_linear_forward(_ptr(x), _ptr(w), _ptr(bias), f(sx), f(sw), f(sx_inv),
                                      f(sw_inv), m, k, n, _ptr(r), nr, _ptr(out), _ptr(s),
                                      _ptr(a), _ptr(g), ctypes.byref(ax), ctypes.byref(aw),
                                      threads or default_threads())
    assert rc == 0
    res = Result(out, s, a)
    res.g = g
    res.amax_x, res.amax_w = ax.value, aw.value
    return res


def fp8_linear_backward(which, g, x, w, sg, sw, sx, sg_inv, sw_inv, sx_inv, m, k, n, rows=None,
                        threads=None):
    """which = "dx": dX = RNE_bf16((q(g) q(w)) * sg * sw), rows of M, [nrows, k];
    which = "dw": dW = RNE_bf16((q(g)^T q(x)) * sg * sx), rows of N, [nrows, k].
    g: [m,n], x: [m,k], w: [n,k] bf16 bits.  Returns a Result with .amax_g."""
    g, x, w = _c(g, np.uint16), _c(x, np.uint16), _c(w, np.uint16)
    code = {"dx": 1, "dw": 2}[which]
    r, nr = _rows_arg(rows, m if code == 1 else n)
    out, s, a = _alloc(nr, k, BF16)
    gg = np.zeros_like(s)
    ag = ctypes.c_float(0.0)
    f = lambda v: float(np.float32(v))
    rc = lib().orc_fp8_linear_backward(code, _ptr(g), _ptr(x), _ptr(w), f(sg), f(sw), f(sx),
                                       f(sg_inv), f(sw_inv), f(sx_inv), m, k, n, _ptr(r), nr,
                                       _ptr(out), _ptr(s), _ptr(a), _ptr(gg), ctypes.byref(ag),
                                       threads or default_threads())
    assert rc == 0
    res = Result(out, s, a)
    res.g = gg
    res.amax_g = ag.value
    return res


def grouped_fwd(dt, inp, weights, row_experts, m, k, n, e, rows=None, threads=None):
    """Y[m] = RNE_T(in[m] Wt[e(m)]^T), zero rows for ids outside [0,E)."""
    st = STORAGE[dt]
    inp, weights = _c(inp, st), _c(weights, st)
    re = _c(row_experts, np.uint32)
    r, nr = _rows_arg(rows, m)
    out, s, a = _alloc(nr, n, dt)
    rc = lib().orc_grouped_fwd(dt, _ptr(inp), _ptr(weights), _ptr(re), m, k, n, e, _ptr(r),
                               nr, _ptr(out), _ptr(s), _ptr(a), threads or default_threads())
    assert rc == 0
    return Result(out, s, a)


def grouped_dinput(dt, grad_out, weights, row_experts, m, k, n, e, rows=None, threads=None):
    """dIn[m] = RNE_T(dY[m] Wt[e(m)]), zero rows for ids outside [0,E)."""
    st = STORAGE[dt]
    g, weights = _c(grad_out, st), _c(weights, st)
    re = _c(row_experts, np.uint32)
    r, nr = _rows_arg(rows, m)
    out, s, a = _alloc(nr, k, dt)
    rc = lib().orc_grouped_dinput(dt, _ptr(g), _ptr(weights), _ptr(re), m, k, n, e, _ptr(r),
                                  nr, _ptr(out), _ptr(s), _ptr(a), threads or default_threads())
    assert rc == 0
    return Result(out, s, a)


def grouped_dweights(dt, inp, grad_out, row_experts, m, k, n, e, rows=None, threads=None):
    """dWt[e,n,:] (f32) for selected flattened rows e*N+n of [E*N, K]."""
    st = STORAGE[dt]
    inp, g = _c(inp, st), _c(grad_out, st)
    re = _c(row_experts, np.uint32)
    r, nr = _rows_arg(rows, e * n)
    out = np.zeros((nr, k), dtype=np.uint32)
    s = np.zeros((nr, k), dtype=np.float64)
    a = np.zeros((nr, k), dtype=np.float64)
    rc = lib().orc_grouped_dweights(dt, _ptr(inp), _ptr(g), _ptr(re), m, k, n, e, _ptr(r), nr,
                                    _ptr(out), _ptr(s), _ptr(a), threads or default_threads())
    assert rc == 0
    return Result(out, s, a)


# scalar codec helpers (used by the codec pins)
def decode_bf16(b): return lib().orc_decode_bf16(int(b))
def decode_f16(b): return lib().orc_decode_f16(int(b))
def decode_e4m3(b): return lib().orc_decode_e4m3(int(b))
def rne_bf16(x): return lib().orc_rne_bf16(float(x))
def rne_f16(x): return lib().orc_rne_f16(float(x))
def rne_f32(x): return lib().orc_rne_f32(float(x))
def rne_e4m3_sat(x): return lib().orc_rne_e4m3_sat(float(x))
def decode_e5m2(b): return lib().orc_decode_e5m2(int(b))
def rne_e5m2_sat(x): return lib().orc_rne_e5m2_sat(float(x))
