"""numpy front end of the CPU oracle (oracle.c, loaded with ctypes).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product library. Every function
takes and returns host numpy arrays; the arithmetic is all in oracle.c.

Float outputs are fp64. Functions that produce a float output also return
`tol`, the per-element sum of the magnitudes of the addends, which scales the
rounding error a correct fp32 kernel may make.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_LIB = None

WQ_SYM127 = 0
WQ_SYM127_5 = 1
W_Q8CSW = 0
W_Q4GSW = 1

_p = C.c_void_p
_i64 = C.c_int64
_i32 = C.c_int32
_f32 = C.c_float
_int = C.c_int

_SIGS = {
    "orc_quantize_weight_int8": [_p, _i64, _i64, _int, _p, _p, _p],
    "orc_quantize_weight_q4gsw": [_p, _i64, _i64, _i64, _p, _p, _p],
    "orc_quantize_act_per_tensor": [_p, _i64, _f32, _i32, _int, _f32, _i32, _p, _p],
    "orc_choose_qparams_rows": [_p, _i64, _i64, _p, _p, _p],
    "orc_gemm_i8_i64": [_p, _p, _i64, _i64, _i64, _p],
    "orc_linear_w8a16": [_p, _i64, _i64, _p, _p, _p, _i64, _p, _p],
    "orc_linear_w8a16_dequant_first": [_p, _i64, _i64, _p, _p, _p, _i64, _p],
    "orc_linear_q8ta_q8csw": [_p, _i64, _i64, _f32, _i32, _int, _f32, _i32, _p, _p, _p,
                              _i64, _p, _p, _p, _p, _p, _p],
    "orc_linear_q8ta_dequant_first": [_p, _p, _i64, _i64, _f32, _i32, _int, _f32, _i32,
                                      _p, _p, _p, _i64, _p],
    "orc_linear_dq8ca": [_p, _i64, _i64, _int, _p, _p, _i64, _p, _i64, _p, _p, _p, _p, _p],
    "orc_linear_dq8ca_dequant_first": [_p, _p, _p, _i64, _i64, _int, _p, _p, _i64, _p,
                                       _i64, _p],
    "orc_minmax_observe": [_p, _i64, _i64, _i64, _int, _f32, _i32, _p],
    "orc_gptq_damp": [_p, _i64, C.c_double, _p, _p],
    "orc_gptq_hinv": [_p, _i64, _p],
    "orc_gptq_quantize": [_p, _i64, _i64, _p, _p, _p, _i64, _p, _i64, _p, _p],
    "orc_minmax_qparams": [_p, _p, _p],
    "orc_set_threads": [_int],
}


def lib():
    """Load liboracle.so, compiling it first if it is missing or stale."""
    global _LIB
    if _LIB is None:
        path = _build.ensure_built()
        L = C.CDLL(path)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = C.c_int
        _LIB = L
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _shape(a, shape, what):
    """Raise unless array a has exactly this shape (the C side trusts the sizes)."""
    if a is not None and tuple(a.shape) != tuple(shape):
        raise ValueError(f"{what}: expected shape {tuple(shape)}, got {tuple(a.shape)}")


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments (rc={rc})")


def quantize_weight_int8(w, mode=WQ_SYM127):
    """w float32 [N, K] -> (q int8 [N, K], scale float32 [N], wsum int32 [N])."""
    w = _c(w, np.float32)
    N, K = w.shape
    q = np.empty((N, K), np.int8)
    s = np.empty(N, np.float32)
    ws = np.empty(N, np.int32)
    _check(lib().orc_quantize_weight_int8(_ptr(w), N, K, mode, _ptr(q), _ptr(s), _ptr(ws)),
           "quantize_weight_int8")
    return q, s, ws


def quantize_weight_q4gsw(w, group=32):
    """w float32 [N, K] -> (q4 uint8 [N, K/2], gs float32 [N, K/group], gsum int32 [N, K/group])."""
    w = _c(w, np.float32)
    N, K = w.shape
    if group <= 0 or K % group or group % 2:
        raise ValueError("K must be a multiple of an even group")
    q4 = np.zeros((N, K // 2), np.uint8)
    gs = np.empty((N, K // group), np.float32)
    gsum = np.empty((N, K // group), np.int32)
    _check(lib().orc_quantize_weight_q4gsw(_ptr(w), N, K, group, _ptr(q4), _ptr(gs), _ptr(gsum)),
           "quantize_weight_q4gsw")
    return q4, gs, gsum


def unpack_q4(q4, K):
    """Packed nibbles [N, K/2] -> int8 codes [N, K] (the layout of oracle.c)."""
    q4 = np.asarray(q4, np.uint8)
    lo = (q4 & 0xF).astype(np.int16)
    hi = (q4 >> 4).astype(np.int16)
    out = np.empty((q4.shape[0], K), np.int16)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    out[out >= 8] -= 16
    return out.astype(np.int8)


def quantize_act_per_tensor(x, s1, z1, two_pass=False, s2=None, z2=0):
    """x float32 (any shape) -> xq1 int8 (and xq2 int8 when two_pass)."""
    x = _c(x, np.float32)
    xq1 = np.empty(x.shape, np.int8)
    xq2 = np.empty(x.shape, np.int8) if two_pass else None
    _check(lib().orc_quantize_act_per_tensor(_ptr(x), x.size, np.float32(s1), int(z1),
                                             int(bool(two_pass)),
                                             np.float32(s2 if two_pass else 1.0), int(z2),
                                             _ptr(xq1), _ptr(xq2)),
           "quantize_act_per_tensor")
    return (xq1, xq2) if two_pass else xq1


def choose_qparams_rows(x, quantize=True):
    """x float32 [M, K] -> (scale float32 [M], zp int32 [M], xq int8 [M, K] or None)."""
    x = _c(x, np.float32)
    M, K = x.shape
    s = np.empty(M, np.float32)
    z = np.empty(M, np.int32)
    xq = np.empty((M, K), np.int8) if quantize else None
    _check(lib().orc_choose_qparams_rows(_ptr(x), M, K, _ptr(s), _ptr(z), _ptr(xq)),
           "choose_qparams_rows")
    return s, z, xq


def gemm_i8(a, b):
    """a int8 [M, K], b int8 [N, K] -> int64 [M, N] = a @ b.T exactly."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    M, K = a.shape
    N = b.shape[0]
    _shape(b, (N, K), "b")
    c = np.empty((M, N), np.int64)
    _check(lib().orc_gemm_i8_i64(_ptr(a), _ptr(b), M, N, K, _ptr(c)), "gemm_i8_i64")
    return c


def linear_w8a16(x_bf16, q, scale, bias_bf16=None):
    """x bf16 bits (uint16) [M, K], q int8 [N, K], scale f32 [N], bias bf16 bits [N]
    -> (y float64 [M, N], tol float64 [M, N])."""
    x = _c(x_bf16, np.uint16)
    q = _c(q, np.int8)
    scale = _c(scale, np.float32)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    M, K = x.shape
    N = q.shape[0]
    _shape(q, (N, K), "q")
    _shape(scale, (N,), "scale")
    _shape(b, (N,), "bias")
    y = np.empty((M, N), np.float64)
    tol = np.empty((M, N), np.float64)
    _check(lib().orc_linear_w8a16(_ptr(x), M, K, _ptr(q), _ptr(scale), _ptr(b), N, _ptr(y),
                                  _ptr(tol)), "linear_w8a16")
    return y, tol


def linear_w8a16_dequant_first(x_bf16, q, scale, bias_bf16=None):
    x = _c(x_bf16, np.uint16)
    q = _c(q, np.int8)
    scale = _c(scale, np.float32)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    M, K = x.shape
    N = q.shape[0]
    _shape(q, (N, K), "q")
    _shape(scale, (N,), "scale")
    _shape(b, (N,), "bias")
    y = np.empty((M, N), np.float64)
    _check(lib().orc_linear_w8a16_dequant_first(_ptr(x), M, K, _ptr(q), _ptr(scale), _ptr(b),
                                                N, _ptr(y)), "linear_w8a16_dequant_first")
    return y


def linear_q8ta_q8csw(x, s1, z1, q, wscale, bias=None, two_pass=False, s2=None, z2=0):
    """Static per-tensor W8A8 linear. Returns dict with y, tol (fp64 [M, N]),
    xq1, xq2 (int8 [M, K]), acc1, acc2 (int64 [M, N])."""
    x = _c(x, np.float32)
    q = _c(q, np.int8)
    wscale = _c(wscale, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    M, K = x.shape
    N = q.shape[0]
    _shape(q, (N, K), "q")
    _shape(wscale, (N,), "wscale")
    _shape(b, (N,), "bias")
    out = {
        "y": np.empty((M, N), np.float64),
        "tol": np.empty((M, N), np.float64),
        "xq1": np.empty((M, K), np.int8),
        "acc1": np.empty((M, N), np.int64),
        "xq2": np.empty((M, K), np.int8) if two_pass else None,
        "acc2": np.empty((M, N), np.int64) if two_pass else None,
    }
    _check(lib().orc_linear_q8ta_q8csw(
        _ptr(x), M, K, np.float32(s1), int(z1), int(bool(two_pass)),
        np.float32(s2 if two_pass else 1.0), int(z2), _ptr(q), _ptr(wscale), _ptr(b), N,
        _ptr(out["y"]), _ptr(out["xq1"]), _ptr(out["xq2"]), _ptr(out["acc1"]),
        _ptr(out["acc2"]), _ptr(out["tol"])), "linear_q8ta_q8csw")
    return out


def linear_q8ta_dequant_first(xq1, xq2, s1, z1, q, wscale, bias=None, two_pass=False,
                              s2=None, z2=0):
    xq1 = _c(xq1, np.int8)
    xq2 = _c(xq2, np.int8) if two_pass else None
    q = _c(q, np.int8)
    wscale = _c(wscale, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    M, K = xq1.shape
    N = q.shape[0]
    _shape(xq2, (M, K), "xq2")
    _shape(q, (N, K), "q")
    _shape(wscale, (N,), "wscale")
    _shape(b, (N,), "bias")
    y = np.empty((M, N), np.float64)
    _check(lib().orc_linear_q8ta_dequant_first(
        _ptr(xq1), _ptr(xq2), M, K, np.float32(s1), int(z1), int(bool(two_pass)),
        np.float32(s2 if two_pass else 1.0), int(z2), _ptr(q), _ptr(wscale), _ptr(b), N,
        _ptr(y)), "linear_q8ta_dequant_first")
    return y


def _wq_shapes(wq, wscale, b, N, K, wfmt, group):
    if wfmt == W_Q8CSW:
        _shape(wq, (N, K), "wq")
        _shape(wscale, (N,), "wscale")
    else:
        if group <= 0 or K % group or group % 2:
            raise ValueError("K must be a multiple of an even group")
        _shape(wq, (N, K // 2), "wq")
        _shape(wscale, (N, K // group), "wscale")
    _shape(b, (N,), "bias")


def linear_dq8ca(x, wq, wscale, wfmt=W_Q8CSW, group=0, bias=None):
    """Dynamic per-row W8A8 linear. wq: int8 [N, K] (W_Q8CSW) or packed q4 uint8
    [N, K/2] (W_Q4GSW). Returns dict with y, tol (fp64 [M, N]), x_scale, x_zp, xq."""
    x = _c(x, np.float32)
    M, K = x.shape
    if wfmt == W_Q8CSW:
        wq = _c(wq, np.int8)
    else:
        wq = _c(wq, np.uint8)
    N = wq.shape[0]
    wscale = _c(wscale, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    _wq_shapes(wq, wscale, b, N, K, wfmt, group)
    out = {
        "y": np.empty((M, N), np.float64),
        "tol": np.empty((M, N), np.float64),
        "x_scale": np.empty(M, np.float32),
        "x_zp": np.empty(M, np.int32),
        "xq": np.empty((M, K), np.int8),
    }
    _check(lib().orc_linear_dq8ca(_ptr(x), M, K, int(wfmt), _ptr(wq), _ptr(wscale), int(group),
                                  _ptr(b), N, _ptr(out["y"]), _ptr(out["x_scale"]),
                                  _ptr(out["x_zp"]), _ptr(out["xq"]), _ptr(out["tol"])),
           "linear_dq8ca")
    return out


def linear_dq8ca_dequant_first(xq, xs, xz, wq, wscale, K, wfmt=W_Q8CSW, group=0, bias=None):
    xq = _c(xq, np.int8)
    xs = _c(xs, np.float32)
    xz = _c(xz, np.int32)
    M = xq.shape[0]
    wq = _c(wq, np.int8 if wfmt == W_Q8CSW else np.uint8)
    N = wq.shape[0]
    wscale = _c(wscale, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    _shape(xq, (M, K), "xq")
    _shape(xs, (M,), "xs")
    _shape(xz, (M,), "xz")
    _wq_shapes(wq, wscale, b, N, K, wfmt, group)
    y = np.empty((M, N), np.float64)
    _check(lib().orc_linear_dq8ca_dequant_first(_ptr(xq), _ptr(xs), _ptr(xz), M, K, int(wfmt),
                                                _ptr(wq), _ptr(wscale), int(group), _ptr(b), N,
                                                _ptr(y)), "linear_dq8ca_dequant_first")
    return y


def minmax_empty():
    """The running (min, max) of an observer that has seen nothing."""
    return np.array([np.inf, -np.inf], np.float32)


def minmax_observe(x, state, seq=0, residual=False, s1=0.0, z1=0):
    """Fold x float32 [rows, cols] (or its two-pass residual against (s1, z1))
    into the running (min, max) float32 [2]; returns the new state. seq > 0
    skips the row at position 0 of every seq rows."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    st = np.array(state, np.float32).copy()
    _check(lib().orc_minmax_observe(_ptr(x), rows, cols, seq, int(bool(residual)), s1, z1,
                                    _ptr(st)), "minmax_observe")
    return st


def minmax_qparams(state):
    """(scale, zero point) of a running (min, max) by the per-tensor affine rule."""
    st = np.array(state, np.float32)
    s = np.empty(1, np.float32)
    z = np.empty(1, np.int32)
    _check(lib().orc_minmax_qparams(_ptr(st), _ptr(s), _ptr(z)), "minmax_qparams")
    return float(s[0]), int(z[0])


def keep_outliers(amax, seam, nseams, factor):
    """flashrt schemes, Fp8Static.decide with keep_outliers: the seams whose
    largest point statistic exceeds factor times the median of all positive
    statistics. amax: per point, NaN for a point without a statistic; seam:
    the seam index of each point. Returns a list of nseams booleans. Written
    with Python floats and statistics.median, as the page computes it."""
    import math
    import statistics
    keep = [False] * nseams
    if not factor:
        return keep
    values = [float(v) for v in amax if not math.isnan(v) and v > 0]
    if not values:
        return keep
    median = statistics.median(values)
    worst = [None] * nseams
    for v, sidx in zip(amax, seam):
        if math.isnan(v):
            continue
        if worst[sidx] is None or float(v) > worst[sidx]:
            worst[sidx] = float(v)
    for i in range(nseams):
        keep[i] = worst[i] is not None and worst[i] > float(factor) * median
    return keep


def gptq_damped(H, damp=0.01):
    """(damped Hessian float64 [K, K], dead columns bool [K]) of gptq_int8."""
    H = _c(H, np.float64)
    K = H.shape[0]
    _shape(H, (K, K), "H")
    Hd = np.empty_like(H)
    dead = np.empty(K, np.uint8)
    _check(lib().orc_gptq_damp(_ptr(H), K, damp, _ptr(Hd), _ptr(dead)), "gptq_damp")
    return Hd, dead.astype(bool)


def gptq_hinv(Hd):
    """Upper factor hinv of Hd^-1 (hinv^T hinv = Hd^-1), float64 [K, K]."""
    Hd = _c(Hd, np.float64)
    K = Hd.shape[0]
    _shape(Hd, (K, K), "Hd")
    hinv = np.empty_like(Hd)
    _check(lib().orc_gptq_hinv(_ptr(Hd), K, _ptr(hinv)), "gptq_hinv")
    return hinv


def gptq_int8(w, H, damp=0.01, block=128, rows=None, hinv=None):
    """GPTQ int8 codes: w float32 [N, K], H float64 [K, K] -> (q int8, scale
    float32 [N], wsum int32). rows: compute only these rows (q, wsum then hold
    them in that order; scale stays [N]). hinv: reuse a factor from gptq_hinv
    of the same damped Hessian."""
    w = _c(w, np.float32)
    N, K = w.shape
    _shape(np.asarray(H), (K, K), "H")
    _, scale, _ = quantize_weight_int8(w, WQ_SYM127_5)
    Hd, dead = gptq_damped(H, damp)
    if hinv is None:
        hinv = gptq_hinv(Hd)
    hinv = _c(hinv, np.float64)
    _shape(hinv, (K, K), "hinv")
    dead8 = dead.astype(np.uint8)
    rl = None if rows is None else np.ascontiguousarray(np.asarray(rows, np.int64))
    if rl is not None and rl.size and (rl.min() < 0 or rl.max() >= N):
        raise ValueError("rows out of range")
    R = N if rl is None else rl.size
    q = np.empty((R, K), np.int8)
    wsum = np.empty(R, np.int32)
    _check(lib().orc_gptq_quantize(_ptr(w), N, K, _ptr(dead8), _ptr(hinv), _ptr(scale), block,
                                   _ptr(rl), 0 if rl is None else rl.size, _ptr(q), _ptr(wsum)),
           "gptq_quantize")
    return q, scale, wsum


_THREADS = None


def set_threads(n):
    """Run the oracle's OpenMP loops on n threads (None: back to the default)."""
    global _THREADS
    _check(lib().orc_set_threads(int(n) if n else _default_threads()), "set_threads")
    _THREADS = int(n) if n else None


def _default_threads():
    v = os.environ.get("OMP_NUM_THREADS")
    return int(v) if v else os.cpu_count()


def threads():
    """OpenMP threads the oracle uses (set_threads, else OMP_NUM_THREADS, else all cores)."""
    return _THREADS or _default_threads()
