"""Python binding of libaql.so, the MI355X (gfx950) per-output-channel INT8
quantized linear.

Argument marshalling only: every function checks dtypes, shapes and devices
of torch tensors, allocates the outputs it was not given (torch.empty on the
input's device), and calls the C entry point of the same name on the current
torch stream. All arithmetic runs in the HIP kernels of libaql.so; there is no
CPU or PyTorch fallback. A non-zero status raises AqlError with the library's
message.

The library is built in-tree (build.py, or __graft_entry__.build()); importing
this package without it raises ImportError.
"""
import ctypes as C
import os

import torch  # loads the HIP runtime that libaql.so then shares (same soname)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libaql.so")

AQL_OK = 0
AQL_ERR_NULL = -1
AQL_ERR_SHAPE = -2
AQL_ERR_ALIGN = -3
AQL_ERR_PARAM = -4
AQL_ERR_WORKSPACE = -5
AQL_ERR_DEVICE = -6
AQL_ERR_HIP = -7

AQL_F32 = 0
AQL_BF16 = 1
AQL_WQ_SYM127 = 0
AQL_WQ_SYM127_5 = 1
AQL_W_Q8CSW = 0
AQL_W_Q4GSW = 1
AQL_OP_Q8TA_Q8CSW = 1
AQL_OP_DQ8CA = 2
AQL_OP_GPTQ_INT8 = 3
AQL_OP_W8A16 = 4
AQL_MAX_K_INT8 = 65536
AQL_NOALLOC_SCRATCH_BYTES = 8 << 20

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run python -c 'import __graft_entry__ as g; "
                      f"g.build()' (or python activation_quantized_linear_amd/build.py)")

_lib = C.CDLL(LIB_PATH)

_p = C.c_void_p
_i64 = C.c_int64
_i32 = C.c_int32
_int = C.c_int
_f32 = C.c_float
_sz = C.c_size_t

_SIGS = {
    "aql_version": ([], C.c_int),
    "aql_last_error": ([], C.c_char_p),
    "aql_workspace_bytes": ([_int, _i64, _i64, _i64], _sz),
    "aql_quantize_weight_int8": ([_p, _int, _i64, _i64, _int, _p, _p, _p, _p], _int),
    "aql_quantize_weight_q4gsw": ([_p, _i64, _i64, _int, _p, _p, _p, _p], _int),
    "aql_choose_qparams_rows": ([_p, _i64, _i64, _p, _p, _p, _p], _int),
    "aql_quantize_act_per_tensor": ([_p, _i64, _i64, _f32, _i32, _int, _f32, _i32, _p, _p, _p],
                                    _int),
    "aql_linear_w8a16": ([_p, _i64, _i64, _p, _p, _p, _i64, _p, _p, _sz, _p], _int),
    "aql_linear_q8ta_q8csw": ([_p, _i64, _i64, _f32, _i32, _int, _f32, _i32, _p, _p, _p, _p,
                               _i64, _p, _p, _sz, _p], _int),
    "aql_linear_q8ta_q8csw_noalloc": ([_p, _i64, _i64, _f32, _i32, _int, _f32, _i32, _p, _p,
                                       _p, _p, _i64, _p, _p], _int),
    "aql_linear_dq8ca": ([_p, _i64, _i64, _int, _p, _p, _p, _int, _p, _i64, _p, _p, _p, _p, _sz,
                          _p], _int),
    "aql_gemm_i8_i32": ([_p, _p, _p, _i64, _i64, _i64, _p], _int),
    "aql_measure_read": ([_p, _i64, _p, _p], _int),
    "aql_measure_mfma_i8": ([_i64, _p, _p], _int),
    "aql_minmax_reset": ([_p, _p], _int),
    "aql_minmax_observe": ([_p, _i64, _i64, _i64, _int, _f32, _i32, _p, _p], _int),
    "aql_minmax_qparams": ([_p, _p, _p, _p], _int),
    "aql_keep_outliers": ([_p, _p, _i64, _i32, C.c_double, _p], _int),
    "aql_gptq_int8": ([_p, _i64, _i64, _p, C.c_double, _i64, _p, _p, _p, _p, _p, _p, _sz, _p],
                      _int),
    "aql_w8a16_group_table_bytes": ([_int], _sz),
    "aql_w8a16_group_plan": ([_p, _int, _p, _sz], _int),
    "aql_linear_w8a16_grouped": ([_p, _p, _p], _int),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)


class AqlError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def _check(fn, rc):
    if rc != AQL_OK:
        raise AqlError(fn, rc, aql_last_error())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(dev):
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _out(t, name, shape, dtype, dev):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    _need(t, name, dtype, device=dev)
    _shape(t, name, shape)
    return t


# ----------------------------------------------------------------- helpers


def aql_version():
    return _lib.aql_version()


def aql_last_error():
    return _lib.aql_last_error().decode()


def aql_workspace_bytes(op, M, N, K):
    return _lib.aql_workspace_bytes(op, M, N, K)


# --------------------------------------------------------------- quantizers


def aql_quantize_weight_int8(w, mode=AQL_WQ_SYM127, q=None, scale=None, wsum=None):
    """w float32 or bfloat16 [N, K] -> (q int8 [N, K], scale float32 [N], wsum int32 [N])."""
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("w must be float32 or bfloat16")
    _need(w, "w", w.dtype, 2)
    N, K = w.shape
    dev = w.device
    q = _out(q, "q", (N, K), torch.int8, dev)
    scale = _out(scale, "scale", (N,), torch.float32, dev)
    wsum = _out(wsum, "wsum", (N,), torch.int32, dev)
    dt = AQL_F32 if w.dtype == torch.float32 else AQL_BF16
    _check("aql_quantize_weight_int8",
           _lib.aql_quantize_weight_int8(_ptr(w), dt, N, K, mode, _ptr(q), _ptr(scale),
                                         _ptr(wsum), _stream(dev)))
    return q, scale, wsum


def aql_quantize_weight_q4gsw(w, group=32, q4=None, gscale=None, gsum=None):
    """w float32 [N, K] -> (q4 uint8 [N, K/2], gscale float32 [N, K/group], gsum int32 [N, K/group])."""
    _need(w, "w", torch.float32, 2)
    N, K = w.shape
    if group <= 0 or K % group:
        raise ValueError("K must be a multiple of group")
    dev = w.device
    q4 = _out(q4, "q4", (N, K // 2), torch.uint8, dev)
    gscale = _out(gscale, "gscale", (N, K // group), torch.float32, dev)
    gsum = _out(gsum, "gsum", (N, K // group), torch.int32, dev)
    _check("aql_quantize_weight_q4gsw",
           _lib.aql_quantize_weight_q4gsw(_ptr(w), N, K, group, _ptr(q4), _ptr(gscale),
                                          _ptr(gsum), _stream(dev)))
    return q4, gscale, gsum


def aql_choose_qparams_rows(x, quantize=True, scale=None, zp=None, xq=None):
    """x float32 [M, K] -> (scale float32 [M], zp int32 [M], xq int8 [M, K] or None)."""
    _need(x, "x", torch.float32, 2)
    M, K = x.shape
    dev = x.device
    scale = _out(scale, "scale", (M,), torch.float32, dev)
    zp = _out(zp, "zp", (M,), torch.int32, dev)
    if quantize:
        xq = _out(xq, "xq", (M, K), torch.int8, dev)
    _check("aql_choose_qparams_rows",
           _lib.aql_choose_qparams_rows(_ptr(x), M, K, _ptr(scale), _ptr(zp),
                                        _ptr(xq) if quantize else None, _stream(dev)))
    return scale, zp, (xq if quantize else None)


def aql_quantize_act_per_tensor(x, s1, z1, two_pass=False, s2=1.0, z2=0, xq1=None, xq2=None):
    """x float32 [M, K] -> xq1 int8 [M, K] (and xq2 with two_pass)."""
    _need(x, "x", torch.float32, 2)
    M, K = x.shape
    dev = x.device
    xq1 = _out(xq1, "xq1", (M, K), torch.int8, dev)
    if two_pass:
        xq2 = _out(xq2, "xq2", (M, K), torch.int8, dev)
    _check("aql_quantize_act_per_tensor",
           _lib.aql_quantize_act_per_tensor(_ptr(x), M, K, float(s1), int(z1), int(bool(two_pass)),
                                            float(s2), int(z2), _ptr(xq1),
                                            _ptr(xq2) if two_pass else None, _stream(dev)))
    return (xq1, xq2) if two_pass else xq1


# -------------------------------------------------------------------- linears


def aql_linear_w8a16(x, q, scale, bias=None, y=None, workspace=None):
    """x bfloat16 [M, K], q int8 [N, K], scale float32 [N], bias bfloat16 [N] -> y bfloat16 [M, N].
    workspace: uint8 device tensor; allocated here when the shape can use one
    (aql_workspace_bytes(AQL_OP_W8A16, ...) > 0) and none is given."""
    _need(x, "x", torch.bfloat16, 2)
    dev = x.device
    _need(q, "q", torch.int8, 2, dev)
    M, K = x.shape
    N = q.shape[0]
    _shape(q, "q", (N, K))
    _need(scale, "scale", torch.float32, 1, dev)
    _shape(scale, "scale", (N,))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, 1, dev)
        _shape(bias, "bias", (N,))
    y = _out(y, "y", (M, N), torch.bfloat16, dev)
    nbytes = aql_workspace_bytes(AQL_OP_W8A16, M, N, K)
    ws = None
    if workspace is not None or nbytes > 0:
        ws = _workspace(workspace, nbytes, dev)
    _check("aql_linear_w8a16",
           _lib.aql_linear_w8a16(_ptr(x), M, K, _ptr(q), _ptr(scale), _ptr(bias), N, _ptr(y),
                                 _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)))
    return y


def _workspace(ws, nbytes, dev):
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _need(ws, "workspace", torch.uint8, device=dev)
    return ws


def aql_linear_q8ta_q8csw(x, s1, z1, q, wsum, wscale, bias=None, two_pass=False, s2=1.0, z2=0,
                          y=None, workspace=None):
    """Static per-tensor W8A8 linear (optional second pass). x float32 [M, K] -> y float32 [M, N]."""
    _need(x, "x", torch.float32, 2)
    dev = x.device
    M, K = x.shape
    _need(q, "q", torch.int8, 2, dev)
    N = q.shape[0]
    _shape(q, "q", (N, K))
    _need(wsum, "wsum", torch.int32, 1, dev)
    _shape(wsum, "wsum", (N,))
    _need(wscale, "wscale", torch.float32, 1, dev)
    _shape(wscale, "wscale", (N,))
    if bias is not None:
        _need(bias, "bias", torch.float32, 1, dev)
        _shape(bias, "bias", (N,))
    y = _out(y, "y", (M, N), torch.float32, dev)
    nbytes = aql_workspace_bytes(AQL_OP_Q8TA_Q8CSW, M, N, K)
    ws = _workspace(workspace, nbytes, dev)
    _check("aql_linear_q8ta_q8csw",
           _lib.aql_linear_q8ta_q8csw(_ptr(x), M, K, float(s1), int(z1), int(bool(two_pass)),
                                      float(s2), int(z2), _ptr(q), _ptr(wsum), _ptr(wscale),
                                      _ptr(bias), N, _ptr(y), _ptr(ws), ws.numel(),
                                      _stream(dev)))
    return y


def aql_linear_q8ta_q8csw_noalloc(x, s1, z1, q, wsum, wscale, bias=None, two_pass=False, s2=1.0,
                                  z2=0, y=None):
    """aql_linear_q8ta_q8csw on the library's fixed per-GPU scratch (no workspace
    argument; the C entry allocates nothing). Pass y to allocate nothing here
    either. Calls that overlap on one GPU race on the shared scratch."""
    _need(x, "x", torch.float32, 2)
    dev = x.device
    M, K = x.shape
    _need(q, "q", torch.int8, 2, dev)
    N = q.shape[0]
    _shape(q, "q", (N, K))
    _need(wsum, "wsum", torch.int32, 1, dev)
    _shape(wsum, "wsum", (N,))
    _need(wscale, "wscale", torch.float32, 1, dev)
    _shape(wscale, "wscale", (N,))
    if bias is not None:
        _need(bias, "bias", torch.float32, 1, dev)
        _shape(bias, "bias", (N,))
    y = _out(y, "y", (M, N), torch.float32, dev)
    _check("aql_linear_q8ta_q8csw_noalloc",
           _lib.aql_linear_q8ta_q8csw_noalloc(_ptr(x), M, K, float(s1), int(z1),
                                              int(bool(two_pass)), float(s2), int(z2), _ptr(q),
                                              _ptr(wsum), _ptr(wscale), _ptr(bias), N, _ptr(y),
                                              _stream(dev)))
    return y


def aql_linear_dq8ca(x, wq, wscale, wsum, wfmt=AQL_W_Q8CSW, group=0, bias=None, y=None,
                     x_scale_out=None, x_zp_out=None, workspace=None):
    """Dynamic per-row W8A8 linear. x float32 [M, K]; wq int8 [N, K] (Q8CSW) or uint8
    [N, K/2] (Q4GSW) -> y float32 [M, N]. x_scale_out / x_zp_out, when given, receive
    the per-row qparams."""
    _need(x, "x", torch.float32, 2)
    dev = x.device
    M, K = x.shape
    if wfmt == AQL_W_Q8CSW:
        _need(wq, "wq", torch.int8, 2, dev)
        N = wq.shape[0]
        _shape(wq, "wq", (N, K))
        sshape = (N,)
    else:
        _need(wq, "wq", torch.uint8, 2, dev)
        N = wq.shape[0]
        _shape(wq, "wq", (N, K // 2))
        if group <= 0 or K % group:
            raise ValueError("K must be a multiple of group")
        sshape = (N, K // group)
    _need(wscale, "wscale", torch.float32, len(sshape), dev)
    _shape(wscale, "wscale", sshape)
    _need(wsum, "wsum", torch.int32, len(sshape), dev)
    _shape(wsum, "wsum", sshape)
    if bias is not None:
        _need(bias, "bias", torch.float32, 1, dev)
        _shape(bias, "bias", (N,))
    y = _out(y, "y", (M, N), torch.float32, dev)
    if x_scale_out is not None:
        x_scale_out = _out(x_scale_out, "x_scale_out", (M,), torch.float32, dev)
    if x_zp_out is not None:
        x_zp_out = _out(x_zp_out, "x_zp_out", (M,), torch.int32, dev)
    nbytes = aql_workspace_bytes(AQL_OP_DQ8CA, M, N, K)
    ws = _workspace(workspace, nbytes, dev)
    _check("aql_linear_dq8ca",
           _lib.aql_linear_dq8ca(_ptr(x), M, K, int(wfmt), _ptr(wq), _ptr(wscale), _ptr(wsum),
                                 int(group), _ptr(bias), N, _ptr(y), _ptr(x_scale_out),
                                 _ptr(x_zp_out), _ptr(ws), ws.numel(), _stream(dev)))
    return y


# ------------------------------------------------------- static calibration


def aql_minmax_state(device="cuda"):
    """A new, empty running (min, max): device float32 [2] = (+inf, -inf)."""
    st = torch.empty(2, dtype=torch.float32, device=device)
    aql_minmax_reset(st)
    return st


def aql_minmax_reset(state):
    _need(state, "state", torch.float32, 1)
    _shape(state, "state", (2,))
    _check("aql_minmax_reset", _lib.aql_minmax_reset(_ptr(state), _stream(state.device)))
    return state


def aql_minmax_observe(x, state, seq=0, residual=None):
    """Fold x float32 [rows, cols] into the running (min, max) `state`. seq > 0
    leaves out the row at position 0 of every seq rows; residual=(s1, z1)
    observes x - fake_quant(x, s1, z1) instead (the two-pass recipe's second
    calibration run)."""
    _need(x, "x", torch.float32, 2)
    _need(state, "state", torch.float32, 1, x.device)
    _shape(state, "state", (2,))
    rows, cols = x.shape
    s1, z1 = residual if residual is not None else (0.0, 0)
    _check("aql_minmax_observe",
           _lib.aql_minmax_observe(_ptr(x), rows, cols, seq, int(residual is not None), s1, z1,
                                   _ptr(state), _stream(x.device)))
    return state


def aql_minmax_qparams(state, scale=None, zp=None):
    """-> (scale float32 [1], zp int32 [1]) device tensors by the per-tensor
    affine observer rule."""
    _need(state, "state", torch.float32, 1)
    dev = state.device
    scale = _out(scale, "scale", (1,), torch.float32, dev)
    zp = _out(zp, "zp", (1,), torch.int32, dev)
    _check("aql_minmax_qparams",
           _lib.aql_minmax_qparams(_ptr(state), _ptr(scale), _ptr(zp), _stream(dev)))
    return scale, zp


def aql_keep_outliers(amax, seam, nseams, factor):
    """Host decision, no GPU: list of nseams booleans (see aql.h)."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(amax, dtype=np.float32))
    sidx = np.ascontiguousarray(np.asarray(seam, dtype=np.int32))
    if a.shape != sidx.shape or a.ndim != 1:
        raise ValueError("amax and seam must be 1-D of the same length")
    keep = np.zeros(max(nseams, 0), np.int32)
    _check("aql_keep_outliers",
           _lib.aql_keep_outliers(a.ctypes.data_as(_p), sidx.ctypes.data_as(_p), a.size, nseams,
                                  float(factor), keep.ctypes.data_as(_p)))
    return [bool(v) for v in keep]


# ---------------------------------------------------------------- GPTQ int8


def aql_gptq_int8(w, H, damp=0.01, block=128, q=None, scale=None, wsum=None, hinv=False,
                  info=None, workspace=None):
    """GPTQ int8 codes on the device. w float32 [N, K], H float64 [K, K] ->
    (q int8 [N, K], scale float32 [N], wsum int32 [N], hinv float64 [K, K] or
    None, info int32 [1]). hinv=True also returns the upper factor of the
    damped Hessian's inverse. info (device) is 0 on success, else the failed
    pivot (see aql.h); it is not read back here, so the call stays
    asynchronous."""
    _need(w, "w", torch.float32, 2)
    dev = w.device
    N, K = w.shape
    _need(H, "H", torch.float64, 2, dev)
    _shape(H, "H", (K, K))
    q = _out(q, "q", (N, K), torch.int8, dev)
    scale = _out(scale, "scale", (N,), torch.float32, dev)
    wsum = _out(wsum, "wsum", (N,), torch.int32, dev)
    hv = torch.empty((K, K), dtype=torch.float64, device=dev) if hinv else None
    info = _out(info, "info", (1,), torch.int32, dev)
    nbytes = aql_workspace_bytes(AQL_OP_GPTQ_INT8, block, N, K)
    ws = _workspace(workspace, nbytes, dev)
    _check("aql_gptq_int8",
           _lib.aql_gptq_int8(_ptr(w), N, K, _ptr(H), float(damp), int(block), _ptr(q),
                              _ptr(scale), _ptr(wsum), _ptr(hv), _ptr(info), _ptr(ws),
                              ws.numel(), _stream(dev)))
    return q, scale, wsum, hv, info


def aql_measure_read(buf, sink):
    """Measurement helper: one launch that reads all of `buf` (a contiguous
    device tensor whose byte size is a multiple of 1024) as a read-only HBM
    stream. sink: a device tensor of at least 4 bytes."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    _check("aql_measure_read", _lib.aql_measure_read(_ptr(buf), nbytes, _ptr(sink),
                                                     _stream(buf.device)))


def aql_measure_mfma_i8(iters, sink):
    """Measurement helper: 2048 waves x 16 * iters int8 16x16x64 MFMAs
    (2048 * 32768 * 16 * iters integer ops)."""
    _check("aql_measure_mfma_i8", _lib.aql_measure_mfma_i8(int(iters), _ptr(sink),
                                                           _stream(sink.device)))


def aql_gemm_i8_i32(a, b, c=None):
    """a int8 [M, K], b int8 [N, K] -> c int32 [M, N] = a @ b.T exactly."""
    _need(a, "a", torch.int8, 2)
    dev = a.device
    _need(b, "b", torch.int8, 2, dev)
    M, K = a.shape
    N = b.shape[0]
    _shape(b, "b", (N, K))
    c = _out(c, "c", (M, N), torch.int32, dev)
    _check("aql_gemm_i8_i32",
           _lib.aql_gemm_i8_i32(_ptr(a), _ptr(b), _ptr(c), M, N, K, _stream(dev)))
    return c


# ------------------------------------------------------------ grouped W8A16


class _Problem(C.Structure):
    _fields_ = [("x", _p), ("q", _p), ("scale", _p), ("bias", _p), ("y", _p),
                ("M", _i64), ("N", _i64), ("K", _i64)]


def aql_w8a16_group_table_bytes(count):
    return _lib.aql_w8a16_group_table_bytes(count)


def aql_w8a16_group_plan(problems):
    """problems: sequence of (x, q, scale, bias or None, y) device tensors, each as
    aql_linear_w8a16 takes them (y preallocated). Returns (host_table, dev_table):
    the plan as a host uint8 tensor and its copy on the problems' device. Keep the
    problems' tensors alive while the tables are in use."""
    arr = (_Problem * len(problems))()
    dev = None
    for i, (x, q, scale, bias, y) in enumerate(problems):
        _need(x, f"problems[{i}].x", torch.bfloat16, 2)
        dev = x.device
        _need(q, f"problems[{i}].q", torch.int8, 2, dev)
        M, K = x.shape
        N = q.shape[0]
        _shape(q, f"problems[{i}].q", (N, K))
        _need(scale, f"problems[{i}].scale", torch.float32, 1, dev)
        _shape(scale, f"problems[{i}].scale", (N,))
        if bias is not None:
            _need(bias, f"problems[{i}].bias", torch.bfloat16, 1, dev)
            _shape(bias, f"problems[{i}].bias", (N,))
        _need(y, f"problems[{i}].y", torch.bfloat16, 2, dev)
        _shape(y, f"problems[{i}].y", (M, N))
        arr[i] = _Problem(x.data_ptr(), q.data_ptr(), scale.data_ptr(),
                          0 if bias is None else bias.data_ptr(), y.data_ptr(), M, N, K)
    nbytes = aql_w8a16_group_table_bytes(len(problems))
    host = torch.empty(max(nbytes, 16), dtype=torch.uint8)
    _check("aql_w8a16_group_plan",
           _lib.aql_w8a16_group_plan(C.cast(arr, _p), len(problems), _ptr(host), host.numel()))
    return host, host.to(dev)


def aql_linear_w8a16_grouped(host_table, dev_table):
    """Launch a planned group on the current stream of dev_table's device."""
    if host_table.is_cuda or host_table.dtype != torch.uint8:
        raise ValueError("host_table must be the host uint8 table from aql_w8a16_group_plan")
    _need(dev_table, "dev_table", torch.uint8)
    _check("aql_linear_w8a16_grouped",
           _lib.aql_linear_w8a16_grouped(_ptr(host_table), _ptr(dev_table),
                                         _stream(dev_table.device)))
