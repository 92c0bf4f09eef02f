"""The C ABI without a GPU: the library loads, exports every function that
include/aql.h declares, and rejects every invalid argument with the documented
status before making any HIP call (fake device addresses are never touched:
validation fails first, or the problem is empty)."""
import ctypes as C
import os
import re

import pytest

import activation_quantized_linear_amd as aql

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aql.h")

A = C.c_void_p(0x10000)      # a fake, 16-byte aligned address (never dereferenced)
B = C.c_void_p(0x20000)
Y = C.c_void_p(0x30000)
MIS = C.c_void_p(0x10004)    # misaligned
NUL = None
L = aql._lib


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aql_\w+)\s*\(", text)))


def test_header_and_exports_agree():
    names = declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(aql.EXPORTED)


def test_version_and_error_text():
    assert aql.aql_version() >= 100
    assert isinstance(aql.aql_last_error(), str)


def test_workspace_bytes():
    assert aql.aql_workspace_bytes(aql.AQL_OP_Q8TA_Q8CSW, 512, 4096, 4096) == 2 * 512 * 4096
    assert aql.aql_workspace_bytes(aql.AQL_OP_DQ8CA, 4, 11008, 4096) >= 4 * 4096 + 8 * 4
    assert aql.aql_workspace_bytes(99, 1, 1, 16) == 0
    assert aql.aql_workspace_bytes(aql.AQL_OP_DQ8CA, -1, 1, 16) == 0
    g = aql.aql_workspace_bytes(aql.AQL_OP_GPTQ_INT8, 128, 4096, 4096)
    assert g >= 4 * 8 * 4096 * 4096 + 8 * 4096 * 4096 + 8 * 4096 * 128 + 4096
    assert aql.aql_workspace_bytes(aql.AQL_OP_GPTQ_INT8, 0, 16, 16) == 0       # block 0
    assert aql.aql_workspace_bytes(aql.AQL_OP_GPTQ_INT8, 257, 16, 16) == 0     # block > 256


def qw(*a):
    return L.aql_quantize_weight_int8(*a, None)


def test_quantize_weight_int8_validation():
    assert qw(NUL, 0, 4, 16, 0, B, Y, None) == aql.AQL_ERR_NULL
    assert qw(A, 0, 4, 16, 0, NUL, Y, None) == aql.AQL_ERR_NULL
    assert qw(A, 2, 4, 16, 0, B, Y, None) == aql.AQL_ERR_PARAM
    assert qw(A, 0, 4, 16, 2, B, Y, None) == aql.AQL_ERR_PARAM
    assert qw(A, 0, 4, 0, 0, B, Y, None) == aql.AQL_ERR_SHAPE
    assert qw(A, 0, 4, 18, 0, B, Y, None) == aql.AQL_ERR_SHAPE
    assert qw(A, 0, -1, 16, 0, B, Y, None) == aql.AQL_ERR_SHAPE
    assert qw(MIS, 0, 4, 16, 0, B, Y, None) == aql.AQL_ERR_ALIGN
    assert qw(A, 0, 0, 16, 0, B, Y, None) == aql.AQL_OK  # empty: nothing launched
    assert "K" in aql.aql_last_error() or aql.aql_last_error() == ""


def test_q4gsw_validation():
    f = L.aql_quantize_weight_q4gsw
    assert f(NUL, 4, 64, 32, B, Y, None, None) == aql.AQL_ERR_NULL
    assert f(A, 4, 64, 16, B, Y, None, None) == aql.AQL_ERR_PARAM
    assert f(A, 4, 48, 32, B, Y, None, None) == aql.AQL_ERR_SHAPE
    assert f(A, 4, 64, 32, MIS, Y, None, None) == aql.AQL_ERR_ALIGN
    assert f(A, 0, 64, 32, B, Y, None, None) == aql.AQL_OK


def test_choose_qparams_validation():
    f = L.aql_choose_qparams_rows
    assert f(NUL, 4, 64, B, Y, None, None) == aql.AQL_ERR_NULL
    assert f(A, 4, 6, B, Y, None, None) == aql.AQL_ERR_SHAPE
    assert f(A, 4, 64, B, Y, MIS, None) == aql.AQL_ERR_ALIGN
    assert f(A, 0, 64, B, Y, None, None) == aql.AQL_OK


def test_act_quant_validation():
    f = L.aql_quantize_act_per_tensor
    assert f(A, 4, 64, 0.0, 0, 0, 1.0, 0, B, None, None) == aql.AQL_ERR_PARAM
    assert f(A, 4, 64, float("inf"), 0, 0, 1.0, 0, B, None, None) == aql.AQL_ERR_PARAM
    assert f(A, 4, 64, float("nan"), 0, 0, 1.0, 0, B, None, None) == aql.AQL_ERR_PARAM
    assert f(A, 4, 64, 0.1, 128, 0, 1.0, 0, B, None, None) == aql.AQL_ERR_PARAM
    assert f(A, 4, 64, 0.1, -129, 0, 1.0, 0, B, None, None) == aql.AQL_ERR_PARAM
    assert f(A, 4, 64, 0.1, 0, 1, 1.0, 0, B, None, None) == aql.AQL_ERR_NULL
    assert f(A, 4, 64, 0.1, 0, 1, -1.0, 0, B, Y, None) == aql.AQL_ERR_PARAM
    assert f(A, 0, 64, 0.1, 0, 1, 0.01, 0, B, Y, None) == aql.AQL_OK


def test_w8a16_validation():
    f = L.aql_linear_w8a16
    assert f(NUL, 1, 64, B, Y, None, 8, Y, None, 0, None) == aql.AQL_ERR_NULL
    assert f(A, 1, 64, B, Y, None, 8, NUL, None, 0, None) == aql.AQL_ERR_NULL
    assert f(A, 1, 40, B, Y, None, 8, Y, None, 0, None) == aql.AQL_ERR_SHAPE
    assert f(A, 1, 0, B, Y, None, 8, Y, None, 0, None) == aql.AQL_ERR_SHAPE
    assert f(A, -1, 64, B, Y, None, 8, Y, None, 0, None) == aql.AQL_ERR_SHAPE
    assert f(A, 1, 64, B, Y, MIS, 8, Y, None, 0, None) == aql.AQL_ERR_ALIGN
    assert f(A, 1, 64, B, Y, None, 8, Y, MIS, 64, None) == aql.AQL_ERR_ALIGN
    assert f(A, 0, 64, B, Y, None, 8, Y, None, 0, None) == aql.AQL_OK
    assert f(A, 3, 64, B, Y, None, 0, Y, None, 0, None) == aql.AQL_OK


def test_w8a16_workspace_bytes():
    """The optional split-K workspace: S x M x N floats for prefill shapes of
    few 128 x 256 tiles and K >= 8192 (S doubles while the units stay <= 256
    and each keeps >= 16 stages of 64 k), and for 12 <= M < 64 rows with fewer
    than 8192 channels and K >= 8192 (4 splits up to 128 tiles of 64 channels
    x 16 rows, 2 up to 256); 0 elsewhere."""
    wb = lambda M, N, K: L.aql_workspace_bytes(aql.AQL_OP_W8A16, M, N, K)
    assert wb(512, 4096, 14336) == 4 * 512 * 4096 * 4    # 64 tiles -> 4 splits
    assert wb(1024, 4096, 14336) == 2 * 1024 * 4096 * 4  # 128 tiles -> 2
    assert wb(128, 4096, 14336) == 8 * 128 * 4096 * 4    # 16 tiles, 224 stages -> 8
    assert wb(64, 300, 16384) == 16 * 64 * 300 * 4
    assert wb(2048, 4096, 14336) == 0                    # 256 wide tiles: no split
    assert wb(512, 14336, 4096) == 0                     # K < 8192
    assert wb(16, 4096, 14336) == 4 * 16 * 4096 * 4      # 64 skinny tiles -> 4
    assert wb(32, 4096, 11008) == 4 * 32 * 4096 * 4      # 128 -> 4
    assert wb(48, 5000, 8192) == 2 * 48 * 5000 * 4       # 237 -> 2
    assert wb(63, 8000, 8192) == 0                       # 500 tiles: no split
    assert wb(11, 4096, 14336) == 0                      # M < 12: the skinny tile
    assert wb(16, 8192, 14336) == 0                      # 8192 channels: shared-x form
    assert wb(16, 4096, 8176) == 0                       # K < 8192
    assert wb(1, 4096, 14336) == 0                       # decode band
    assert wb(4, 4096, 14336) == 0
    assert wb(512, 4096, -1) == 0


def test_q8ta_validation():
    f = L.aql_linear_q8ta_q8csw
    args = lambda **k: [k.get("x", A), k.get("M", 4), k.get("K", 64), k.get("s1", 0.1),
                        k.get("z1", 0), k.get("two", 1), k.get("s2", 0.001), k.get("z2", 0),
                        k.get("q", B), k.get("wsum", Y), k.get("wsc", Y), None, k.get("N", 8),
                        k.get("y", Y), k.get("ws", A), k.get("wsb", 1 << 20), None]
    assert f(*args(q=NUL)) == aql.AQL_ERR_NULL
    assert f(*args(wsum=NUL)) == aql.AQL_ERR_NULL
    assert f(*args(s1=-0.1)) == aql.AQL_ERR_PARAM
    assert f(*args(s2=0.0)) == aql.AQL_ERR_PARAM
    assert f(*args(z2=300)) == aql.AQL_ERR_PARAM
    assert f(*args(K=72)) == aql.AQL_ERR_SHAPE
    assert f(*args(K=aql.AQL_MAX_K_INT8 + 16)) == aql.AQL_ERR_SHAPE
    assert f(*args(y=MIS)) == aql.AQL_ERR_ALIGN
    assert f(*args(wsb=100)) == aql.AQL_ERR_WORKSPACE
    assert f(*args(ws=NUL)) == aql.AQL_ERR_WORKSPACE
    assert f(*args(M=0)) == aql.AQL_OK


def test_q8ta_noalloc_validation():
    """The allocation-free static W8A8 entry: the same checks as the workspace
    entry, and a call needing more than the fixed scratch is refused before any
    HIP call."""
    f = L.aql_linear_q8ta_q8csw_noalloc
    args = lambda **k: [k.get("x", A), k.get("M", 4), k.get("K", 64), k.get("s1", 0.1),
                        k.get("z1", 0), k.get("two", 1), k.get("s2", 0.001), k.get("z2", 0),
                        k.get("q", B), k.get("wsum", Y), k.get("wsc", Y), None, k.get("N", 8),
                        k.get("y", Y), None]
    assert f(*args(q=NUL)) == aql.AQL_ERR_NULL
    assert f(*args(x=NUL)) == aql.AQL_ERR_NULL
    assert f(*args(s1=float("inf"))) == aql.AQL_ERR_PARAM
    assert f(*args(z2=-129)) == aql.AQL_ERR_PARAM
    assert f(*args(K=40)) == aql.AQL_ERR_SHAPE
    assert f(*args(x=MIS)) == aql.AQL_ERR_ALIGN
    # 2 * M * K bytes of codes: 1024 x 4096 fits the 8 MiB exactly, one more row does not
    assert aql.aql_workspace_bytes(aql.AQL_OP_Q8TA_Q8CSW, 1024, 8, 4096) == \
        aql.AQL_NOALLOC_SCRATCH_BYTES
    assert f(*args(M=1025, K=4096)) == aql.AQL_ERR_WORKSPACE
    assert "scratch" in aql.aql_last_error()
    assert f(*args(M=0)) == aql.AQL_OK
    assert f(*args(N=0, M=5000, K=4096)) == aql.AQL_OK  # empty: nothing launched, no scratch


def test_dq8ca_validation():
    f = L.aql_linear_dq8ca
    args = lambda **k: [A, k.get("M", 4), k.get("K", 64), k.get("wfmt", 0), B, Y, Y,
                        k.get("group", 0), None, k.get("N", 8), k.get("y", Y), None, None,
                        k.get("ws", A), k.get("wsb", 1 << 20), None]
    assert f(*args(group=32)) == aql.AQL_ERR_PARAM
    assert f(*args(wfmt=1, group=0)) == aql.AQL_ERR_PARAM
    assert f(*args(wfmt=2)) == aql.AQL_ERR_PARAM
    assert f(*args(wfmt=1, group=32, K=48)) == aql.AQL_ERR_SHAPE
    assert f(*args(K=8)) == aql.AQL_ERR_SHAPE
    assert f(*args(y=NUL)) == aql.AQL_ERR_NULL
    assert f(*args(wsb=10)) == aql.AQL_ERR_WORKSPACE
    assert f(*args(N=0)) == aql.AQL_OK


def test_gemm_validation():
    f = L.aql_gemm_i8_i32
    assert f(NUL, B, Y, 4, 4, 64, None) == aql.AQL_ERR_NULL
    assert f(A, B, Y, 4, 4, 24, None) == aql.AQL_ERR_SHAPE
    assert f(A, B, MIS, 4, 4, 64, None) == aql.AQL_ERR_ALIGN
    assert f(A, B, Y, 0, 4, 64, None) == aql.AQL_OK


def test_measure_helpers_validation():
    r = L.aql_measure_read
    assert r(NUL, 1024, Y, None) == aql.AQL_ERR_NULL
    assert r(A, 1024, NUL, None) == aql.AQL_ERR_NULL
    assert r(MIS, 1024, Y, None) == aql.AQL_ERR_ALIGN
    assert r(A, 1000, Y, None) == aql.AQL_ERR_SHAPE
    assert r(A, 0, Y, None) == aql.AQL_ERR_SHAPE
    assert r(A, 1 << 31, Y, None) == aql.AQL_ERR_SHAPE
    m = L.aql_measure_mfma_i8
    assert m(0, Y, None) == aql.AQL_ERR_SHAPE
    assert m((1 << 30) + 1, Y, None) == aql.AQL_ERR_SHAPE
    assert m(4, NUL, None) == aql.AQL_ERR_NULL
    assert m(4, MIS, None) == aql.AQL_ERR_ALIGN


def test_calibration_validation():
    o = L.aql_minmax_observe
    st = C.c_void_p(0x40000)
    assert o(A, 4, 6, 0, 0, 0.0, 0, st, None) == aql.AQL_ERR_SHAPE      # cols % 4
    assert o(A, -1, 8, 0, 0, 0.0, 0, st, None) == aql.AQL_ERR_SHAPE
    assert o(A, 4, 8, -2, 0, 0.0, 0, st, None) == aql.AQL_ERR_SHAPE
    assert o(A, 4, 8, 0, 1, 0.0, 0, st, None) == aql.AQL_ERR_PARAM      # residual needs s1 > 0
    assert o(A, 4, 8, 0, 1, 0.5, 128, st, None) == aql.AQL_ERR_PARAM
    assert o(A, 4, 8, 0, 1, float("inf"), 0, st, None) == aql.AQL_ERR_PARAM
    assert o(A, 4, 8, 0, 0, 0.0, 0, NUL, None) == aql.AQL_ERR_NULL
    assert o(NUL, 4, 8, 0, 0, 0.0, 0, st, None) == aql.AQL_ERR_NULL
    assert o(MIS, 4, 8, 0, 0, 0.0, 0, st, None) == aql.AQL_ERR_ALIGN
    assert o(NUL, 0, 8, 0, 0, 0.0, 0, st, None) == aql.AQL_OK            # empty: no-op
    assert L.aql_minmax_reset(NUL, None) == aql.AQL_ERR_NULL
    assert L.aql_minmax_reset(MIS, None) == aql.AQL_ERR_ALIGN
    assert L.aql_minmax_qparams(st, NUL, Y, None) == aql.AQL_ERR_NULL
    assert L.aql_minmax_qparams(st, A, MIS, None) == aql.AQL_ERR_ALIGN
    k = L.aql_keep_outliers
    keep = (C.c_int32 * 2)()
    amax = (C.c_float * 2)(1.0, 2.0)
    seam = (C.c_int32 * 2)(0, 2)
    assert k(amax, seam, 2, 2, 20.0, keep) == aql.AQL_ERR_PARAM           # seam 2 of 2
    assert k(amax, seam, -1, 2, 20.0, keep) == aql.AQL_ERR_SHAPE
    assert k(NUL, seam, 2, 2, 20.0, keep) == aql.AQL_ERR_NULL
    assert k(NUL, NUL, 0, 0, 20.0, NUL) == aql.AQL_OK


def test_gptq_validation():
    gq = L.aql_gptq_int8
    big = 1 << 40
    W = C.c_void_p(0x50000)
    I = C.c_void_p(0x60000)
    # (w, N, K, H, damp, block, q, scale, wsum, hinv, info, ws, ws_bytes, stream)
    assert gq(A, 4, 6, B, 0.01, 128, Y, Y, NUL, NUL, I, W, big, None) == aql.AQL_ERR_SHAPE   # K % 4
    assert gq(A, 4, 0, B, 0.01, 128, Y, Y, NUL, NUL, I, W, big, None) == aql.AQL_ERR_SHAPE
    assert gq(A, -1, 8, B, 0.01, 128, Y, Y, NUL, NUL, I, W, big, None) == aql.AQL_ERR_SHAPE
    assert gq(A, 4, 8, B, 0.01, 0, Y, Y, NUL, NUL, I, W, big, None) == aql.AQL_ERR_SHAPE
    assert gq(A, 4, 8, B, 0.01, 257, Y, Y, NUL, NUL, I, W, big, None) == aql.AQL_ERR_SHAPE
    assert gq(A, 4, 8, B, -0.5, 128, Y, Y, NUL, NUL, I, W, big, None) == aql.AQL_ERR_PARAM
    assert gq(A, 4, 8, B, float("nan"), 128, Y, Y, NUL, NUL, I, W, big, None) == aql.AQL_ERR_PARAM
    assert gq(A, 4, 8, NUL, 0.01, 128, Y, Y, NUL, NUL, I, W, big, None) == aql.AQL_ERR_NULL
    assert gq(A, 4, 8, B, 0.01, 128, Y, Y, NUL, NUL, NUL, W, big, None) == aql.AQL_ERR_NULL  # info
    assert gq(A, 4, 8, B, 0.01, 128, Y, Y, NUL, MIS, I, W, big, None) == aql.AQL_ERR_ALIGN
    assert gq(A, 4, 8, B, 0.01, 128, Y, Y, NUL, NUL, I, W, 64, None) == aql.AQL_ERR_WORKSPACE
    assert gq(A, 4, 8, B, 0.01, 128, Y, Y, NUL, NUL, I, NUL, big, None) == aql.AQL_ERR_WORKSPACE
    assert gq(NUL, 0, 8, NUL, 0.01, 128, NUL, NUL, NUL, NUL, NUL, NUL, 0, None) == aql.AQL_OK


def test_keep_outliers_matches_oracle():
    """The host decision against the oracle's, on random statistics with
    missing points, non-positive values, ties and both count parities."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(5)
    for trial in range(300):
        npts = int(rng.integers(0, 30))
        nseams = int(rng.integers(1, 8))
        amax = rng.lognormal(0.0, 2.0, npts).astype(np.float32)
        amax[rng.random(npts) < 0.1] = np.nan
        amax[rng.random(npts) < 0.1] = 0.0
        amax[rng.random(npts) < 0.05] = -1.0
        if npts > 3 and trial % 7 == 0:
            amax[1] = amax[0]  # a tie
        seam = rng.integers(0, nseams, npts).astype(np.int32)
        factor = float(rng.choice([0.0, 1.0, 5.0, 20.0]))
        got = aql.aql_keep_outliers(amax, seam, nseams, factor)
        want = oracle.keep_outliers([float(v) for v in amax], [int(v) for v in seam], nseams,
                                    factor)
        assert got == want, (trial, amax, seam, factor)


def test_valid_call_without_gpu_reports_device():
    """On a host without a gfx950, a valid non-empty call fails with
    AQL_ERR_DEVICE before launching anything."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc = L.aql_gemm_i8_i32(A, B, Y, 4, 4, 64, None)
    assert rc == aql.AQL_ERR_DEVICE
    assert "device" in aql.aql_last_error().lower()


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        aql.aql_gemm_i8_i32(torch.zeros(4, 64, dtype=torch.int8), torch.zeros(4, 64, dtype=torch.int8))


def _problems(n, over=None):
    over = over or {}
    arr = (aql._Problem * n)()
    for i in range(n):
        d = dict(x=0x10000, q=0x20000, scale=0x30000, bias=0, y=0x40000, M=1, N=32, K=64)
        d.update(over.get(i, {}))
        arr[i] = aql._Problem(d["x"], d["q"], d["scale"], d["bias"], d["y"], d["M"], d["N"], d["K"])
    return arr


def test_group_plan_validation():
    """The grouped W8A16 plan is host-only: it validates every problem and writes
    the table without touching device memory."""
    import numpy as np
    nb = aql.aql_w8a16_group_table_bytes(3)
    assert nb == 64 + 3 * 80 and aql.aql_w8a16_group_table_bytes(0) == 0
    buf = np.zeros(nb, np.uint8)
    tp = C.c_void_p(buf.ctypes.data)
    f = L.aql_w8a16_group_plan
    assert f(C.cast(_problems(3), C.c_void_p), 3, tp, nb) == aql.AQL_OK
    # header: magic, version, count, blocks, waves, mblocks, tgroups, cgroups, xlds
    hdr = buf[:36].view(np.int32)
    assert hdr[1] == 2
    rows = 4 * hdr[6] * hdr[7]  # channels per workgroup
    assert hdr[2] == 3 and hdr[3] == 3 * (-(-32 // rows))  # 3 problems of N = 32, M = 1
    assert hdr[4] in (1, 2, 4, 8) and hdr[5] == 0  # M = 1: the single-row tile
    assert hdr[7] in (1, 2, 4) and hdr[8] == 1024  # x of K = 64 shared through 1 KiB of LDS
    # the LDS holding x is sized for the largest K of the group; past 16384 x is not shared
    assert f(C.cast(_problems(3, {1: dict(K=4096)}), C.c_void_p), 3, tp, nb) == aql.AQL_OK
    assert hdr[8] == 8192
    assert f(C.cast(_problems(3, {2: dict(K=16400)}), C.c_void_p), 3, tp, nb) == aql.AQL_OK
    assert hdr[8] == 0
    # single rows with 768 <= K <= 4096 take the contiguous-pieces kernel: 4 waves,
    # 32 channels a workgroup up to K = 1024, 8 above (N = 32: 1 and 4 workgroups)
    assert f(C.cast(_problems(3, {0: dict(K=960), 1: dict(K=2560), 2: dict(K=768)}), C.c_void_p),
             3, tp, nb) == aql.AQL_OK
    hk = buf[:40].view(np.int32)
    assert hk[9] == 1 and hk[4] == 4 and hk[5] == 0 and hk[7] == 1 and hk[8] == 0
    assert hk[3] == 1 + 4 + 1
    # one problem outside the range keeps the whole group on the tile kernels
    assert f(C.cast(_problems(3, {0: dict(K=960), 1: dict(K=2560), 2: dict(K=4112)}), C.c_void_p),
             3, tp, nb) == aql.AQL_OK
    assert buf[:40].view(np.int32)[9] == 0
    assert f(C.cast(_problems(3, {0: dict(K=960, M=2), 1: dict(K=2560)}), C.c_void_p),
             3, tp, nb) == aql.AQL_OK
    assert buf[:40].view(np.int32)[9] == 0
    # a pieces table whose launch fields were altered is refused
    assert f(C.cast(_problems(3, {0: dict(K=960), 1: dict(K=2560), 2: dict(K=768)}), C.c_void_p),
             3, tp, nb) == aql.AQL_OK
    tampered = buf.copy()
    tampered[16:20] = np.array([2], np.int32).view(np.uint8)  # waves
    assert L.aql_linear_w8a16_grouped(C.c_void_p(tampered.ctypes.data), A, None) == aql.AQL_ERR_PARAM
    # M > 1 tiles have one wave tile per workgroup and load x directly
    assert f(C.cast(_problems(3, {0: dict(M=5)}), C.c_void_p), 3, tp, nb) == aql.AQL_OK
    assert hdr[5] > 0 and hdr[7] == 1 and hdr[8] == 0
    assert f(C.cast(_problems(3), C.c_void_p), 3, tp, nb - 1) == aql.AQL_ERR_WORKSPACE
    assert f(C.cast(_problems(3), C.c_void_p), 0, tp, nb) == aql.AQL_ERR_SHAPE
    assert f(C.cast(_problems(3, {1: dict(K=40)}), C.c_void_p), 3, tp, nb) == aql.AQL_ERR_SHAPE
    assert "problem 1" in aql.aql_last_error()
    assert f(C.cast(_problems(3, {2: dict(q=0)}), C.c_void_p), 3, tp, nb) == aql.AQL_ERR_NULL
    assert f(C.cast(_problems(3, {0: dict(y=0x40004)}), C.c_void_p), 3, tp, nb) == aql.AQL_ERR_ALIGN
    # empty problems are dropped from the table
    assert f(C.cast(_problems(3, {1: dict(M=0, x=0, q=0, y=0)}), C.c_void_p), 3, tp, nb) == aql.AQL_OK
    assert buf[:20].view(np.int32)[2] == 2
    # a table not written by the plan is refused; an all-empty group is a no-op
    bad = np.zeros(nb, np.uint8)
    assert L.aql_linear_w8a16_grouped(C.c_void_p(bad.ctypes.data), A, None) == aql.AQL_ERR_PARAM
    assert f(C.cast(_problems(1, {0: dict(N=0, q=0, scale=0, y=0)}), C.c_void_p), 1, tp, nb) == aql.AQL_OK
    assert L.aql_linear_w8a16_grouped(tp, None, None) == aql.AQL_OK
