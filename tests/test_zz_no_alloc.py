"""The allocation-free static W8A8 entry point (aql_linear_q8ta_q8csw_noalloc)
against the workspace entry point it mirrors, through the C ABI: outputs must
be identical bit for bit (the same kernels run on the library's fixed scratch
instead of a caller workspace) and within the fp32 tolerance of the oracle.
Two calls in a row, the second on a smaller input, so the second runs on
scratch that still holds the first call's codes."""
import numpy as np
import pytest
import torch

import activation_quantized_linear_amd as aql
import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FP32 = (1e-3, 1e-5)


def _case(seed, M, K, N, two_pass, z2, with_bias):
    d = workloads.two_pass(seed=seed, M=M, K=K, N=N)
    x = d["x"]
    calib = x[1:].reshape(1, -1).contiguous()
    sc, zc, _ = oracle.choose_qparams_rows(calib.numpy(), quantize=False)
    s1, z1 = float(sc[0]), int(zc[0])
    s2 = float(np.float32(s1) / np.float32(255.0))
    g = workloads.gen(seed + 1)
    b = workloads.small_matrix(g, 1, N)[0] if with_bias else None
    return x, d["w"], b, s1, z1, s2, z2, two_pass


def _run(x, w, b, s1, z1, s2, z2, two_pass):
    xd = x.to(DEV)
    bd = None if b is None else b.to(DEV)
    q, ws, wsum = aql.aql_quantize_weight_int8(w.to(DEV), aql.AQL_WQ_SYM127_5)
    y_ref = aql.aql_linear_q8ta_q8csw(xd, s1, z1, q, wsum, ws, bd, two_pass, s2, z2)
    y = torch.full_like(y_ref, float("nan"))
    aql.aql_linear_q8ta_q8csw_noalloc(xd, s1, z1, q, wsum, ws, bd, two_pass, s2, z2, y=y)
    torch.cuda.synchronize()
    yh, yrh = y.cpu().numpy(), y_ref.cpu().numpy()
    assert np.array_equal(yh.view(np.uint32), yrh.view(np.uint32)), "noalloc differs from workspace entry"
    o = oracle.linear_q8ta_q8csw(x.numpy(), s1, z1, q.cpu().numpy(), ws.cpu().numpy(),
                                 None if b is None else b.numpy(), two_pass, s2, z2)
    err = np.abs(yh.astype(np.float64) - o["y"])
    assert np.all(err <= FP32[0] * np.abs(o["y"]) + FP32[1] * o["tol"])


def test_noalloc_matches_workspace_entry_twice_shrinking():
    # the W8A8 workload's shape (two passes, M x K = 2 Mi: 4 MiB of scratch) ...
    print("noalloc: 512x4096x4096 two-pass", flush=True)
    _run(*_case(0, 512, 4096, 4096, True, 0, False))
    # ... then a smaller, ragged call with bias and a second zero point
    print("noalloc: 37x272x200 two-pass z2=-5 bias", flush=True)
    _run(*_case(3, 37, 272, 200, True, -5, True))
    print("noalloc: 5x64x48 one-pass", flush=True)
    _run(*_case(4, 5, 64, 48, False, 0, False))


def test_noalloc_largest_call_then_small():
    # exactly the scratch's capacity (2 * 1024 * 4096 bytes), then a tiny call
    print("noalloc: 1024x4096x256 two-pass (full scratch)", flush=True)
    _run(*_case(5, 1024, 4096, 256, True, 2, False))
    print("noalloc: 2x16x16 two-pass", flush=True)
    _run(*_case(6, 2, 16, 16, True, 0, True))


def test_noalloc_rejects_oversize_without_launch():
    x = torch.zeros(1025, 4096, dtype=torch.float32, device=DEV)
    q = torch.zeros(16, 4096, dtype=torch.int8, device=DEV)
    wsum = torch.zeros(16, dtype=torch.int32, device=DEV)
    ws = torch.ones(16, dtype=torch.float32, device=DEV)
    with pytest.raises(aql.AqlError) as e:
        aql.aql_linear_q8ta_q8csw_noalloc(x, 0.1, 0, q, wsum, ws, None, True, 0.001, 0)
    assert e.value.code == aql.AQL_ERR_WORKSPACE
