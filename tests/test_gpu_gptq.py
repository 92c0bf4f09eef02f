"""GPU parity for GPTQ int8 (aql_gptq_int8) against the CPU oracle.

Both sides compute in binary64 with the same summation order (ascending sums
from 0, no fused multiply-add, correctly rounded division and square root), so
everything is compared bit for bit: the codes, the scales, the code sums and
the upper factor hinv of the damped Hessian's inverse. Sizes: ragged shapes
that end panels and column blocks mid-way (K = 4, 96, 132, 200, 256 against
the 64-column panels, 128-wide tiles and blocks of 1 to 256), dead columns at
either end, both SmolVLM-500M MLP shapes at full size (K = 960 with all of
the 2560 rows, K = 2560 on sampled rows; rows are independent, so the oracle
runs only those), a Hessian that is not positive definite, and the identity
Hessian, whose codes are plain rounding to nearest.
"""
import numpy as np
import pytest
import torch

import activation_quantized_linear_amd as aql
import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def run_gpu(w, H, damp, block, hinv=True):
    q, s, ws, hv, info = aql.aql_gptq_int8(w.contiguous().to(DEV), torch.from_numpy(H).to(DEV),
                                           damp=damp, block=block, hinv=hinv)
    torch.cuda.synchronize()
    return (q.cpu().numpy(), s.cpu().numpy(), ws.cpu().numpy(),
            None if hv is None else hv.cpu().numpy(), int(info.cpu()[0]))


def same_f64(a, b, what):
    assert a.shape == b.shape, what
    eq = a == b
    if not eq.all():
        i = np.unravel_index(np.argmin(eq), eq.shape)
        raise AssertionError(f"{what}: {int((~eq).sum())} of {eq.size} differ; first at {i}: "
                             f"{a[i]!r} vs {b[i]!r}")


@pytest.mark.parametrize("K,N,block,dead", [
    (4, 3, 1, ()),
    (96, 40, 32, (5,)),
    (132, 7, 256, ()),
    (200, 33, 128, (0, 199)),
    (256, 70, 64, (63, 64)),
])
def test_gptq_small(K, N, block, dead):
    say(f"gptq K={K} N={N} block={block} dead={dead}")
    d = workloads.gptq(K, N, seed=K + N, dead=dead)
    w, H = d["w"], d["H"]
    q, s, ws, hv, info = run_gpu(w, H, 0.01, block)
    assert info == 0
    Hd, dd = oracle.gptq_damped(H, 0.01)
    hv_ref = oracle.gptq_hinv(Hd)
    same_f64(hv, hv_ref, "hinv")
    qo, so, wso = oracle.gptq_int8(w.numpy(), H, damp=0.01, block=block, hinv=hv_ref)
    np.testing.assert_array_equal(s, so)
    np.testing.assert_array_equal(q, qo)
    np.testing.assert_array_equal(ws, wso)
    assert not q[:, list(dead)].any() if dead else True


def test_gptq_smolvlm_up_full():
    """SmolVLM-500M up/gate shape (K = 960, N = 2560), every row."""
    K, N = workloads.SMOLVLM_HIDDEN, workloads.SMOLVLM_FFN
    say(f"gptq smolvlm up K={K} N={N}")
    d = workloads.gptq(K, N, seed=1, dead=(17,))
    q, s, ws, hv, info = run_gpu(d["w"], d["H"], 0.01, 128)
    assert info == 0
    hv_ref = oracle.gptq_hinv(oracle.gptq_damped(d["H"], 0.01)[0])
    same_f64(hv, hv_ref, "hinv")
    qo, so, wso = oracle.gptq_int8(d["w"].numpy(), d["H"], block=128, hinv=hv_ref)
    np.testing.assert_array_equal(s, so)
    np.testing.assert_array_equal(q, qo)
    np.testing.assert_array_equal(ws, wso)


def test_gptq_smolvlm_down_sampled():
    """SmolVLM-500M down shape (K = 2560, N = 960): hinv in full, 48 sampled rows."""
    K, N = workloads.SMOLVLM_FFN, workloads.SMOLVLM_HIDDEN
    say(f"gptq smolvlm down K={K} N={N}")
    d = workloads.gptq(K, N, seed=2)
    q, s, ws, hv, info = run_gpu(d["w"], d["H"], 0.01, 128)
    assert info == 0
    hv_ref = oracle.gptq_hinv(oracle.gptq_damped(d["H"], 0.01)[0])
    same_f64(hv, hv_ref, "hinv")
    rows = np.random.default_rng(5).choice(N, 48, replace=False)
    rows = np.unique(np.concatenate([rows, [0, N - 1]]))
    qo, so, wso = oracle.gptq_int8(d["w"].numpy(), d["H"], block=128, rows=rows, hinv=hv_ref)
    np.testing.assert_array_equal(s, so)
    np.testing.assert_array_equal(q[rows], qo)
    np.testing.assert_array_equal(ws[rows], wso)


def test_gptq_not_positive_definite_reports_the_pivot():
    """Column 3 (0-based) carries a negative diagonal that damping cannot lift:
    the first factorization stops at pivot 4 (1-based), as the definition of
    the Cholesky factor requires; the oracle refuses the same matrix."""
    K = 8
    H = np.eye(K)
    H[3, 3] = -2.0
    w = workloads.small_matrix(workloads.gen(3), 5, K, std=0.02)
    *_, info = run_gpu(w, H, 0.01, 4, hinv=False)
    assert info == 4
    with pytest.raises(Exception):
        oracle.gptq_hinv(oracle.gptq_damped(H, 0.01)[0])


def test_gptq_identity_hessian_is_round_to_nearest():
    """H = I: hinv is a multiple of I, no error moves, and the codes are
    binary64 rounding to nearest of w / s, with s the weight quantizer's scale
    (a different kernel)."""
    K, N = 192, 50
    w = workloads.small_matrix(workloads.gen(4), N, K, std=0.02)
    q, s, ws, hv, info = run_gpu(w, np.eye(K), 0.01, 128)
    assert info == 0
    _, sr, _ = aql.aql_quantize_weight_int8(w.to(DEV), mode=aql.AQL_WQ_SYM127_5)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s, sr.cpu().numpy())
    rtn = np.clip(np.rint(w.numpy().astype(np.float64) / s.astype(np.float64)[:, None]), -128, 127)
    np.testing.assert_array_equal(q, rtn.astype(np.int8))
    np.testing.assert_array_equal(ws, rtn.sum(axis=1).astype(np.int32))
    off = hv - np.diag(np.diag(hv))
    assert not off.any()
