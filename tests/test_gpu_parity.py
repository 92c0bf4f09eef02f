"""GPU parity: every C-ABI entry point against the CPU oracle on the same
seeded inputs.

Integer results (codes, scales of the quantizers, zero points, weight sums,
int32 accumulators) must match bit for bit. Float outputs must satisfy, per
element, |y - y_ref| <= rtol |y_ref| + atol * T, where T is the oracle's sum
of the magnitudes of the addends (so cancellation near zero cannot fail a
correct kernel), and, over the whole output, ||y - y_ref|| <= norm ||y_ref||:
    fp32 outputs: rtol 1e-3, atol 1e-5, norm 1e-5
    bf16 outputs: rtol 2e-2, atol 1e-4, norm 4e-3
Sizes: small ragged shapes spanning several tiles with tails, the edge cases
(empty, all-zero rows, one-sided rows, tiny scales, saturating outliers), and
every workload at its full size, compared on all outputs where the oracle
finishes in seconds (all but the 7B prefill GEMMs) and otherwise on one row
from every 64-row band (rows are independent, so the oracle runs on those
rows only).
"""
import numpy as np
import pytest
import torch

import activation_quantized_linear_amd as aql
import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FP32 = (1e-3, 1e-5, 1e-5)
BF16 = (2e-2, 1e-4, 4e-3)


def dev(t):
    return t.contiguous().to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits(t):
    return workloads.bf16_bits(t.cpu())


def check_float(y, ref, tol, crit, what):
    rtol, atol, norm = crit
    y = np.asarray(y, np.float64)
    assert y.shape == ref.shape, what
    assert np.all(np.isfinite(y)), what
    err = np.abs(y - ref)
    bound = rtol * np.abs(ref) + atol * tol
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at "
                             f"{i}: got {y[i]!r} want {ref[i]!r} (T={tol[i]!r})")
    den = max(np.linalg.norm(ref), 1e-300)
    assert np.linalg.norm(y - ref) <= norm * den + 1e-300, f"{what}: normwise error too large"


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ quantizers


@pytest.mark.parametrize("mode", [aql.AQL_WQ_SYM127, aql.AQL_WQ_SYM127_5])
@pytest.mark.parametrize("wdt", ["f32", "bf16"])
@pytest.mark.parametrize("N,K", [(256, 256), (37, 4), (5, 12), (70, 260), (9, 1028), (33, 4100),
                                 (3, 17000), (130, 960)])
def test_quantize_weight_int8(mode, wdt, N, K):
    say("quantize_weight_int8", mode, wdt, N, K)
    g = workloads.gen(100 + N + K)
    w = workloads.small_matrix(g, N, K, std=0.02)
    w[N // 2] = 0.0
    if N > 3:
        w[1] *= 1e-30  # subnormal-scale row
        w[2, 0] = 5.0   # one outlier
    if wdt == "bf16":
        w = w.to(torch.bfloat16)
    q, s, ws = aql.aql_quantize_weight_int8(dev(w), mode)
    qo, so, wso = oracle.quantize_weight_int8(w.float().numpy(), mode)
    assert np.array_equal(host(q), qo)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(ws), wso)


def test_quantize_weight_tiny_zero_row():
    d = workloads.tiny()
    q, s, ws = aql.aql_quantize_weight_int8(dev(d["w"]), aql.AQL_WQ_SYM127)
    qo, so, wso = oracle.quantize_weight_int8(d["w"].numpy(), 0)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    assert host(s)[7] == 1.0 and not host(q)[7].any() and host(ws)[7] == 0


@pytest.mark.parametrize("K,N,mode", [(4096, 14336, 0), (14336, 4096, 0), (4096, 4096, 1)])
def test_quantize_weight_full_size(K, N, mode):
    say("quantize_weight full", K, N, mode)
    d = workloads.llm7b(K, N, 1, seed=1)
    q, s, ws = aql.aql_quantize_weight_int8(dev(d["w"]), mode)
    qo, so, wso = oracle.quantize_weight_int8(d["w"].numpy(), mode)
    assert np.array_equal(host(s), so)
    assert np.array_equal(host(ws), wso)
    assert np.array_equal(host(q), qo)


@pytest.mark.parametrize("N,K", [(7, 32), (33, 96), (100, 4096), (11008, 4096)])
def test_quantize_weight_q4gsw(N, K):
    say("q4gsw", N, K)
    g = workloads.gen(200 + N)
    w = workloads.small_matrix(g, N, K, std=0.02)
    w[0, :32] = 0.0
    q4, gs, gsum = aql.aql_quantize_weight_q4gsw(dev(w), 32)
    q4o, gso, gsumo = oracle.quantize_weight_q4gsw(w.numpy(), 32)
    assert np.array_equal(host(q4), q4o)
    assert np.array_equal(host(gs), gso)
    assert np.array_equal(host(gsum), gsumo)


def _edge_rows(x):
    M = x.shape[0]
    if M >= 6:
        x[1] = x[1].abs()
        x[2] = -x[2].abs()
        x[3] = 0.0
        x[4] *= 1e-30
        x[5, 1] = 3000.0
    return x


@pytest.mark.parametrize("M,K", [(1, 4), (3, 100), (6, 256), (64, 4096), (2048, 4096), (5, 20000),
                                 (9, 1028)])
def test_choose_qparams_rows(M, K):
    say("choose_qparams_rows", M, K)
    g = workloads.gen(300 + M + K)
    x = _edge_rows(workloads.small_matrix(g, M, K, std=2.0))
    s, z, xq = aql.aql_choose_qparams_rows(dev(x))
    so, zo, xqo = oracle.choose_qparams_rows(x.numpy())
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(z), zo)
    assert np.array_equal(host(xq), xqo)
    s2, z2, none = aql.aql_choose_qparams_rows(dev(x), quantize=False)
    assert none is None and np.array_equal(host(s2), so) and np.array_equal(host(z2), zo)


def test_per_tensor_calibration_as_one_row():
    """The workload's static (s1, z1) is the per-row rule applied to all
    calibration rows as one row; GPU and oracle agree bit for bit."""
    d = workloads.two_pass()
    calib = d["x"][d["calib_rows"]].reshape(1, -1).contiguous()
    s, z, _ = aql.aql_choose_qparams_rows(dev(calib), quantize=False)
    so, zo, _ = oracle.choose_qparams_rows(calib.numpy(), quantize=False)
    assert host(s)[0] == so[0] and host(z)[0] == zo[0]


@pytest.mark.parametrize("two_pass", [False, True])
@pytest.mark.parametrize("M,K", [(1, 4), (37, 256), (512, 4096)])
def test_quantize_act_per_tensor(two_pass, M, K):
    say("quantize_act_per_tensor", two_pass, M, K)
    d = workloads.two_pass(seed=7, M=max(M, 2), K=K, N=8)
    x = d["x"][:M].contiguous()
    s1, z1 = 0.0372, -3
    s2, z2 = float(np.float32(s1) / np.float32(255.0)), 2
    out = aql.aql_quantize_act_per_tensor(dev(x), s1, z1, two_pass, s2, z2)
    ref = oracle.quantize_act_per_tensor(x.numpy(), s1, z1, two_pass, s2, z2)
    if two_pass:
        assert np.array_equal(host(out[0]), ref[0]) and np.array_equal(host(out[1]), ref[1])
    else:
        assert np.array_equal(host(out), ref)


# ------------------------------------------------------------- integer GEMM


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (17, 33, 80), (130, 257, 272), (256, 256, 4096),
                                   (3, 500, 64), (2050, 2100, 32)])
def test_gemm_i8_i32(M, N, K):
    """int32 stage entry: 64-row tiles while 128-row tiles would be fewer than
    256, 128-row tiles from there (2050 x 2100: 17 x 17 of them)."""
    say("gemm_i8_i32", M, N, K)
    rng = np.random.default_rng(M * 7 + N + K)
    a = rng.integers(-128, 128, size=(M, K), dtype=np.int64).astype(np.int8)
    b = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    a[0, :] = -128
    b[0, :] = -128  # the largest products
    c = aql.aql_gemm_i8_i32(dev(torch.from_numpy(a)), dev(torch.from_numpy(b)))
    assert np.array_equal(host(c).astype(np.int64), oracle.gemm_i8(a, b))


def test_gemm_i8_i32_full_size():
    """The int32 stage entry at the W8A8 workload's shape, every accumulator."""
    M, N, K = 512, 4096, 4096
    say("gemm_i8_i32 full", M, N, K)
    rng = np.random.default_rng(9)
    a = rng.integers(-128, 128, size=(M, K), dtype=np.int64).astype(np.int8)
    b = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    c = host(aql.aql_gemm_i8_i32(dev(torch.from_numpy(a)), dev(torch.from_numpy(b))))
    assert np.array_equal(c.astype(np.int64), oracle.gemm_i8(a, b))


# -------------------------------------------------------------------- W8A16


def _w8a16_case(x, w, bias=None):
    """Quantize w on the device (codes and scales checked bit for bit against
    the oracle's quantizer), run the W8A16 linear, return (y, y_ref, T)."""
    q, s, _ = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127)
    qo, so, _ = oracle.quantize_weight_int8(w.float().numpy(), oracle.WQ_SYM127)
    assert np.array_equal(host(q), qo), "device weight codes differ from the oracle's"
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32)), "weight scales differ"
    b = None if bias is None else dev(bias)
    y = aql.aql_linear_w8a16(dev(x), q, s, b)
    yref, tol = oracle.linear_w8a16(bits(x), qo, so, None if bias is None else bits(bias))
    return host(y.float()), yref, tol


def test_w8a16_tiny():
    d = workloads.tiny()
    y, yref, tol = _w8a16_case(d["x"], d["w"])
    check_float(y, yref, tol, BF16, "tiny")
    assert np.all(y[:, 7] == 0.0)


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (2, 15, 80), (1, 100, 960), (3, 33, 2560),
                                   (16, 64, 4112), (17, 50, 128), (33, 129, 256), (70, 40, 1024),
                                   (1, 9, 272), (1, 70, 16384), (1, 37, 16400), (1, 200, 20000),
                                   (1, 4100, 48), (1, 70001, 32), (1, 1000, 8208),
                                   (1, 4100, 12288), (1, 9, 2048), (1, 8, 4096), (1, 17, 2064),
                                   (1, 3, 8192), (1, 5, 6160), (1, 13, 65536),
                                   (1, 2049, 4080), (2, 9, 2048), (4, 17, 16384), (3, 1000, 6160),
                                   (4, 8, 4096), (2, 4100, 14336), (3, 7, 16400), (3, 14336, 2048),
                                   (3, 1000, 4096), (4, 3000, 2048)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_w8a16_shapes(M, N, K, with_bias):
    """Ragged W8A16 shapes for every M band. M = 1 with 2048 <= K <= 8192 runs
    the contiguous single-row kernel, 2 <= M <= 4 with 2048 <= K <= 16384 the
    contiguous few-rows kernel (one or two pieces of 1 KB per wave and row,
    the last piece partly past K, N not a multiple of 8); K = 16400 at M = 3
    falls back to the skinny tile."""
    say("w8a16", M, N, K, with_bias)
    g = workloads.gen(400 + M + N + K)
    w = workloads.small_matrix(g, N, K, std=0.02)
    x = workloads.small_matrix(g, M, K).to(torch.bfloat16)
    b = workloads.small_matrix(g, 1, N)[0].to(torch.bfloat16) if with_bias else None
    if N > 2:
        w[1] = 0.0
    y, yref, tol = _w8a16_case(x, w, b)
    check_float(y, yref, tol, BF16, f"w8a16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(9, 8200, 512), (12, 45, 4096), (31, 8195, 272),
                                   (63, 100, 1040), (16, 32, 16), (10, 17, 14336),
                                   (4, 100, 272), (4, 8200, 1040), (4, 33, 16), (4, 7, 14352),
                                   (17, 12300, 4096), (16, 16384, 6000), (5, 8192, 16)])
def test_w8a16_skinny_tile(M, N, K):
    """4 <= M < 64 runs the 16-row skinny tile on 16x16x32 MFMAs, from N = 8192
    in its shared-x form (64 channels a workgroup; one K range for K <= 4096
    from N = 12288, else two): ragged channel and row tiles (M = 4 fills a
    quarter of the 16 rows, M = 17 and 31 a second row block), one 16-k step,
    a last 256-k step partly past K, and a K whose steps are split over the
    most waves."""
    say("w8a16 skinny", M, N, K)
    g = workloads.gen(900 + M + N + K)
    w = workloads.small_matrix(g, N, K, std=0.02)
    x = workloads.small_matrix(g, M, K).to(torch.bfloat16)
    b = workloads.small_matrix(g, 1, N)[0].to(torch.bfloat16)
    y, yref, tol = _w8a16_case(x, w, b)
    check_float(y, yref, tol, BF16, f"w8a16 skinny {M}x{N}x{K}")


def test_w8a16_grouped_skinny():
    """A grouped launch whose largest M selects the skinny tile for every
    problem (M from 1 to 40)."""
    g = workloads.gen(910)
    shapes = [(40, 300, 512), (1, 2560, 960), (9, 8200, 256), (16, 70, 4112)]
    probs, refs = [], []
    for M, N, K in shapes:
        w = workloads.small_matrix(g, N, K, std=0.02)
        x = workloads.small_matrix(g, M, K).to(torch.bfloat16)
        q, s, _ = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127)
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        probs.append((dev(x), q, s, None, y))
        refs.append(x)
    host_t, dev_t = aql.aql_w8a16_group_plan(probs)
    aql.aql_linear_w8a16_grouped(host_t, dev_t)
    for (x, q, s, _, y), xc in zip(probs, refs):
        yref, tol = oracle.linear_w8a16(bits(xc), host(q), host(s), None)
        check_float(host(y.float()), yref, tol, BF16, f"grouped skinny {tuple(y.shape)}")


def test_w8a16_smolvlm_sweep():
    layers = workloads.smolvlm(seed=0)
    say("w8a16 smolvlm sweep", len(layers))
    for li, L in enumerate(layers):
        for wname, xname in (("w_up", "x_up"), ("w_gate", "x_up"), ("w_down", "x_down")):
            y, yref, tol = _w8a16_case(L[xname], L[wname])
            check_float(y, yref, tol, BF16, f"layer {li} {wname}")


@pytest.mark.parametrize("M,N,K", [(64, 128, 64), (65, 129, 80), (128, 300, 1040), (200, 257, 4096),
                                   (513, 130, 272), (1024, 2048, 512), (2000, 4100, 272),
                                   (1920, 8200, 80), (2100, 8200, 144), (2000, 4100, 16),
                                   (2100, 8200, 48)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_w8a16_prefill_shapes(M, N, K, with_bias):
    """Prefill-sized M runs the tiled bf16-MFMA GEMM (64 x 128, 128 x 128 or,
    from 160 tiles on, 128 x 256 tiles, with a 2-stage ring from 512 on):
    ragged M, N and K (K % 64 != 0), N not a multiple of 8, with and without
    bias."""
    say("w8a16 prefill", M, N, K, with_bias)
    g = workloads.gen(700 + M + N + K)
    w = workloads.small_matrix(g, N, K, std=0.02)
    x = workloads.small_matrix(g, M, K).to(torch.bfloat16)
    b = workloads.small_matrix(g, 1, N)[0].to(torch.bfloat16) if with_bias else None
    w[1] = 0.0
    y, yref, tol = _w8a16_case(x, w, b)
    check_float(y, yref, tol, BF16, f"w8a16 prefill {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(200, 1000, 8208), (64, 300, 16384), (513, 130, 12304)])
def test_w8a16_prefill_split_k(M, N, K):
    """Few wide tiles and long rows: with a workspace the wide tile splits K
    (7, 16 and 8 splits here; ragged M, N and a partial last stage) and a
    second launch adds the partial sums; with a workspace below the size asked
    for, the same call runs unsplit. Both against the oracle."""
    say("w8a16 split-K", M, N, K)
    nb = aql.aql_workspace_bytes(aql.AQL_OP_W8A16, M, N, K)
    assert nb > 0
    g = workloads.gen(750 + M + N + K)
    w = workloads.small_matrix(g, N, K, std=0.02)
    x = workloads.small_matrix(g, M, K).to(torch.bfloat16)
    b = workloads.small_matrix(g, 1, N)[0].to(torch.bfloat16)
    q, s, _ = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127)
    yref, tol = oracle.linear_w8a16(bits(x), host(q), host(s), bits(b))
    for nbytes in (nb, 16):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        y = aql.aql_linear_w8a16(dev(x), q, s, dev(b), workspace=ws)
        check_float(host(y.float()), yref, tol, BF16, f"w8a16 split-K {M}x{N}x{K} ws={nbytes}")


@pytest.mark.parametrize("M,N,K", [(12, 1000, 8192), (40, 4100, 9008), (63, 2052, 16400),
                                   (13, 70, 65536), (16, 4096, 14336)])
def test_w8a16_skinny_split_k(M, N, K):
    """12 <= M < 64, fewer than 8192 channels and long rows: with a workspace
    the shared-x skinny tile splits K (4 ranges up to 128 tiles of 64 x 16, 2
    up to 256; a last range shorter than the others, a last 256-k step partly
    past K, ragged rows and channels) and a second launch adds the partial
    sums; with a workspace below the size asked for, the same call runs the
    skinny tile. Both against the oracle."""
    say("w8a16 skinny split-K", M, N, K)
    nb = aql.aql_workspace_bytes(aql.AQL_OP_W8A16, M, N, K)
    assert nb > 0
    g = workloads.gen(770 + M + N + K)
    w = workloads.small_matrix(g, N, K, std=0.02)
    x = workloads.small_matrix(g, M, K).to(torch.bfloat16)
    b = workloads.small_matrix(g, 1, N)[0].to(torch.bfloat16)
    q, s, _ = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127)
    yref, tol = oracle.linear_w8a16(bits(x), host(q), host(s), bits(b))
    for nbytes in (nb, 16):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        y = aql.aql_linear_w8a16(dev(x), q, s, dev(b), workspace=ws)
        check_float(host(y.float()), yref, tol, BF16, f"w8a16 skinny split-K {M}x{N}x{K} ws={nbytes}")


@pytest.mark.parametrize("K,N", list(workloads.LLM7B_SHAPES))
@pytest.mark.parametrize("M", [512, 2048])
def test_w8a16_llm7b_prefill_full_size(K, N, M):
    """7B shapes at M = 512 and 2048 (the tiled GEMM at its real sizes, both
    tile shapes; M = 512, K = 14336 splits K over 4 workgroups, the binding
    allocating the workspace), checked on every channel of one random row from
    each 64-row band (so every 64- and 128-row tile is visited), plus the
    first and last rows."""
    say("w8a16 7b prefill", K, N, M)
    d = workloads.llm7b(K, N, M, seed=6)
    q, s, _ = aql.aql_quantize_weight_int8(dev(d["w"]), aql.AQL_WQ_SYM127)
    y = host(aql.aql_linear_w8a16(dev(d["x"]), q, s).float())
    rng = np.random.default_rng(K + N)
    rows = np.unique(np.r_[0, M - 1, np.arange(0, M, 64) + rng.integers(0, 64, M // 64)])
    yref, tol = oracle.linear_w8a16(bits(d["x"][rows]), host(q), host(s), None)
    check_float(y[rows], yref, tol, BF16, f"7b prefill {K}x{N}")


@pytest.mark.parametrize("K,N", list(workloads.LLM7B_SHAPES))
@pytest.mark.parametrize("M", [1, 4, 16])
def test_w8a16_llm7b_full(K, N, M):
    say("w8a16 7b", K, N, M)
    d = workloads.llm7b(K, N, M, seed=2)
    y, yref, tol = _w8a16_case(d["x"], d["w"])
    check_float(y, yref, tol, BF16, f"7b {K}x{N} M={M}")


# ------------------------------------------------------ W8A8 static two-pass


def _calib(x_rows):
    s, z, _ = oracle.choose_qparams_rows(np.ascontiguousarray(x_rows.reshape(1, -1)), quantize=False)
    return float(s[0]), int(z[0])


@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (37, 200, 256), (130, 129, 272), (64, 128, 1024),
                                   (2050, 2100, 64)])
@pytest.mark.parametrize("two_pass,z2", [(False, 0), (True, 0), (True, -5), (True, 7)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_q8ta_shapes(M, N, K, two_pass, z2, with_bias):
    """Static W8A8 on ragged shapes, one and two passes; the second pass with
    its own zero point z2 (folded as acc2 - z2 * wsum). One pass takes 64-row
    tiles while 128-row tiles would be fewer than 256, 128-row tiles from
    there (2050 x 2100: 17 x 17 of them)."""
    say("q8ta", M, N, K, two_pass, z2, with_bias)
    d = workloads.two_pass(seed=11 + M, M=max(M, 2), K=K, N=N)
    x = d["x"][:M].contiguous()
    s1, z1 = _calib(d["x"][1:].numpy())
    s2 = float(np.float32(s1) / np.float32(255.0))
    g = workloads.gen(500 + N)
    b = workloads.small_matrix(g, 1, N)[0] if with_bias else None
    q, ws, wsum = aql.aql_quantize_weight_int8(dev(d["w"]), aql.AQL_WQ_SYM127_5)
    y = aql.aql_linear_q8ta_q8csw(dev(x), s1, z1, q, wsum, ws, None if b is None else dev(b),
                                  two_pass, s2, z2)
    o = oracle.linear_q8ta_q8csw(x.numpy(), s1, z1, host(q), host(ws),
                                 None if b is None else b.numpy(), two_pass, s2, z2)
    check_float(host(y), o["y"], o["tol"], FP32, "q8ta")


@pytest.mark.parametrize("z2", [0, 3])
def test_q8ta_two_pass_full_size(z2):
    """The two-pass W8A8 workload (M = 512, K = N = 4096, attention-sink row 0)
    at full size: weight codes, both passes' activation codes, both int32
    accumulators (through the stage entry) bit for bit, and every output
    within the fp32 tolerance; z2 = 0 is the workload, z2 = 3 exercises the
    second zero point's fold."""
    d = workloads.two_pass()
    x, w = d["x"], d["w"]
    say("q8ta full", tuple(x.shape), tuple(w.shape), z2)
    s1, z1 = _calib(x[d["calib_rows"]].numpy())
    s2 = float(np.float32(s1) / np.float32(255.0))
    q, ws, wsum = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127_5)
    qh, wsh, wsumh = host(q), host(ws), host(wsum)
    qo, wso, wsumo = oracle.quantize_weight_int8(w.numpy(), 1)
    assert np.array_equal(qh, qo) and np.array_equal(wsh, wso) and np.array_equal(wsumh, wsumo)
    y = host(aql.aql_linear_q8ta_q8csw(dev(x), s1, z1, q, wsum, ws, None, True, s2, z2))
    xq1, xq2 = aql.aql_quantize_act_per_tensor(dev(x), s1, z1, True, s2, z2)
    o = oracle.linear_q8ta_q8csw(x.numpy(), s1, z1, qh, wsh, None, True, s2, z2)
    assert np.array_equal(host(xq1), o["xq1"]) and np.array_equal(host(xq2), o["xq2"])
    check_float(y, o["y"], o["tol"], FP32, f"q8ta full z2={z2}")
    acc1 = host(aql.aql_gemm_i8_i32(xq1, q))
    acc2 = host(aql.aql_gemm_i8_i32(xq2, q))
    assert np.array_equal(acc1.astype(np.int64), o["acc1"])
    assert np.array_equal(acc2.astype(np.int64), o["acc2"])


# ----------------------------------------------------- W8A8 dynamic (8da4w)


def _dq8ca_case(x, w, wfmt, bias=None):
    if wfmt == aql.AQL_W_Q8CSW:
        wq, wsc, wsum = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127)
        group = 0
    else:
        wq, wsc, wsum = aql.aql_quantize_weight_q4gsw(dev(w), 32)
        group = 32
    M = x.shape[0]
    xs = torch.empty(M, dtype=torch.float32, device=DEV)
    xz = torch.empty(M, dtype=torch.int32, device=DEV)
    y = aql.aql_linear_dq8ca(dev(x), wq, wsc, wsum, wfmt, group,
                             None if bias is None else dev(bias), x_scale_out=xs, x_zp_out=xz)
    return host(y), host(wq), host(wsc), host(xs), host(xz), group


@pytest.mark.parametrize("wfmt", [aql.AQL_W_Q8CSW, aql.AQL_W_Q4GSW])
@pytest.mark.parametrize("M,N,K", [(1, 30, 64), (4, 100, 4096), (16, 17, 96), (17, 200, 256),
                                   (128, 129, 512), (200, 64, 160), (40, 33, 32), (17, 1, 64),
                                   (2050, 2100, 64)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_dq8ca_shapes(wfmt, M, N, K, with_bias):
    say("dq8ca", wfmt, M, N, K, with_bias)
    g = workloads.gen(600 + M + N + K)
    x = _edge_rows(workloads.small_matrix(g, M, K))
    w = workloads.small_matrix(g, N, K, std=0.02)
    b = workloads.small_matrix(g, 1, N)[0] if with_bias else None
    y, wq, wsc, xs, xz, group = _dq8ca_case(x, w, wfmt, b)
    o = oracle.linear_dq8ca(x.numpy(), wq, wsc, wfmt, group, None if b is None else b.numpy())
    assert np.array_equal(xs, o["x_scale"]) and np.array_equal(xz, o["x_zp"])
    check_float(y, o["y"], o["tol"], FP32, f"dq8ca {wfmt} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 17, 64), (3, 100, 2048), (4, 15, 2080),
                                   (4, 1000, 4096), (1, 33, 4128), (4, 70, 8192), (3, 9, 8224),
                                   (4, 11008, 4096)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_dq8ca_q4_few_rows(M, N, K, with_bias):
    """M <= 4 and K <= 8192 run the few-rows 4-bit kernel (group sums on the
    4x4x4 int8 matrix-core blocks, 1, 2, 4, 8 or 16 steps of 512 k in flight,
    the last partly past K; N not a multiple of 16); K = 8224 takes the general
    streaming kernel. Rows: all zero, one-sided positive, one-sided negative, a
    saturating outlier."""
    say("dq8ca q4 small M", M, N, K, with_bias)
    g = workloads.gen(660 + M + N + K)
    x = workloads.small_matrix(g, M, K)
    x[0] = 0.0 if M > 1 else x[0]
    if M > 1:
        x[1] = x[1].abs()
    if M > 2:
        x[2] = -x[2].abs()
    if M > 3:
        x[3, K // 2] = 3000.0
    w = workloads.small_matrix(g, N, K, std=0.02)
    b = workloads.small_matrix(g, 1, N)[0] if with_bias else None
    y, wq, wsc, xs, xz, group = _dq8ca_case(x, w, aql.AQL_W_Q4GSW, b)
    o = oracle.linear_dq8ca(x.numpy(), wq, wsc, aql.AQL_W_Q4GSW, group, None if b is None else b.numpy())
    assert np.array_equal(xs.view(np.uint32), o["x_scale"].view(np.uint32))
    assert np.array_equal(xz, o["x_zp"])
    check_float(y, o["y"], o["tol"], FP32, f"dq8ca q4 small {M}x{N}x{K}")
    # without the qparams outputs
    q4, gs, gsum = aql.aql_quantize_weight_q4gsw(dev(w), 32)
    y2 = aql.aql_linear_dq8ca(dev(x), q4, gs, gsum, aql.AQL_W_Q4GSW, 32,
                              None if b is None else dev(b))
    assert np.array_equal(host(y2), y)


@pytest.mark.parametrize("M,N,K", [(2600, 4100, 96), (2000, 4100, 96), (1000, 4100, 160),
                                   (50, 1000, 224), (33, 47, 4064), (30, 201, 4064),
                                   (150, 1001, 160), (65, 11008, 4096), (300, 700, 96),
                                   (100, 7000, 1056), (128, 9650, 224), (80, 11008, 96)])
def test_dq8ca_q4_large_tiles_ragged(M, N, K):
    """Each tile shape of the 4-bit tiled kernel with ragged edges in M and N
    and group counts that leave the last stage partly empty (K = 96, 160, 224,
    1056 and 4064): 128 x 128 (2600 x 4100: 693 of them), 128 x 96 (2000 x 4100,
    1000 x 4100), and with the groups over 4 waves 64 x 64 (300 x 700), 64 x 96
    (100 x 7000, 128 x 9650: one round of tiles where 64 x 48 would need two),
    64 x 48 (the rest of 65 <= M <= 256, 80 x 11008 with its last row tile a
    quarter full), 32 x 96 (33 <= M <= 64) and 32 x 48 (M <= 32)."""
    say("dq8ca q4 large ragged", M, N, K)
    g = workloads.gen(650)
    x = _edge_rows(workloads.small_matrix(g, M, K))
    w = workloads.small_matrix(g, N, K, std=0.02)
    b = workloads.small_matrix(g, 1, N)[0]
    y, wq, wsc, xs, xz, group = _dq8ca_case(x, w, aql.AQL_W_Q4GSW, b)
    o = oracle.linear_dq8ca(x.numpy(), wq, wsc, aql.AQL_W_Q4GSW, group, b.numpy())
    assert np.array_equal(xs, o["x_scale"]) and np.array_equal(xz, o["x_zp"])
    check_float(y, o["y"], o["tol"], FP32, f"dq8ca q4 {M}x{N}x{K}")


@pytest.mark.parametrize("M", list(workloads.DYN_MS))
def test_dq8ca_8da4w_full_size(M):
    d = workloads.dyn8da4w(M, seed=4)
    say("dq8ca 8da4w full", M)
    x, w = d["x"], d["w"]
    y, wq, wsc, xs, xz, _ = _dq8ca_case(x, w, aql.AQL_W_Q4GSW)
    q4o, gso, _ = oracle.quantize_weight_q4gsw(w.numpy(), 32)
    assert np.array_equal(wq, q4o) and np.array_equal(wsc, gso)
    o = oracle.linear_dq8ca(x.numpy(), wq, wsc, oracle.W_Q4GSW, 32)
    assert np.array_equal(xs, o["x_scale"]) and np.array_equal(xz, o["x_zp"])
    check_float(y, o["y"], o["tol"], FP32, f"8da4w M={M}")


def test_empty_problems_are_noops():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    q = torch.zeros(8, 64, dtype=torch.int8, device=DEV)
    s = torch.ones(8, dtype=torch.float32, device=DEV)
    y = aql.aql_linear_w8a16(x, q, s)
    assert tuple(y.shape) == (0, 8)


def test_w8a16_grouped_mixed():
    """One grouped launch over ragged problems (different M, N, K, with and
    without bias, one empty) equals each problem's oracle result."""
    g = workloads.gen(700)
    shapes = [(1, 2560, 960, False), (1, 960, 2560, True), (4, 100, 80, False), (0, 64, 64, False),
              (17, 33, 4112, True), (16, 1, 16, False), (1, 14336, 4096, False)]
    probs, refs = [], []
    for M, N, K, hb in shapes:
        w = workloads.small_matrix(g, N, K, std=0.02)
        x = workloads.small_matrix(g, M, K).to(torch.bfloat16)
        b = workloads.small_matrix(g, 1, N)[0].to(torch.bfloat16) if hb else None
        q, s, _ = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127)
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        probs.append((dev(x), q, s, None if b is None else dev(b), y))
        refs.append((x, b))
    host_t, dev_t = aql.aql_w8a16_group_plan(probs)
    for rep in range(2):
        for p in probs:
            p[4].fill_(float("nan"))
        aql.aql_linear_w8a16_grouped(host_t, dev_t)
        for (x, q, s, b, y), (xc, bc) in zip(probs, refs):
            if x.shape[0] == 0:
                continue
            yref, tol = oracle.linear_w8a16(bits(xc), host(q), host(s),
                                            None if bc is None else bits(bc))
            check_float(host(y.float()), yref, tol, BF16, f"grouped {tuple(y.shape)}")


def test_w8a16_grouped_single_row_mixed_k():
    """A grouped launch of single-row problems whose K differ (x is shared in
    LDS sized for the largest K) and whose N leave workgroups partly or wholly
    past the last channel."""
    g = workloads.gen(710)
    shapes = [(9, 4112), (2560, 960), (1, 16), (33, 2560), (100, 64), (70, 16384)]
    _grouped_single_row(g, shapes)


def test_w8a16_grouped_single_row_past_lds():
    """As above with one K past the LDS budget for x: every wave then loads its x."""
    _grouped_single_row(workloads.gen(711), [(9, 4112), (40, 16400), (2560, 960)])


def _grouped_single_row(g, shapes):
    probs, refs = [], []
    for N, K in shapes:
        w = workloads.small_matrix(g, N, K, std=0.02)
        x = workloads.small_matrix(g, 1, K).to(torch.bfloat16)
        q, s, _ = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127)
        y = torch.full((1, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        probs.append((dev(x), q, s, None, y))
        refs.append(x)
    host_t, dev_t = aql.aql_w8a16_group_plan(probs)
    aql.aql_linear_w8a16_grouped(host_t, dev_t)
    for (x, q, s, _, y), xc in zip(probs, refs):
        yref, tol = oracle.linear_w8a16(bits(xc), host(q), host(s), None)
        check_float(host(y.float()), yref, tol, BF16, f"grouped single-row {tuple(y.shape)}")


def test_w8a16_grouped_smolvlm_sweep_in_graph():
    """The decode sweep as one grouped launch, captured in a HIP graph and
    replayed three times, each replay checked against the oracle."""
    layers = workloads.smolvlm(seed=1, layers=8)
    probs, refs = [], []
    for L in layers:
        for wn, xn in (("w_up", "x_up"), ("w_gate", "x_up"), ("w_down", "x_down")):
            q, s, _ = aql.aql_quantize_weight_int8(dev(L[wn]), aql.AQL_WQ_SYM127)
            x = dev(L[xn])
            y = torch.empty(1, q.shape[0], dtype=torch.bfloat16, device=DEV)
            probs.append((x, q, s, None, y))
            refs.append(L[xn])
    host_t, dev_t = aql.aql_w8a16_group_plan(probs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aql.aql_linear_w8a16_grouped(host_t, dev_t)
    expect = [oracle.linear_w8a16(bits(xc), host(p[1]), host(p[2])) for p, xc in zip(probs, refs)]
    for rep in range(3):
        for p in probs:
            p[4].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for p, (yref, tol) in zip(probs, expect):
            check_float(host(p[4].float()), yref, tol, BF16, f"graph replay {rep}")


# ---------------------------------------------------------- static calibration


def _observe_case(x, batches, seq=0, residual=None):
    """Device observer over row batches of x vs the oracle's, bit for bit."""
    st = aql.aql_minmax_state(DEV)
    ost = oracle.minmax_empty()
    for part in np.array_split(np.arange(x.shape[0]), batches):
        xb = x[part[0]:part[-1] + 1] if len(part) else x[:0]
        aql.aql_minmax_observe(dev(xb), st, seq=seq, residual=residual)
        r = {} if residual is None else dict(residual=True, s1=residual[0], z1=residual[1])
        ost = oracle.minmax_observe(xb.numpy(), ost, seq=seq, **r)
    got = host(st)
    assert np.array_equal(got, ost), (got, ost)
    s, z = aql.aql_minmax_qparams(st)
    assert (float(host(s)[0]), int(host(z)[0])) == oracle.minmax_qparams(ost)
    return got


@pytest.mark.parametrize("rows,cols,batches,seq", [(1, 4, 1, 0), (37, 96, 3, 12), (300, 1028, 5, 0),
                                                   (64, 4096, 2, 16), (5, 8, 1, 5)])
def test_minmax_observe(rows, cols, batches, seq):
    say("minmax observe", rows, cols, batches, seq)
    g = workloads.gen(900 + rows + cols)
    x = workloads.small_matrix(g, rows, cols, std=3.0)
    if rows > 13:
        x[12, 1] = 1e4   # at position 0 of a 12-row sequence
        x[13, 2] = -7e3
    _observe_case(x, batches, seq)


def test_minmax_empty_and_qparams_defaults():
    st = aql.aql_minmax_state(DEV)
    x = torch.zeros(0, 64, dtype=torch.float32, device=DEV)
    aql.aql_minmax_observe(x, st)
    # one row, at position 0 of its sequence: not observed
    aql.aql_minmax_observe(torch.ones(1, 8, dtype=torch.float32, device=DEV), st, seq=5)
    s, z = aql.aql_minmax_qparams(st)
    assert float(host(s)[0]) == 1.0 and int(host(z)[0]) == 0
    assert np.array_equal(host(st), oracle.minmax_empty())


def test_two_pass_calibration_on_the_workload():
    """The static two-pass calibration of the W8A8 workload: the first
    observer (sink row left out) reproduces the workload's (s1, z1), the second
    observes the first pass's rounding error; both bit for bit with the oracle."""
    d = workloads.two_pass(seed=0)
    x = d["x"]
    M = x.shape[0]
    st1 = _observe_case(x, 1, seq=M)  # one call: the workload is one 512-token sequence
    s1, z1 = oracle.minmax_qparams(st1)
    cs, cz, _ = oracle.choose_qparams_rows(x[1:].reshape(1, -1).numpy(), quantize=False)
    assert (s1, z1) == (float(cs[0]), int(cz[0]))
    st2 = _observe_case(x, 1, seq=M, residual=(s1, z1))
    s2, _ = oracle.minmax_qparams(st2)
    assert 0 < s2 < s1 / 100  # the residual spans about one first-pass step
