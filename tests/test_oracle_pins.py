"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values
worked by hand from the pages' rules (tests/golden), library routines that
implement the same definitions independently (torch.ao observers,
quantized_decomposed ops), the pages' own torch expressions run by torch,
brute force with exact Python integers / fractions, closed-form identities
(the scale factorization, the zero-point fold) and the error bounds the
pages state (the two-pass residual). Together they are chosen so that a
dropped term, a wrong sign or index, a transposed operand, a wrong rounding
mode or a wrong clamp range in the oracle fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

import torch.ao.quantization.fx._decomposed  # noqa: E402,F401  registers quantized_decomposed
from torch.ao.quantization.observer import MinMaxObserver, PerChannelMinMaxObserver  # noqa: E402

qd = torch.ops.quantized_decomposed
F32_EPS = float(np.finfo(np.float32).eps)


def _floats(v):
    return np.array([float(t) for t in v], np.float32)


def _ints(v):
    return np.array([int(t) for t in v], np.int64)


# ------------------------------------------------------------ weight quantizer


def test_weight_quant_worked_examples(golden):
    for c in golden("weight_quant_worked.txt"):
        w = _floats(c["w"])[None, :]
        q, s, ws = oracle.quantize_weight_int8(w, int(c["mode"][0]))
        assert s[0] == np.float32(float(c["scale"][0])), c["case"]
        assert np.array_equal(q[0].astype(np.int64), _ints(c["q"])), c["case"]
        assert int(ws[0]) == int(c["wsum"][0]), c["case"]


def _nearest_code(t, lo, hi):
    """Brute force: the code c in [lo, hi] nearest to the float t, ties to even c."""
    best = None
    for c in range(lo, hi + 1):
        d = abs(Fraction(float(t)) - c)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


@pytest.mark.parametrize("mode,lo,den", [(0, -127, 127.0), (1, -128, 127.5)])
def test_weight_quant_brute_force_nearest(mode, lo, den):
    g = workloads.gen(11)
    w = workloads.small_matrix(g, 6, 40, std=0.02).numpy()
    w[2, 5] = 0.0
    w[4, :] = 0.0  # all-zero row
    q, s, ws = oracle.quantize_weight_int8(w, mode)
    for n in range(w.shape[0]):
        amax = np.float32(np.max(np.abs(w[n])))
        if amax == 0:
            assert s[n] == 1.0 and not q[n].any() and ws[n] == 0
            continue
        assert s[n] == np.float32(amax / np.float32(den))
        for k in range(w.shape[1]):
            t = np.float32(w[n, k] / s[n])  # the page's w / scale, one binary32 division
            assert q[n, k] == _nearest_code(t, lo, 127), (n, k)
        assert ws[n] == int(q[n].astype(np.int64).sum())


def test_weight_quant_sym127_invariants():
    g = workloads.gen(12)
    w = workloads.small_matrix(g, 64, 500, std=0.02).numpy()
    w[10] *= 1e-20  # tiny but nonzero row
    q, s, _ = oracle.quantize_weight_int8(w, 0)
    # every non-zero row reaches the clamp value exactly once the absmax is divided out
    assert np.all(np.abs(q.astype(np.int32)).max(axis=1) == 127)
    assert q.min() >= -127
    # reconstruction error within half a step (plus fp32 rounding of w/s)
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-6))


def test_weight_quant_matches_page_expressions():
    """Ming int8_linear quantize_weight and tiny-llm quantize_per_channel, run as
    printed on torch CPU, give the same codes; scales equal except tiny-llm's
    all-zero-row scale 0 (the convention fixed here is scale 1)."""
    g = workloads.gen(13)
    w = workloads.small_matrix(g, 300, 260, std=0.02)
    w[3] = 0.0
    q, s, _ = oracle.quantize_weight_int8(w.numpy(), 0)
    wf = w.float()
    absmax = wf.abs().amax(dim=1)
    scale = absmax / 127.0
    zero = scale == 0
    scale = torch.where(zero, torch.ones_like(scale), scale)
    qt = torch.round(wf / scale[:, None]).clamp(-127, 127).to(torch.int8)
    qt = torch.where(zero[:, None], torch.zeros_like(qt), qt)
    assert np.array_equal(qt.numpy(), q)
    assert np.array_equal(scale.numpy(), s)
    s3 = w.abs().amax(dim=1) / 127
    q3 = torch.round(w / s3.clamp_min(1e-12)[:, None]).clamp_(-127, 127).to(torch.int8)
    assert np.array_equal(q3.numpy(), q)
    diff = np.nonzero(s3.numpy() != s)[0]
    assert list(diff) == [3] and s3[3] == 0 and s[3] == 1.0


def test_weight_quant_sym127_5_matches_observer():
    """SmolVLM recipe weight_int8: torch.ao's per-channel symmetric observer gives
    the same scale bit for bit, and the page's w / scale rounding the same codes."""
    g = workloads.gen(14)
    w = workloads.small_matrix(g, 200, 333, std=0.02)
    obs = PerChannelMinMaxObserver(ch_axis=0, dtype=torch.qint8, quant_min=-128, quant_max=127,
                                   qscheme=torch.per_channel_symmetric)
    obs(w)
    scale, zp = obs.calculate_qparams()
    assert int(zp.abs().max()) == 0
    q, s, _ = oracle.quantize_weight_int8(w.numpy(), 1)
    assert np.array_equal(scale.float().numpy(), s)
    qt = torch.clamp(torch.round(w / scale.float()[:, None]), -128, 127).to(torch.int8)
    assert np.array_equal(qt.numpy(), q)
    # a row whose absmax is 127.5 * 2^-3 maps +-amax to 127 / -128
    w2 = np.zeros((1, 4), np.float32)
    w2[0] = [127.5 / 8, -127.5 / 8, 1 / 8, 0]
    q2, s2, _ = oracle.quantize_weight_int8(w2, 1)
    assert s2[0] == np.float32(1 / 8) and list(q2[0]) == [127, -128, 1, 0]


def test_int8_codes_exact_in_bf16():
    """tiny-llm quant docstring: |q| <= 127 < 256, so int8 -> bf16 is exact (also -128)."""
    v = torch.arange(-128, 128, dtype=torch.int32)
    assert torch.equal(v.to(torch.bfloat16).to(torch.int32), v)


# --------------------------------------------------------------- q4gsw packer


def test_q4gsw_codes_scales_and_packing():
    g = workloads.gen(15)
    N, K, G = 12, 128, 32
    w = workloads.small_matrix(g, N, K, std=0.02).numpy()
    w[1, 32:64] = 0.0  # all-zero group
    w[2, 0:32] = 0.0
    w[2, 3] = 7.5 * 0.25  # group absmax 1.875 -> gs = 0.25 exactly
    w[2, 4] = -7.5 * 0.25
    w[2, 5] = 0.25 * 2.5  # tie -> even 2
    q4, gs, gsum = oracle.quantize_weight_q4gsw(w, G)
    codes = oracle.unpack_q4(q4, K).astype(np.int64)
    assert codes.min() >= -8 and codes.max() <= 7
    for n in range(N):
        for gi in range(K // G):
            blk = w[n, gi * G:(gi + 1) * G]
            amax = np.float32(np.abs(blk).max())
            c = codes[n, gi * G:(gi + 1) * G]
            if amax == 0:
                assert gs[n, gi] == 1.0 and not c.any()
            else:
                assert gs[n, gi] == np.float32(amax / np.float32(7.5))
                for j in range(G):
                    t = np.float32(blk[j] / gs[n, gi])
                    assert c[j] == _nearest_code(t, -8, 7)
            assert gsum[n, gi] == c.sum()
    assert gs[1, 1] == 1.0
    assert gs[2, 0] == np.float32(0.25)
    assert list(codes[2, 3:6]) == [7, -8, 2]
    # packing: byte n*K/2 + k/2, k even in the low nibble
    assert (q4[2, 1] & 0xF) == (codes[2, 2] & 0xF) and (q4[2, 1] >> 4) == (codes[2, 3] & 0xF)


# ----------------------------------------------------- activation quantization


def test_act_quant_worked_examples(golden):
    for c in golden("act_quant_worked.txt"):
        x = _floats(c["x"])
        two = int(c["two_pass"][0]) == 1
        args = dict(s1=float(c["s1"][0]), z1=int(c["z1"][0]))
        if two:
            xq1, xq2 = oracle.quantize_act_per_tensor(x, two_pass=True, s2=float(c["s2"][0]),
                                                      z2=int(c["z2"][0]), **args)
            assert np.array_equal(xq2.astype(np.int64), _ints(c["xq2"])), c["case"]
        else:
            xq1 = oracle.quantize_act_per_tensor(x, **args)
        assert np.array_equal(xq1.astype(np.int64), _ints(c["xq1"])), c["case"]


def test_act_quant_matches_quantized_decomposed():
    """SmolVLM recipe Q8Linear.forward: quantize_per_tensor for both passes and the
    residual through the page's fake_quant expression; codes bit-identical."""
    d = workloads.two_pass(seed=3, M=64, K=512, N=8)
    x = d["x"]
    s1, z1 = 0.0372, -5
    s2, z2 = np.float32(s1) / np.float32(255.0), 0
    xq1, xq2 = oracle.quantize_act_per_tensor(x.numpy(), s1, z1, True, float(s2), z2)
    t1 = qd.quantize_per_tensor(x, float(np.float32(s1)), z1, -128, 127, torch.int8)
    assert np.array_equal(t1.numpy(), xq1)

    def fake_quant(v, s, z):
        return (torch.clamp(torch.round(v * (1.0 / s)) + z, -128, 127) - z) * s

    s1f = float(np.float32(s1))
    r = x - fake_quant(x, s1f, z1)
    t2 = qd.quantize_per_tensor(r, float(s2), z2, -128, 127, torch.int8)
    assert np.array_equal(t2.numpy(), xq2)


def test_two_pass_error_bound():
    """SmolVLM recipe docstring: with s2 ~ s1/255 the activation error drops from
    s1/2 to about s1/510. For unclamped elements: one pass <= s1/2, two passes
    <= s2/2 (= s1/510) plus fp32 rounding."""
    d = workloads.two_pass(seed=4, M=128, K=1024, N=8)
    x = d["x"].numpy()
    calib = x[1:]
    s1 = np.float32(0.0)
    lo, hi = min(calib.min(), 0.0), max(calib.max(), 0.0)
    s1 = np.float32((np.float32(hi) - np.float32(lo)) / np.float32(255.0))
    z1 = int(-128 - np.rint(np.float32(lo) / s1))
    s2 = np.float32(s1 / np.float32(255.0))
    xq1, xq2 = oracle.quantize_act_per_tensor(x, float(s1), z1, True, float(s2), 0)
    dq1 = (xq1.astype(np.float64) - z1) * float(s1)
    dq2 = xq2.astype(np.float64) * float(s2)
    inside = (x[1:] > lo + float(s1)) & (x[1:] < hi - float(s1))
    e1 = np.abs(x[1:] - dq1[1:])[inside]
    e2 = np.abs(x[1:] - dq1[1:] - dq2[1:])[inside]
    ulp = np.spacing(np.float32(np.abs(x).max()))
    assert e1.max() <= float(s1) / 2 * (1 + 1e-6) + ulp
    assert e2.max() <= float(s1) / 510 * (1 + 1e-3) + 2 * ulp
    assert e2.max() < e1.max() / 100
    # the sink row's outlier channels saturate the first pass
    ch = d["outlier_channels"].numpy()
    assert set(np.unique(xq1[0, ch])) <= {-128, 127}


# -------------------------------------------------------- per-row qparams


def test_choose_qparams_worked_examples(golden):
    for c in golden("choose_qparams_worked.txt"):
        x = _floats(c["x"])[None, :]
        s, z, xq = oracle.choose_qparams_rows(x)
        if "scale_eps" in c:
            assert s[0] == np.float32(F32_EPS), c["case"]
        else:
            assert s[0] == np.float32(np.float32(float(c["scale_num"][0])) / np.float32(255.0))
        assert z[0] == int(c["zp"][0]), c["case"]
        assert np.array_equal(xq[0].astype(np.int64), _ints(c["xq"])), c["case"]


def test_choose_qparams_matches_minmax_observer():
    g = workloads.gen(16)
    x = workloads.small_matrix(g, 40, 300).numpy()
    x[3] = np.abs(x[3])  # all positive
    x[4] = -np.abs(x[4])  # all negative
    x[5] = 0.0  # all zero
    x[6] *= 1e-30  # subnormal-range scale clamps to eps
    x[7, 10] = 3000.0  # one massive activation
    s, z, xq = oracle.choose_qparams_rows(x)
    for m in range(x.shape[0]):
        ob = MinMaxObserver(dtype=torch.qint8, quant_min=-128, quant_max=127,
                            qscheme=torch.per_tensor_affine)
        ob(torch.from_numpy(x[m]))
        ss, zz = ob.calculate_qparams()
        assert ss.item() == s[m] and zz.item() == z[m], m
        t = qd.quantize_per_tensor(torch.from_numpy(x[m]), float(s[m]), int(z[m]), -128, 127,
                                   torch.int8)
        assert np.array_equal(t.numpy(), xq[m]), m


def test_choose_qparams_invariants():
    g = workloads.gen(17)
    x = workloads.small_matrix(g, 50, 777, std=3.0).numpy()
    s, z, xq = oracle.choose_qparams_rows(x)
    dq = (xq.astype(np.float64) - z[:, None]) * s[:, None].astype(np.float64)
    # zero is exactly representable: the code of 0 is zp
    assert np.all(z >= -128) and np.all(z <= 127)
    # row extremes land on (within one code of) the range ends
    for m in range(x.shape[0]):
        assert xq[m].min() <= -127 and xq[m].max() >= 126
    err = np.abs(x - dq)
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))


# ---------------------------------------------------------- integer contraction


def test_gemm_brute_force_and_numpy():
    g = np.random.default_rng(5)
    a = g.integers(-128, 128, size=(5, 37), dtype=np.int64).astype(np.int8)
    b = g.integers(-128, 128, size=(7, 37), dtype=np.int64).astype(np.int8)
    c = oracle.gemm_i8(a, b)
    for m in range(5):
        for n in range(7):
            assert c[m, n] == sum(int(a[m, k]) * int(b[n, k]) for k in range(37))
    a2 = g.integers(-128, 128, size=(33, 300), dtype=np.int64).astype(np.int8)
    b2 = g.integers(-128, 128, size=(45, 300), dtype=np.int64).astype(np.int8)
    assert np.array_equal(oracle.gemm_i8(a2, b2), a2.astype(np.int64) @ b2.astype(np.int64).T)
    # extremes: -128 * -128 summed over K
    a3 = np.full((1, 4096), -128, np.int8)
    assert oracle.gemm_i8(a3, a3)[0, 0] == 4096 * 16384


def test_zero_point_fold_identity():
    g = np.random.default_rng(6)
    xq = g.integers(-128, 128, size=(9, 64), dtype=np.int64).astype(np.int8)
    q = g.integers(-127, 128, size=(11, 64), dtype=np.int64).astype(np.int8)
    z = 37
    lhs = (xq.astype(np.int64) - z) @ q.astype(np.int64).T
    rhs = oracle.gemm_i8(xq, q) - z * q.astype(np.int64).sum(axis=1)[None, :]
    assert np.array_equal(lhs, rhs)


# -------------------------------------------------------------------- W8A16


def _bf16(t):
    return workloads.bf16_bits(t)


def test_w8a16_exact_rational_brute_force():
    g = workloads.gen(18)
    x = workloads.small_matrix(g, 3, 24).to(torch.bfloat16)
    w = workloads.small_matrix(g, 5, 24, std=0.02).numpy()
    b = workloads.small_matrix(g, 1, 5).to(torch.bfloat16)[0]
    q, s, _ = oracle.quantize_weight_int8(w, 0)
    y, tol = oracle.linear_w8a16(_bf16(x), q, s, _bf16(b))
    xf = x.float().numpy()
    bf = b.float().numpy()
    for m in range(3):
        for n in range(5):
            exact = Fraction(float(s[n])) * sum(Fraction(float(xf[m, k])) * int(q[n, k])
                                                for k in range(24)) + Fraction(float(bf[n]))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(1, 10**12) * Fraction(tol[m, n])
            mag = Fraction(abs(float(s[n]))) * sum(abs(Fraction(float(xf[m, k])) * int(q[n, k]))
                                                   for k in range(24)) + abs(Fraction(float(bf[n])))
            assert abs(Fraction(tol[m, n]) - mag) <= Fraction(1, 10**12) * mag


def test_w8a16_scale_factorization():
    """tiny-llm Step 4.6: y_j = sum_i x_i (q_ji s_j) = s_j sum_i x_i q_ji, the same
    values as dequantizing W first (Ming Int8Linear.forward)."""
    d = workloads.tiny(seed=0)
    q, s, _ = oracle.quantize_weight_int8(d["w"].numpy(), 0)
    x = _bf16(d["x"])
    y, tol = oracle.linear_w8a16(x, q, s)
    y2 = oracle.linear_w8a16_dequant_first(x, q, s)
    assert np.all(np.abs(y - y2) <= 1e-12 * tol)
    assert np.all(y[:, 7] == 0.0)  # the all-zero weight row
    # the literal Ming forward in fp32 torch agrees within its own rounding
    wdq = (torch.from_numpy(q).float() * torch.from_numpy(s)[:, None]).to(torch.bfloat16)
    yt = torch.nn.functional.linear(d["x"].float(), wdq.float()).double().numpy()
    assert np.all(np.abs(yt - y) <= 4e-3 * tol + 1e-6)


# ----------------------------------------------------- W8A8 static, two passes


def _calib(rows):
    lo = np.float32(min(rows.min(), 0.0))
    hi = np.float32(max(rows.max(), 0.0))
    s = np.float32((hi - lo) / np.float32(255.0))
    z = int(np.clip(-128 - np.rint(lo / s), -128, 127))
    return float(s), z


@pytest.mark.parametrize("two_pass,z2", [(False, 0), (True, 0), (True, -5), (True, 7)])
def test_q8ta_matches_q8linear_forward(two_pass, z2):
    """SmolVLM recipe Q8Linear.forward, run with torch's quantized_decomposed ops
    and F.linear in fp64, against the oracle's int-accumulate-then-scale form.
    The second pass takes its own affine pair (s2, z2): with z2 != 0 the fold
    acc2 - z2 * wsum must reproduce dequantize (r1q - z2) * s2."""
    d = workloads.two_pass(seed=5, M=24, K=256, N=40)
    x, w = d["x"], d["w"]
    s1, z1 = _calib(x[1:].numpy())
    s2 = float(np.float32(s1) / np.float32(255.0))
    q, ws, _ = oracle.quantize_weight_int8(w.numpy(), 1)
    g = workloads.gen(50)
    bias = workloads.small_matrix(g, 1, 40)[0].numpy()
    o = oracle.linear_q8ta_q8csw(x.numpy(), s1, z1, q, ws, bias, two_pass, s2, z2)
    qt = torch.from_numpy(q)
    wt = qd.dequantize_per_channel(qt, torch.from_numpy(ws), torch.zeros(40, dtype=torch.int64),
                                   0, -128, 127, torch.int8).double()
    x1q = qd.quantize_per_tensor(x, s1, z1, -128, 127, torch.int8)
    assert np.array_equal(x1q.numpy(), o["xq1"])
    x1 = (x1q.double() - z1) * np.float64(np.float32(s1))
    y = torch.nn.functional.linear(x1, wt, torch.from_numpy(bias).double())
    if two_pass:
        r = x - (torch.clamp(torch.round(x * (1.0 / s1)) + z1, -128, 127) - z1) * s1
        r1q = qd.quantize_per_tensor(r, s2, z2, -128, 127, torch.int8)
        assert np.array_equal(r1q.numpy(), o["xq2"])
        r1 = (r1q.double() - z2) * np.float64(np.float32(s2))
        y = y + torch.nn.functional.linear(r1, wt)
    # dequantize_per_channel returns fp32 weights: q * ws is rounded once (2^-24)
    assert np.all(np.abs(y.numpy() - o["y"]) <= 2.0**-23 * o["tol"])
    y2 = oracle.linear_q8ta_dequant_first(o["xq1"], o["xq2"], s1, z1, q, ws, bias, two_pass,
                                          s2, z2)
    assert np.all(np.abs(y2 - o["y"]) <= 1e-12 * o["tol"])
    acc = oracle.gemm_i8(o["xq1"], q)
    assert np.array_equal(acc, o["acc1"])
    if two_pass:
        assert np.array_equal(oracle.gemm_i8(o["xq2"], q), o["acc2"])


def test_q8ta_two_pass_improves_output():
    """The second pass shrinks the output error against the unquantized-activation
    linear, as the recipe's s1/2 -> s1/510 statement predicts."""
    d = workloads.two_pass(seed=6, M=33, K=512, N=24)
    x, w = d["x"].numpy(), d["w"].numpy()
    s1, z1 = _calib(x[1:])
    s2 = float(np.float32(s1) / np.float32(255.0))
    q, ws, _ = oracle.quantize_weight_int8(w, 1)
    wdq = q.astype(np.float64) * ws[:, None].astype(np.float64)
    yref = x[1:].astype(np.float64) @ wdq.T
    y1 = oracle.linear_q8ta_q8csw(x, s1, z1, q, ws)["y"][1:]
    y2 = oracle.linear_q8ta_q8csw(x, s1, z1, q, ws, None, True, s2, 0)["y"][1:]
    e1 = np.linalg.norm(y1 - yref)
    e2 = np.linalg.norm(y2 - yref)
    assert e2 < e1 / 100


# --------------------------------------------------------- W8A8 dynamic (8da4w)


@pytest.mark.parametrize("wfmt", [oracle.W_Q8CSW, oracle.W_Q4GSW])
def test_dq8ca_matches_printed_fold(wfmt):
    """ExecuTorch 8da4w PR: out[m,n] = s[m] * sum_k (xq[m,k] - z[m]) * dequant(w)."""
    d = workloads.dyn8da4w(M=9, K=256, N=30, seed=7)
    x, w = d["x"].numpy(), d["w"].numpy()
    x[2] = np.abs(x[2])
    x[3] = 0.0
    if wfmt == oracle.W_Q8CSW:
        wq, ws, _ = oracle.quantize_weight_int8(w, 0)
        group = 0
    else:
        wq, ws, _ = oracle.quantize_weight_q4gsw(w, 32)
        group = 32
    g = workloads.gen(51)
    bias = workloads.small_matrix(g, 1, 30)[0].numpy()
    o = oracle.linear_dq8ca(x, wq, ws, wfmt, group, bias)
    s, z, xq = oracle.choose_qparams_rows(x)
    assert np.array_equal(s, o["x_scale"]) and np.array_equal(z, o["x_zp"])
    assert np.array_equal(xq, o["xq"])
    y2 = oracle.linear_dq8ca_dequant_first(xq, s, z, wq, ws, 256, wfmt, group, bias)
    assert np.all(np.abs(y2 - o["y"]) <= 1e-12 * o["tol"])
    assert np.all(o["y"][3] == bias.astype(np.float64))  # all-zero row: xq == zp everywhere


def test_dq8ca_q4_exact_rational_brute_force():
    d = workloads.dyn8da4w(M=2, K=64, N=3, seed=8)
    x, w = d["x"].numpy(), d["w"].numpy()
    q4, gs, gsum = oracle.quantize_weight_q4gsw(w, 32)
    codes = oracle.unpack_q4(q4, 64)
    o = oracle.linear_dq8ca(x, q4, gs, oracle.W_Q4GSW, 32)
    s, z, xq = o["x_scale"], o["x_zp"], o["xq"]
    for m in range(2):
        for n in range(3):
            exact = Fraction(float(s[m])) * sum(
                (int(xq[m, k]) - int(z[m])) * int(codes[n, k]) * Fraction(float(gs[n, k // 32]))
                for k in range(64))
            assert abs(Fraction(o["y"][m, n]) - exact) <= Fraction(1, 10**12) * Fraction(o["tol"][m, n])
    assert np.array_equal(gsum, codes.reshape(3, 2, 32).astype(np.int64).sum(axis=2))


# ---------------------------------------------------------- static calibration


def test_minmax_observe_matches_numpy_and_folds():
    g = workloads.gen(30)
    x = workloads.small_matrix(g, 37, 96, std=2.0).numpy()
    x[0, 5] = 500.0    # rows 0, 12, 24, 36 start a 12-row sequence:
    x[12, 3] = -400.0  # with seq = 12 they are not observed
    st = oracle.minmax_observe(x, oracle.minmax_empty())
    assert st[0] == x.min() and st[1] == x.max()
    kept = np.array([r % 12 != 0 for r in range(x.shape[0])])
    st = oracle.minmax_observe(x, oracle.minmax_empty(), seq=12)
    assert st[0] == x[kept].min() and st[1] == x[kept].max()
    assert st[1] < 500.0 and st[0] > -400.0
    # observing in two calls is observing once
    a = oracle.minmax_observe(x[:20], oracle.minmax_empty())
    assert np.array_equal(oracle.minmax_observe(x[20:], a),
                          oracle.minmax_observe(x, oracle.minmax_empty()))
    # nothing observed: the state stays empty
    st = oracle.minmax_observe(x[:1], oracle.minmax_empty(), seq=5)
    assert st[0] == np.inf and st[1] == -np.inf


def test_minmax_observe_residual_matches_torch_fake_quant():
    """The second calibration run observes x - fake_quant(x, s1, z1); torch's
    fake_quantize_per_tensor_affine is an independent implementation of that
    fake quantizer (reciprocal scale, round half to even, clamp)."""
    g = workloads.gen(31)
    x = workloads.small_matrix(g, 50, 64, std=4.0).numpy()
    x[3, :8] = 3000.0  # clipped by the first pass: a large residual
    s1, z1 = oracle.minmax_qparams(oracle.minmax_observe(x[4:], oracle.minmax_empty()))
    st = oracle.minmax_observe(x, oracle.minmax_empty(), residual=True, s1=s1, z1=z1)
    xt = torch.from_numpy(x)
    r = (xt - torch.fake_quantize_per_tensor_affine(xt, s1, z1, -128, 127)).numpy()
    assert st[0] == r.min() and st[1] == r.max()
    # rows the first pass does not clip leave residuals within half a step
    st4 = oracle.minmax_observe(x[4:], oracle.minmax_empty(), residual=True, s1=s1, z1=z1)
    assert max(-st4[0], st4[1]) <= 0.5 * s1 * (1 + 1e-5)


def test_minmax_qparams_matches_observer():
    g = workloads.gen(32)
    base = workloads.small_matrix(g, 24, 40, std=3.0).numpy()
    cases = [base, np.abs(base), -np.abs(base), np.zeros_like(base), base * 1e-30]
    for x in cases:
        ob = MinMaxObserver(dtype=torch.qint8, quant_min=-128, quant_max=127,
                            qscheme=torch.per_tensor_affine)
        st = oracle.minmax_empty()
        for chunk in np.array_split(x, 3):  # several calibration batches
            ob(torch.from_numpy(np.ascontiguousarray(chunk)))
            st = oracle.minmax_observe(chunk, st)
        ss, zz = ob.calculate_qparams()
        assert oracle.minmax_qparams(st) == (ss.item(), zz.item())
    # an observer that saw nothing returns its defaults
    ob = MinMaxObserver(dtype=torch.qint8, quant_min=-128, quant_max=127,
                        qscheme=torch.per_tensor_affine)
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        ss, zz = ob.calculate_qparams()
    assert oracle.minmax_qparams(oracle.minmax_empty()) == (ss.item(), zz.item()) == (1.0, 0)


def test_keep_outliers_worked_example():
    """Worked by hand from the keep-outliers rule: the positive statistics of
    all points are 1, 2, 3, 100, whose median is (2 + 3) / 2 = 2.5; at factor
    20 the bar is 50, so only seam 2 (worst point 100) stays at host
    precision; at factor 40 the bar is 100 and the comparison is strict."""
    nan = float("nan")
    amax = [1.0, 2.0, 3.0, nan, 100.0, 0.0, -1.0]
    seam = [0, 0, 1, 1, 2, 3, 3]
    assert oracle.keep_outliers(amax, seam, 5, 20.0) == [False, False, True, False, False]
    assert oracle.keep_outliers(amax, seam, 5, 40.0) == [False] * 5
    assert oracle.keep_outliers(amax, seam, 5, 0.0) == [False] * 5
    # odd count: 1, 2, 3, 50, 100 -> median 3, bar 60: seam 2 kept, seam 1 (50) not
    amax2 = amax + [50.0]
    seam2 = seam + [1]
    assert oracle.keep_outliers(amax2, seam2, 5, 20.0) == [False, False, True, False, False]
    # no positive statistic: nothing to compare against
    assert oracle.keep_outliers([nan, 0.0], [0, 1], 2, 20.0) == [False, False]


# ------------------------------------------------------------------- GPTQ


def _spd_hessian(g, K, rows, dead=()):
    X = workloads.small_matrix(g, rows, K).double()
    for d in dead:
        X[:, d] = 0.0
    return (X.T @ X).numpy()


def test_gptq_hinv_is_the_upper_factor_of_the_inverse():
    g = workloads.gen(40)
    H = _spd_hessian(g, 48, 200)
    Hd, dead = oracle.gptq_damped(H, 0.01)
    assert not dead.any()
    assert np.allclose(np.diag(Hd) - np.diag(H), 0.01 * np.mean(np.diag(H)), rtol=1e-12)
    hinv = oracle.gptq_hinv(Hd)
    assert np.array_equal(hinv, np.triu(hinv)) and np.all(np.diag(hinv) > 0)
    ref = np.linalg.cholesky(np.linalg.inv(Hd)).T  # numpy's LAPACK, independent
    assert np.allclose(hinv, ref, rtol=1e-9, atol=1e-12 * np.abs(ref).max())
    assert np.allclose(hinv.T @ hinv @ Hd, np.eye(48), atol=1e-9)


def test_gptq_identity_hessian_is_round_to_nearest():
    """With H = I the factor is diagonal and no rounding error is passed on:
    GPTQ is plain round-to-nearest of w / s in binary64."""
    g = workloads.gen(41)
    w = workloads.small_matrix(g, 30, 70, std=0.02).numpy()
    q, s, wsum = oracle.gptq_int8(w, np.eye(70), block=16)
    ref = np.clip(np.rint(w.astype(np.float64) / s[:, None].astype(np.float64)), -128, 127)
    assert np.array_equal(q, ref.astype(np.int8))
    assert np.array_equal(wsum, q.astype(np.int64).sum(1))
    _, s_rtn, _ = oracle.quantize_weight_int8(w, oracle.WQ_SYM127_5)
    assert np.array_equal(s, s_rtn)  # the scales are the SYM127_5 quantizer's


def _gptq_unblocked_torch(w, H, damp=0.01):
    """GPTQ without lazy blocks (every rounding error is pushed onto all later
    columns at once), its factor from torch's own Cholesky and inverse: equal
    to the blocked algorithm in exact arithmetic."""
    _, s, _ = oracle.quantize_weight_int8(w, oracle.WQ_SYM127_5)
    W = torch.from_numpy(w).double().clone()
    Ht = torch.from_numpy(H).double().clone()
    K = W.shape[1]
    dead = torch.diag(Ht) == 0
    Ht[dead, dead] = 1.0
    W[:, dead] = 0.0
    Ht += damp * torch.mean(torch.diag(Ht)) * torch.eye(K, dtype=torch.float64)
    U = torch.linalg.cholesky(torch.linalg.inv(Ht)).T
    sc = torch.from_numpy(s).double()
    Q = torch.zeros_like(W)
    for i in range(K):
        Q[:, i] = torch.clamp(torch.round(W[:, i] / sc), -128, 127)
        e = (W[:, i] - Q[:, i] * sc) / U[i, i]
        W[:, i:] -= e[:, None] * U[i, i:][None, :]
    return Q.numpy().astype(np.int8)


def test_gptq_matches_unblocked_torch_reference():
    g = workloads.gen(42)
    K, N = 96, 40
    H = _spd_hessian(g, K, 300, dead=(5, 77))
    w = workloads.small_matrix(g, N, K, std=0.02).numpy()
    q, _, _ = oracle.gptq_int8(w, H, block=32)
    ref = _gptq_unblocked_torch(w, H)
    diff = q.astype(np.int32) - ref.astype(np.int32)
    # reduction orders differ (LAPACK vs plain sums, lazy vs eager updates):
    # only near-ties may round the other way, by one code
    assert np.abs(diff).max() <= 1 and (diff != 0).mean() < 0.002
    assert np.all(q[:, [5, 77]] == 0)  # dead columns


def test_gptq_lowers_the_hessian_weighted_error():
    """What GPTQ is for: its codes reproduce X W^T better than round-to-nearest."""
    g = workloads.gen(43)
    K, N = 128, 64
    Z = workloads.small_matrix(g, 400, K).double().numpy()
    mix = workloads.small_matrix(g, K, K).double().numpy()
    X = Z @ (np.eye(K) + 0.3 * mix)  # correlated input channels, as real activations are
    X[:, :8] *= 6.0                  # and a few dominant ones
    H = X.T @ X
    w = workloads.small_matrix(g, N, K, std=0.02).numpy()
    q, s, _ = oracle.gptq_int8(w, H, block=32)
    qr, sr, _ = oracle.quantize_weight_int8(w, oracle.WQ_SYM127_5)
    W = w.astype(np.float64)
    e_gptq = np.linalg.norm(X @ (W - q * s[:, None].astype(np.float64)).T)
    e_rtn = np.linalg.norm(X @ (W - qr * sr[:, None].astype(np.float64)).T)
    assert e_gptq < 0.9 * e_rtn
    # the block size changes only the rounding of the updates
    q2, _, _ = oracle.gptq_int8(w, H, block=128)
    assert (q2 != q).mean() < 0.002


# ------------------------------------------------------------- thread count


def test_oracle_results_do_not_depend_on_the_thread_count():
    """The OpenMP loops split only independent output rows, so one thread and
    all threads give the same bits (quantizer, GEMV, W8A8 two-pass, 8da4w)."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((37, 96)) * 0.02).astype(np.float32)
    x = rng.standard_normal((5, 96)).astype(np.float32)
    xb = workloads.bf16_bits(torch.from_numpy(x).to(torch.bfloat16))

    def run():
        q, s, wsum = oracle.quantize_weight_int8(w, oracle.WQ_SYM127_5)
        y16 = oracle.linear_w8a16(xb, q, s)
        y8 = oracle.linear_q8ta_q8csw(x, 0.03, 3, q, s, two_pass=True, s2=0.03 / 255, z2=0)
        q4, gs, _ = oracle.quantize_weight_q4gsw(w)
        yd = oracle.linear_dq8ca(x, q4, gs, wfmt=oracle.W_Q4GSW, group=32)
        return [q, s, wsum, y16, y8, q4, gs, yd]

    many = run()
    oracle.set_threads(1)
    try:
        assert oracle.threads() == 1
        one = run()
    finally:
        oracle.set_threads(None)
    def flat(items):
        out = []
        for v in items:
            if isinstance(v, dict):
                out += [v[k] for k in sorted(v) if v[k] is not None]
            elif isinstance(v, tuple):
                out += list(v)
            else:
                out.append(v)
        return out

    a, b = flat(many), flat(one)
    assert len(a) == len(b) > 8
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_oracle_rejects_mismatched_shapes():
    """The C side trusts the sizes it is given, so the wrappers refuse operands
    whose shapes disagree instead of reading past them."""
    q = np.zeros((4, 32), np.int8)
    s = np.ones(4, np.float32)
    with pytest.raises(ValueError):
        oracle.linear_w8a16(np.zeros((2, 64), np.uint16), q, s)
    with pytest.raises(ValueError):
        oracle.linear_w8a16(np.zeros((2, 32), np.uint16), q, np.ones(3, np.float32))
    with pytest.raises(ValueError):
        oracle.linear_q8ta_q8csw(np.zeros((2, 16), np.float32), 1.0, 0, q, s)
    with pytest.raises(ValueError):
        oracle.linear_dq8ca(np.zeros((2, 32), np.float32), np.zeros((4, 8), np.uint8),
                            np.ones((4, 1), np.float32), wfmt=oracle.W_Q4GSW, group=32)
    with pytest.raises(ValueError):
        oracle.gemm_i8(np.zeros((2, 31), np.int8), q)
    with pytest.raises(ValueError):
        oracle.gptq_int8(np.zeros((4, 8), np.float32), np.eye(9))
