"""GPU parity, part two: exact rounding ties through every quantizer, and the
grouped single-row W8A16 launch in the configuration the decode-sweep
benchmark runs (two 8-channel wave tiles sharing a workgroup).

Ties: the pages round with torch.round, which rounds half to even; inputs
built so that w / s or x * (1/s) is exactly k + 0.5 show whether a kernel
rounds half to even (rintf) or half away from zero. The hand-worked golden
cases (tests/golden/*_worked.txt) run through the device quantizers too,
padded to the multiple of 4 the entry points need with values that change
no scale, zero point or code: zeros (the weight amax, the activation
min(., 0) / max(., 0) and a per-tensor code z all stay as they were).
"""
import numpy as np
import pytest
import torch

import activation_quantized_linear_amd as aql
import oracle
import workloads

from test_gpu_parity import BF16, DEV, bits, check_float, dev, host, say

pytestmark = pytest.mark.gpu


def _pad4(v, width=None):
    v = [float(t) for t in v]
    n = width if width is not None else -(-len(v) // 4) * 4
    return np.array(v + [0.0] * (n - len(v)), np.float32)


def _half_even(v):
    """Round half to even (numpy's rint), the reading of torch.round."""
    return np.rint(np.asarray(v, np.float64))


# ------------------------------------------------------------- weight quantizer


def _weight_rows():
    """Rows whose w / s are exact ties, with s an exact power of two."""
    rows = []
    ks = np.arange(-126, 126)
    # SYM127: amax 127 -> s = 1; amax 254 -> s = 2 (w = 2k + 1 -> w / s = k + 0.5)
    rows.append((aql.AQL_WQ_SYM127, np.r_[127.0, ks + 0.5], 1.0, -127))
    rows.append((aql.AQL_WQ_SYM127, np.r_[-254.0, 2.0 * ks + 1.0], 2.0, -127))
    # SYM127_5: amax 127.5 -> s = 1, clamp [-128, 127]; -127.5 is a tie at the low end
    rows.append((aql.AQL_WQ_SYM127_5, np.r_[127.5, -127.5, np.arange(-128, 127) + 0.5], 1.0, -128))
    return rows


@pytest.mark.parametrize("width", [None, 2048])
@pytest.mark.parametrize("wdt", ["f32", "bf16"])
def test_weight_quant_ties(width, wdt):
    """Every w / s an exact tie (both modes, both input dtypes; the short row
    runs the wave-per-row kernel, width 2048 the workgroup-per-row one)."""
    for mode, row, scale, lo in _weight_rows():
        w = _pad4(row, width or -(-len(row) // 4) * 4)[None, :]
        wt = torch.from_numpy(w)
        if wdt == "bf16":
            assert np.array_equal(wt.to(torch.bfloat16).float().numpy(), w)  # exact in bf16
            wt = wt.to(torch.bfloat16)
        say("weight ties", mode, wdt, w.shape)
        q, s, ws = aql.aql_quantize_weight_int8(dev(wt), mode)
        qh, sh, wsh = host(q), host(s), host(ws)
        want = np.clip(_half_even(w / scale), lo, 127).astype(np.int8)
        assert sh[0] == scale
        assert np.array_equal(qh, want)
        assert wsh[0] == int(want.astype(np.int64).sum())
        qo, so, wso = oracle.quantize_weight_int8(w, mode)
        assert np.array_equal(qh, qo) and np.array_equal(sh, so) and np.array_equal(wsh, wso)


@pytest.mark.parametrize("width", [None, 2048])
def test_weight_quant_golden_on_device(golden, width):
    for c in golden("weight_quant_worked.txt"):
        n = len(c["w"])
        w = _pad4(c["w"], width)[None, :]
        mode = int(c["mode"][0])
        q, s, ws = aql.aql_quantize_weight_int8(dev(torch.from_numpy(w)), mode)
        qh = host(q)[0]
        assert np.array_equal(qh[:n], np.array(c["q"], np.int64)), c["case"]
        assert not qh[n:].any(), c["case"]
        assert host(s)[0] == float(c["scale"][0]), c["case"]
        assert host(ws)[0] == int(c["wsum"][0]), c["case"]


# ------------------------------------------------- per-tensor activation quant


@pytest.mark.parametrize("K", [None, 4096])
def test_act_quant_golden_on_device(golden, K):
    for c in golden("act_quant_worked.txt"):
        n = len(c["x"])
        x = _pad4(c["x"], K)[None, :]
        s1, z1 = float(c["s1"][0]), int(c["z1"][0])
        tp = bool(int(c["two_pass"][0]))
        s2 = float(c["s2"][0]) if tp else 1.0
        z2 = int(c["z2"][0]) if tp else 0
        out = aql.aql_quantize_act_per_tensor(dev(torch.from_numpy(x)), s1, z1, tp, s2, z2)
        xq1 = host(out[0] if tp else out)[0]
        assert np.array_equal(xq1[:n], np.array(c["xq1"], np.int64)), c["case"]
        assert np.all(xq1[n:] == z1), c["case"]
        ref = oracle.quantize_act_per_tensor(x, s1, z1, tp, s2, z2)
        assert np.array_equal(xq1, (ref[0] if tp else ref)[0]), c["case"]
        if tp:
            xq2 = host(out[1])[0]
            assert np.array_equal(xq2[:n], np.array(c["xq2"], np.int64)), c["case"]
            assert np.array_equal(xq2, ref[1][0]), c["case"]


@pytest.mark.parametrize("two_pass", [False, True])
def test_act_quant_ties(two_pass):
    """s1 = 1/2 (1/s1 = 2 exactly) and x = (k + 0.5) / 2: every x * (1/s1) is a
    tie, over the whole code range and past both clamps. The residual is then
    +-1/4, and s2 = 1/2 makes every second-pass value a tie at +-1/2."""
    ks = np.arange(-140, 140)
    x = _pad4((ks + 0.5) / 2.0)[None, :]
    s1, z1, s2, z2 = 0.5, 3, 0.5, -3
    say("act ties", two_pass, x.shape)
    out = aql.aql_quantize_act_per_tensor(dev(torch.from_numpy(x)), s1, z1, two_pass, s2, z2)
    xq1 = host(out[0] if two_pass else out)
    want1 = np.clip(_half_even(x * 2.0) + z1, -128, 127)
    assert np.array_equal(xq1, want1.astype(np.int8))
    ref = oracle.quantize_act_per_tensor(x, s1, z1, two_pass, s2, z2)
    assert np.array_equal(xq1, ref[0] if two_pass else ref)
    if two_pass:
        r = x - (want1 - z1) * s1  # exact: every term is a short binary fraction
        want2 = np.clip(_half_even(r * 2.0) + z2, -128, 127)
        assert np.array_equal(host(out[1]), want2.astype(np.int8))
        assert np.array_equal(host(out[1]), ref[1])


# ------------------------------------------------------- per-row qparams


@pytest.mark.parametrize("K", [None, 4096])
def test_choose_qparams_golden_on_device(golden, K):
    for c in golden("choose_qparams_worked.txt"):
        n = len(c["x"])
        x = _pad4(c["x"], K)[None, :]
        s, z, xq = aql.aql_choose_qparams_rows(dev(torch.from_numpy(x)))
        sh, zh, xqh = host(s)[0], host(z)[0], host(xq)[0]
        if "scale_eps" in c:
            assert sh == np.finfo(np.float32).eps, c["case"]
        else:
            assert sh == np.float32(np.float32(c["scale_num"][0]) / np.float32(255.0)), c["case"]
        assert zh == int(c["zp"][0]), c["case"]
        assert np.array_equal(xqh[:n], np.array(c["xq"], np.int64)), c["case"]
        so, zo, xqo = oracle.choose_qparams_rows(x)
        assert sh == so[0] and zh == zo[0] and np.array_equal(xqh, xqo[0]), c["case"]


@pytest.mark.parametrize("K", [260, 4100])
def test_choose_qparams_ties(K):
    """min -64, max 63.5: s = 127.5 / 255 = 1/2 exactly, zp = 0, and every other
    x = (k + 0.5) / 2, so x * (1/s) is a tie for every code; a second row puts
    the same ties around a non-zero zero point (min -32, max 95.5 -> zp = -64)."""
    ks = np.arange(-128, 127)
    r0 = _pad4(np.r_[-64.0, 63.5, (ks + 0.5) / 2.0], K)
    ks1 = np.arange(-64, 191)
    r1 = _pad4(np.r_[-32.0, 95.5, (ks1 + 0.5) / 2.0], K)
    x = np.stack([r0, r1])
    say("qparams ties", x.shape)
    s, z, xq = aql.aql_choose_qparams_rows(dev(torch.from_numpy(x)))
    sh, zh, xqh = host(s), host(z), host(xq)
    assert np.array_equal(sh, np.array([0.5, 0.5], np.float32))
    assert np.array_equal(zh, np.array([0, -64], np.int32))
    want = np.clip(_half_even(x * 2.0) + zh[:, None], -128, 127).astype(np.int8)
    assert np.array_equal(xqh, want)
    so, zo, xqo = oracle.choose_qparams_rows(x)
    assert np.array_equal(sh, so) and np.array_equal(zh, zo) and np.array_equal(xqh, xqo)


# ------------------------------------------------ grouped single-row W8A16


def _plan_header(host_table):
    """(count, total_blocks, waves, mblocks, tgroups, cgroups, xlds, kind) of a plan."""
    h = host_table[:64].view(torch.int32).tolist()
    return dict(count=h[2], total_blocks=h[3], waves=h[4], mblocks=h[5], tgroups=h[6],
                cgroups=h[7], xlds=h[8], kind=h[9])


def test_w8a16_grouped_full_decode_sweep_pieces():
    """The 32-layer decode sweep exactly as the benchmark plans it (96 GEMVs,
    weights quantized on the device): single rows with 768 <= K <= 4096, so
    the plan takes the contiguous-pieces kernel (up and gate, K = 960: 32
    channels a workgroup; down, K = 2560: 8 channels whose three pieces go to
    three waves), 8,960 workgroups; every output of every GEMV is checked, once
    eagerly and on three replays of a HIP graph."""
    layers = workloads.smolvlm(seed=0)
    F, H = workloads.SMOLVLM_FFN, workloads.SMOLVLM_HIDDEN
    probs, refs = [], []
    for L in layers:
        xu, xd = dev(L["x_up"]), dev(L["x_down"])
        for wn, x, xc in (("w_up", xu, L["x_up"]), ("w_gate", xu, L["x_up"]),
                          ("w_down", xd, L["x_down"])):
            q, s, _ = aql.aql_quantize_weight_int8(dev(L[wn]), aql.AQL_WQ_SYM127)
            y = torch.full((1, q.shape[0]), float("nan"), dtype=torch.bfloat16, device=DEV)
            probs.append((x, q, s, None, y))
            refs.append(xc)
    assert len(probs) == 96
    host_t, dev_t = aql.aql_w8a16_group_plan(probs)
    h = _plan_header(host_t)
    say("sweep plan", h)
    assert h["kind"] == 1 and h["mblocks"] == 0 and h["waves"] == 4 and h["count"] == 96
    assert h["total_blocks"] == 32 * (2 * (F // 32) + H // 8) == 8960
    expect = [oracle.linear_w8a16(bits(xc), host(p[1]), host(p[2])) for p, xc in zip(probs, refs)]

    def check(what):
        for i, (p, (yref, tol)) in enumerate(zip(probs, expect)):
            check_float(host(p[4].float()), yref, tol, BF16, f"{what} GEMV {i}")

    aql.aql_linear_w8a16_grouped(host_t, dev_t)
    check("eager")
    graph = torch.cuda.CUDAGraph()
    for p in probs:
        p[4].fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        aql.aql_linear_w8a16_grouped(host_t, dev_t)
    for rep in range(3):
        for p in probs:
            p[4].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check(f"graph replay {rep}")


@pytest.mark.parametrize("dense", [False, True])
def test_w8a16_grouped_pieces_ragged(dense):
    """The contiguous-pieces kernel at the edges of its range: K = 768 (its
    smallest), 1024 (one whole piece), 1040 (a second piece of 16 bytes), 2064,
    4096 (four pieces, one per wave), with N leaving the last workgroup's waves
    partly or wholly past the last channel (N = 1, 9, 33, 41, 2570); with
    `dense` the weights are all +-127 and x is large, so every product is at
    the top of its range."""
    g = workloads.gen(713 + dense)
    shapes = [(2570, 768), (9, 1024), (33, 1040), (1, 2064), (41, 4096), (2560, 960),
              (300, 2560), (8, 4096), (7, 1024)]
    probs, refs = [], []
    for N, K in shapes:
        w = workloads.small_matrix(g, N, K, std=0.02)
        if dense:
            w = torch.where(w >= 0, 1.0, -1.0)
        x = workloads.small_matrix(g, 1, K, std=30.0 if dense else 1.0).to(torch.bfloat16)
        q, s, _ = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127)
        y = torch.full((1, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        probs.append((dev(x), q, s, None, y))
        refs.append(x)
    host_t, dev_t = aql.aql_w8a16_group_plan(probs)
    h = _plan_header(host_t)
    say("pieces ragged plan", h)
    assert h["kind"] == 1
    assert h["total_blocks"] == sum(-(-N // (8 if K > 1024 else 32)) for N, K in shapes)
    aql.aql_linear_w8a16_grouped(host_t, dev_t)
    for (x, q, s, _, y), xc in zip(probs, refs):
        yref, tol = oracle.linear_w8a16(bits(xc), host(q), host(s), None)
        check_float(host(y.float()), yref, tol, BF16, f"pieces ragged {tuple(q.shape)}")


@pytest.mark.parametrize("count", [1, 2, 3, 4, 5])
def test_w8a16_grouped_pieces_small_groups(count):
    """Groups of at most 4 problems go to the pieces kernel by value in the
    kernel arguments (a group of 5 reads its table from memory): each workgroup
    must pick its own problem, including the last block of a ragged N and
    problems with K above and below one 1 KB piece."""
    g = workloads.gen(730 + count)
    pool = [(2570, 960), (9, 2560), (1, 1040), (41, 4096), (960, 768)]
    shapes = pool[:count]
    probs, refs = [], []
    for N, K in shapes:
        w = workloads.small_matrix(g, N, K, std=0.02)
        x = workloads.small_matrix(g, 1, K).to(torch.bfloat16)
        q, s, _ = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127)
        b = workloads.small_matrix(g, 1, N).to(torch.bfloat16)[0]
        y = torch.full((1, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        probs.append((dev(x), q, s, dev(b), y))
        refs.append((x, b))
    host_t, dev_t = aql.aql_w8a16_group_plan(probs)
    h = _plan_header(host_t)
    say("pieces small group", count, h)
    assert h["kind"] == 1 and h["count"] == count
    aql.aql_linear_w8a16_grouped(host_t, dev_t)
    for (x, q, s, _, y), (xc, bc) in zip(probs, refs):
        yref, tol = oracle.linear_w8a16(bits(xc), host(q), host(s), bits(bc))
        check_float(host(y.float()), yref, tol, BF16, f"small group {count} {tuple(q.shape)}")


@pytest.mark.parametrize("N,K", [(1, 2048), (9, 2560), (960, 2560), (2048, 4096), (2049, 4096),
                                 (1000, 3000 // 16 * 16)])
def test_w8a16_single_row_contiguous_small_grids(N, K):
    """The contiguous single-row GEMV at grids of at most one workgroup a CU
    (all 8 weight loads of a wave in flight at once) and just past it (N =
    2049: batches of 2)."""
    g = workloads.gen(740 + N)
    w = workloads.small_matrix(g, N, K, std=0.02)
    x = workloads.small_matrix(g, 1, K).to(torch.bfloat16)
    say("m1c small grid", N, K)
    q, s, _ = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127)
    y = host(aql.aql_linear_w8a16(dev(x), q, s, None).float())
    yref, tol = oracle.linear_w8a16(bits(x), host(q), host(s), None)
    check_float(y, yref, tol, BF16, f"m1c small grid N={N} K={K}")


def test_w8a16_grouped_paired_tiles_ragged_n():
    """A single-row group past 8,192 wave tiles (so tiles are paired per
    workgroup) whose channel counts leave the second tile of a pair partly
    (N = 9, 2570) or wholly (N = 2568, 1) past the last channel, with mixed K."""
    g = workloads.gen(712)
    shapes = [(2560, 960)] * 20 + [(9, 960), (2568, 960), (2570, 1024), (14336, 1024), (1, 512),
                                   (40, 4096)]
    probs, refs = [], []
    for N, K in shapes:
        w = workloads.small_matrix(g, N, K, std=0.02)
        x = workloads.small_matrix(g, 1, K).to(torch.bfloat16)
        q, s, _ = aql.aql_quantize_weight_int8(dev(w), aql.AQL_WQ_SYM127)
        y = torch.full((1, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        probs.append((dev(x), q, s, None, y))
        refs.append(x)
    host_t, dev_t = aql.aql_w8a16_group_plan(probs)
    h = _plan_header(host_t)
    say("ragged paired plan", h)
    assert h["kind"] == 0 and h["mblocks"] == 0 and h["cgroups"] == 2
    assert h["total_blocks"] == sum(-(-N // 16) for N, _ in shapes)
    aql.aql_linear_w8a16_grouped(host_t, dev_t)
    for (x, q, s, _, y), xc in zip(probs, refs):
        yref, tol = oracle.linear_w8a16(bits(xc), host(q), host(s), None)
        check_float(host(y.float()), yref, tol, BF16, f"paired ragged {tuple(y.shape)}")


def test_w8a16_decode_step_with_dependencies():
    """The dependent decode step the benchmark times: per layer one grouped
    launch of up and gate on the same x, then down on up's output, the next
    layer on down's output (8 layers, in a HIP graph replayed twice). Each
    launch's output is checked against the oracle on the input that launch
    actually read."""
    layers = workloads.smolvlm(seed=2, layers=8)
    F, H = workloads.SMOLVLM_FFN, workloads.SMOLVLM_HIDDEN
    x0 = dev(layers[0]["x_up"])
    acts, work = [], []
    for li, L in enumerate(layers):
        qs = {wn: aql.aql_quantize_weight_int8(dev(L[wn]), aql.AQL_WQ_SYM127)[:2]
              for wn in ("w_up", "w_gate", "w_down")}
        yu = torch.empty(1, F, dtype=torch.bfloat16, device=DEV)
        yg = torch.empty(1, F, dtype=torch.bfloat16, device=DEV)
        yd = torch.empty(1, H, dtype=torch.bfloat16, device=DEV)
        x = x0 if li == 0 else acts[-1][2]
        plan = aql.aql_w8a16_group_plan([(x, *qs["w_up"], None, yu), (x, *qs["w_gate"], None, yg)])
        acts.append((yu, yg, yd))
        work.append((x, plan, qs, yu, yg, yd))

    def step():
        for x, plan, qs, yu, yg, yd in work:
            aql.aql_linear_w8a16_grouped(*plan)
            aql.aql_linear_w8a16(yu, *qs["w_down"], None, yd)

    def check(what):
        for li, (x, plan, qs, yu, yg, yd) in enumerate(work):
            xb = bits(x)
            for y, wn, xin in ((yu, "w_up", xb), (yg, "w_gate", xb), (yd, "w_down", bits(yu))):
                yref, tol = oracle.linear_w8a16(xin, host(qs[wn][0]), host(qs[wn][1]))
                check_float(host(y.float()), yref, tol, BF16, f"{what} layer {li} {wn}")

    step()
    check("eager")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(2):
        for yu, yg, yd in acts:
            yu.fill_(float("nan"))
            yg.fill_(float("nan"))
            yd.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(f"graph replay {rep}")
