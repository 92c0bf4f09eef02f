#!/usr/bin/env python3
"""Benchmark of the INT8 quantized linear on one MI355X; prints one JSON line.

Headline (the metric's first half, on the SmolVLM-500M decode workload): one
step is a full 32-layer decode sweep of the text decoder's MLP linears, 96
W8A16 GEMVs (per layer up and gate [2560, 960], down [960, 2560], M = 1, bf16
activations, int8 per-channel weights). The weights were quantized on the GPU
beforehand (bind time, not timed). The layers' linears do not feed one
another, so a step is one grouped launch over all 96 (planned once per weight
copy). Three copies of the 32-layer weight set (712 MB, more than twice the
256 MB Infinity Cache) are rotated step by step so every step streams its
weights from HBM. value = algorithmic bytes of a sweep / time of a sweep, in
GB/s (weights N*K + fp32 scales 4N + bf16 x 2MK + bf16 y 2MN per GEMV). The
same sweep as 96 separate launches in a HIP graph is a secondary row.

Secondary rows (reported in "secondary"): the 7B-shape W8A16 GEMV/skinny GEMM
(M = 1, 4, 16), the W8A8 static two-pass linear (M = 512, K = N = 4096; the
metric's second half, TOPS against the int8 MFMA peak), the 8da4w dynamic
linear, and the weight quantizer. Each is timed with HIP events on the stream
the kernels run on, bracketing a run of back-to-back calls that rotates enough
weight copies to exceed the Infinity Cache (the short activation-quantizer
prologue of the W8A8 row is timed from replays of a HIP graph of such calls,
as its host overhead exceeds its GPU time).

Before the first timing, each run drives its workload back to back for ~50 ms
of GPU time (settle()): coming out of idle the GPU streams memory about 10%
slower for the first 10-20 ms of sustained load, and the figures here are
steady-state ones. Matrix-core rows (prefill GEMMs, W8A8, GPTQ) also run their
own call for ~40 ms right before they are timed: their clock ramps again under
their own load (an M = 2048 prefill call falls from ~285 to ~235 us over its
first ~30 ms).

cpu_baseline: the CPU oracle (test infrastructure; its only use here) timed on
the host on a bounded sample of the headline workload.
"""
import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W8A16 decode GEMV GB/s (% HBM peak); W8A8 prefill GEMM TOPS (% int8 MFMA)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP64_PEAK_TFLOPS = 78.6      # MI355X fp64 vector (fused multiply-add counted as 2)
MALL_BYTES = 256 << 20
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PROFILE = "k_w8a16_m1p_grouped_smolvlm_decode_sweep_traffic.md"
HEADLINE_SOURCES = ("activation_quantized_linear_amd/csrc/w8a16.hip",
                    "activation_quantized_linear_amd/csrc/w8a16.h",
                    "activation_quantized_linear_amd/csrc/common.h")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-secondary", action="store_true", help="headline only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's CPU time for cpu_baseline")
    ap.add_argument("--only", default=None,
                    help="run just one workload (sweep|chain|llm7b|q8ta|dq8ca|quant|calib|gptq|copy), or a "
                         "measurement outside the default run (wsweep: working-set sweep; oracle: "
                         "the CPU oracle at full size beside the GPU)")
    ap.add_argument("--no-settle", action="store_true",
                    help="profile helper: skip the settle phase (counter runs serialize every "
                         "dispatch, so settling there only costs time)")
    return ap.parse_args()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


_SETTLED = [False]


def event_time_ms(torch, fn, reps, rotate, trials=5, graph=False, warm_ms=0.0):
    """Per-call time (ms): HIP events on the current stream bracket `reps`
    back-to-back calls (rotating over `rotate` buffer sets); median of `trials`.
    Where the host keeps ahead of the GPU this is the GPU's time per call. For
    calls shorter than their host overhead, graph=True captures the `reps`
    calls once in a HIP graph and times its replays instead (each graph node
    costs a little launch time of its own, so the longer calls are timed
    eagerly). The first timing of a process is preceded by settle(); warm_ms
    > 0 runs fn itself that long first (matrix-core rows: their clock ramps
    over the first ~30 ms of their own load, whatever ran before)."""
    if not _SETTLED[0]:
        settle(torch, lambda i: fn(i % rotate))
        _SETTLED[0] = True
    if warm_ms > 0:
        settle(torch, lambda i: fn(i % rotate), warm_ms)
    g = None
    if graph:
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                fn(i % rotate)
        g.replay()
        torch.cuda.synchronize()
    res = []
    for _ in range(trials):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        if g is not None:
            g.replay()
        else:
            for i in range(reps):
                fn(i % rotate)
        b.record()
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) / reps)
    return statistics.median(res), res


_NO_SETTLE = [False]


def settle(torch, fn, gpu_ms=50.0):
    """Run fn back to back for about gpu_ms of GPU time before anything is
    warmed up or timed. Coming out of idle the GPU streams memory measurably
    slower for the first 10-20 ms of sustained load (kernel durations of the
    same launch fall by about 10% and then stay flat), so a run is brought to
    that steady state once, at setup, rather than inside the timed region."""
    if _NO_SETTLE[0]:
        return 0
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    done, i = 0.0, 0
    while done < gpu_ms:
        a.record()
        for _ in range(64):
            fn(i)
            i += 1
        b.record()
        torch.cuda.synchronize()
        done += a.elapsed_time(b)
    return i


def raw_call(aql, torch, name, argsets):
    """fn(i) calling the C entry point `name` directly with the i-th prebuilt
    ctypes argument tuple (device pointers, sizes, the current stream): the
    same launch as the binding's, without its per-call checks, so that for
    calls of ~10 us the host stays ahead of the GPU and events time the GPU."""
    import ctypes as C
    f = getattr(aql._lib, name)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)

    def conv(a):
        if a is None:
            return None
        if isinstance(a, torch.Tensor):
            return C.c_void_p(a.data_ptr())
        return a

    built = [tuple(conv(a) for a in args) + (st,) for args in argsets]
    return lambda i: f(*built[i])


def copies_for(nbytes, minimum=2):
    return max(minimum, -(-2 * MALL_BYTES // max(nbytes, 1)))


# --------------------------------------------------------------- headline


def sweep_workload(torch, aql, workloads, dev):
    layers = workloads.smolvlm(seed=0)
    base, xs = [], []
    for L in layers:
        e = {}
        for wn in ("w_up", "w_gate", "w_down"):
            q, s, _ = aql.aql_quantize_weight_int8(L[wn].to(dev), aql.AQL_WQ_SYM127)
            e[wn] = (q, s)
        xs.append((L["x_up"].to(dev), L["x_down"].to(dev)))
        base.append(e)
    torch.cuda.synchronize()
    copies = 3
    sets = [base] + [[{k: (v[0].clone(), v[1].clone()) for k, v in e.items()} for e in base]
                     for _ in range(copies - 1)]
    F, H = workloads.SMOLVLM_FFN, workloads.SMOLVLM_HIDDEN
    ys = [(torch.empty(1, F, dtype=torch.bfloat16, device=dev),
           torch.empty(1, F, dtype=torch.bfloat16, device=dev),
           torch.empty(1, H, dtype=torch.bfloat16, device=dev)) for _ in layers]
    calls = []
    for c in range(copies):
        cl = []
        for li, e in enumerate(sets[c]):
            xu, xd = xs[li]
            yu, yg, yd = ys[li]
            cl.append((xu, e["w_up"][0], e["w_up"][1], yu))
            cl.append((xu, e["w_gate"][0], e["w_gate"][1], yg))
            cl.append((xd, e["w_down"][0], e["w_down"][1], yd))
        calls.append(cl)

    def nbytes(x, q, y):
        M, K = x.shape
        N = q.shape[0]
        return N * K + 4 * N + 2 * M * K + 2 * M * N

    step_bytes = sum(nbytes(x, q, y) for x, q, s, y in calls[0])
    return calls, step_bytes, nbytes, layers


def run_sweep(torch, aql, dev, args, calls, step_bytes):
    """Headline: each step is one grouped launch over the 96 GEMVs of one weight
    copy; the timed region is bracketed by HIP events on the launch stream, so
    its average is the grouped kernel's average launch duration."""
    plans = [aql.aql_w8a16_group_plan([(x, q, s, None, y) for x, q, s, y in cl]) for cl in calls]
    for h, d in plans:
        aql.aql_linear_w8a16_grouped(h, d)
    settle(torch, lambda i: aql.aql_linear_w8a16_grouped(*plans[i % len(plans)]))
    _SETTLED[0] = True
    for i in range(args.warmup):
        h, d = plans[i % len(plans)]
        aql.aql_linear_w8a16_grouped(h, d)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    t0 = time.perf_counter()
    for i in range(args.steps):
        h, d = plans[i % len(plans)]
        aql.aql_linear_w8a16_grouped(h, d)
    t1 = time.perf_counter()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    say(f"sweep (grouped): {ms * 1e3:.1f} us/step, {step_bytes / (ms * 1e-3) / 1e9:.1f} GB/s; "
        f"host submit {(t1 - t0) / args.steps * 1e6:.1f} us/step")
    return ms


def sweep_as_graph(torch, aql, calls, step_bytes, reps=60):
    """Secondary row: the same sweep as 96 separate launches captured in a HIP graph."""
    def sweep(cl):
        for x, q, s, y in cl:
            aql.aql_linear_w8a16(x, q, s, None, y)

    for cl in calls:
        sweep(cl)
    torch.cuda.synchronize()
    graphs = []
    for cl in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sweep(cl)
        graphs.append(g)
    med, _ = event_time_ms(torch, lambda i: graphs[i].replay(), reps, len(graphs))
    row = {"workload": "smolvlm500m_decode_sweep as 96 W8A16 launches in a HIP graph",
           "us": med * 1e3, "GB/s": step_bytes / (med * 1e-3) / 1e9,
           "frac_hbm": step_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS}
    say(row)
    return row


def sec_decode_chain(torch, aql, workloads, dev, copies=3):
    """Secondary row: the decode sweep with the dependencies of a real decode
    step (flashrt schemes, W8A16Decode on a decoder_ffn seam). Per layer one
    grouped launch computes up and gate from the same x, then down reads up's
    output (the gated activation between them is not part of the quantized
    linear and is left out: down reads the up projection as it is), and the
    next layer reads down's output. 64 launches per step over the same 237 MB
    of weights as the headline; 3 weight copies rotate. Timed eagerly and as
    one HIP graph per copy."""
    layers = workloads.smolvlm(seed=0)
    F, H = workloads.SMOLVLM_FFN, workloads.SMOLVLM_HIDDEN
    base = []
    for L in layers:
        e = {}
        for wn in ("w_up", "w_gate", "w_down"):
            q, s, _ = aql.aql_quantize_weight_int8(L[wn].to(dev), aql.AQL_WQ_SYM127)
            e[wn] = (q, s)
        base.append(e)
    sets = [base] + [[{k: (v[0].clone(), v[1].clone()) for k, v in e.items()} for e in base]
                     for _ in range(copies - 1)]
    x0 = layers[0]["x_up"].to(dev)
    acts = [(torch.empty(1, F, dtype=torch.bfloat16, device=dev),
             torch.empty(1, F, dtype=torch.bfloat16, device=dev),
             torch.empty(1, H, dtype=torch.bfloat16, device=dev)) for _ in layers]
    steps = []
    for c in range(copies):
        st = []
        for li, e in enumerate(sets[c]):
            x = x0 if li == 0 else acts[li - 1][2]
            yu, yg, yd = acts[li]
            plan = aql.aql_w8a16_group_plan([(x, e["w_up"][0], e["w_up"][1], None, yu),
                                             (x, e["w_gate"][0], e["w_gate"][1], None, yg)])
            st.append((plan, yu, e["w_down"][0], e["w_down"][1], yd))
        steps.append(st)
    del layers

    def step(i):
        for plan, yu, qd, sd, yd in steps[i]:
            aql.aql_linear_w8a16_grouped(*plan)
            aql.aql_linear_w8a16(yu, qd, sd, None, yd)

    step_bytes = 32 * (2 * (F * H + 4 * F + 2 * H + 2 * F) + (H * F + 4 * H + 2 * F + 2 * H))
    for i in range(copies):
        step(i)
    eager, _ = event_time_ms(torch, step, 20, copies)
    med, _ = event_time_ms(torch, step, 20, copies, graph=True)
    rows = []
    for how, ms in (("eager", eager), ("HIP graph", med)):
        gbs = step_bytes / (ms * 1e-3) / 1e9
        rows.append({"workload": f"smolvlm500m decode step with dependencies, {how}: 32 x (grouped "
                                 f"up+gate sharing x, then down on up's output), 64 launches",
                     "us": ms * 1e3, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                     "us_per_launch": ms * 1e3 / 64})
        say(rows[-1])
    return rows


# -------------------------------------------------------------- secondary


def sec_llm7b(torch, aql, workloads, dev):
    rows = []
    for K, N in workloads.LLM7B_SHAPES:
        d = workloads.llm7b(K, N, 1, seed=2)
        q, s, _ = aql.aql_quantize_weight_int8(d["w"].to(dev), aql.AQL_WQ_SYM127)
        del d
        ncopy = copies_for(N * K)
        qs = [q] + [q.clone() for _ in range(ncopy - 1)]
        for M in (1, 4, 16, 512, 2048):
            x = workloads.llm7b(K, 16, M, seed=3)["x"].to(dev)
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            nws = aql.aql_workspace_bytes(aql.AQL_OP_W8A16, M, N, K)
            wsb = torch.empty(nws, dtype=torch.uint8, device=dev) if nws > 0 else None
            fn = lambda i: aql.aql_linear_w8a16(x, qs[i], s, None, y, workspace=wsb)
            for i in range(ncopy):
                fn(i)
            if M <= 16:  # short calls: the C entry point with prebuilt arguments
                fn = raw_call(aql, torch, "aql_linear_w8a16",
                              [(x, M, K, qs[i], s, None, N, y, wsb, nws) for i in range(ncopy)])
            med, _ = event_time_ms(torch, fn, 50 if M <= 16 else 10, ncopy,
                                   warm_ms=0.0 if M <= 16 else 40.0)
            nb = N * K + 4 * N + 2 * M * K + 2 * M * N
            gbs = nb / (med * 1e-3) / 1e9
            tf = 2 * M * N * K / (med * 1e-3) / 1e12
            row = {"workload": f"llm7b_w8a16 K={K} N={N} M={M}", "us": med * 1e3,
                   "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "TFLOP/s": tf}
            if M > 16:  # prefill: the tiled bf16-MFMA GEMM
                row["frac_bf16"] = tf / BF16_PEAK_TFLOPS
            rows.append(row)
            say(rows[-1])
        del qs, q
    return rows


def sec_q8ta(torch, aql, workloads, dev):
    d = workloads.two_pass(seed=0)
    x = d["x"].to(dev)
    calib = d["x"][d["calib_rows"]].reshape(1, -1).contiguous().to(dev)
    sc, zc, _ = aql.aql_choose_qparams_rows(calib, quantize=False)
    s1, z1 = float(sc.item()), int(zc.item())
    import numpy as np
    s2 = float(np.float32(s1) / np.float32(255.0))
    q, ws, wsum = aql.aql_quantize_weight_int8(d["w"].to(dev), aql.AQL_WQ_SYM127_5)
    M, K = x.shape
    N = q.shape[0]
    ncopy = copies_for(N * K + 8 * N)
    qs = [(q, ws, wsum)] + [(q.clone(), ws.clone(), wsum.clone()) for _ in range(ncopy - 1)]
    y = torch.empty(M, N, dtype=torch.float32, device=dev)
    wsb = torch.empty(aql.aql_workspace_bytes(aql.AQL_OP_Q8TA_Q8CSW, M, N, K), dtype=torch.uint8,
                      device=dev)
    xq1 = torch.empty(M, K, dtype=torch.int8, device=dev)
    xq2 = torch.empty(M, K, dtype=torch.int8, device=dev)
    rows = []
    for two in (True, False):
        fn = lambda i: aql.aql_linear_q8ta_q8csw(x, s1, z1, qs[i][0], qs[i][2], qs[i][1], None,
                                                 two, s2, 0, y, wsb)
        for i in range(ncopy):
            fn(i)
        fn = raw_call(aql, torch, "aql_linear_q8ta_q8csw",
                      [(x, M, K, s1, z1, int(two), s2, 0, qs[i][0], qs[i][2], qs[i][1], None, N,
                        y, wsb, wsb.numel()) for i in range(ncopy)])
        med, _ = event_time_ms(torch, fn, 40, ncopy, warm_ms=40.0)
        pro = lambda i: aql.aql_quantize_act_per_tensor(x, s1, z1, two, s2, 0, xq1, xq2)
        pmed, _ = event_time_ms(torch, pro, 40, 1, graph=True)
        ops = (2 if two else 1) * 2 * M * N * K
        nb = 4 * M * K + N * K + 8 * N + 4 * M * N
        gemm_ms = max(med - pmed, 1e-6)
        rows.append({"workload": f"w8a8_q8ta {'two' if two else 'one'}-pass M={M} K={K} N={N}",
                     "us": med * 1e3, "prologue_us": pmed * 1e3,
                     "TOPS": ops / (med * 1e-3) / 1e12,
                     "frac_int8": ops / (med * 1e-3) / 1e12 / INT8_PEAK_TOPS,
                     "gemm_TOPS_est": ops / (gemm_ms * 1e-3) / 1e12,
                     "GB/s": nb / (med * 1e-3) / 1e9})
        say(rows[-1])
    return rows


def sec_dq8ca(torch, aql, workloads, dev):
    rows = []
    d = workloads.dyn8da4w(4, seed=0)
    q4, gs, gsum = aql.aql_quantize_weight_q4gsw(d["w"].to(dev), 32)
    N, K = q4.shape[0], q4.shape[1] * 2
    wbytes = q4.numel() + 8 * gs.numel()
    ncopy = copies_for(wbytes)
    ws = [(q4, gs, gsum)] + [(q4.clone(), gs.clone(), gsum.clone()) for _ in range(ncopy - 1)]
    for M in workloads.DYN_MS:
        x = workloads.dyn8da4w(M, seed=1, N=16)["x"].to(dev)
        y = torch.empty(M, N, dtype=torch.float32, device=dev)
        wsb = torch.empty(aql.aql_workspace_bytes(aql.AQL_OP_DQ8CA, M, N, K), dtype=torch.uint8,
                          device=dev)
        fn = lambda i: aql.aql_linear_dq8ca(x, ws[i][0], ws[i][1], ws[i][2], aql.AQL_W_Q4GSW, 32,
                                            None, y, workspace=wsb)
        for i in range(ncopy):
            fn(i)
        if M <= 16:  # short calls: the C entry point with prebuilt arguments
            fn = raw_call(aql, torch, "aql_linear_dq8ca",
                          [(x, M, K, aql.AQL_W_Q4GSW, ws[i][0], ws[i][1], ws[i][2], 32, None, N,
                            y, None, None, wsb, wsb.numel()) for i in range(ncopy)])
        med, _ = event_time_ms(torch, fn, 20 if M > 1000 else 40, ncopy,
                               warm_ms=40.0 if M > 16 else 0.0)
        ops = 2 * M * N * K
        nb = N * K // 2 + 4 * gs.numel() + 4 * M * K + 4 * M * N + 8 * M
        rows.append({"workload": f"dq8ca_8da4w M={M} K={K} N={N}", "us": med * 1e3,
                     "GB/s": nb / (med * 1e-3) / 1e9, "frac_hbm": nb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "TOPS": ops / (med * 1e-3) / 1e12,
                     "frac_int8": ops / (med * 1e-3) / 1e12 / INT8_PEAK_TOPS})
        say(rows[-1])
    return rows


def sec_quant(torch, aql, workloads, dev):
    K, N = 4096, 14336
    w = workloads.llm7b(K, N, 1, seed=5)["w"].to(dev)
    q = torch.empty(N, K, dtype=torch.int8, device=dev)
    s = torch.empty(N, dtype=torch.float32, device=dev)
    wsum = torch.empty(N, dtype=torch.int32, device=dev)
    fn = lambda i: aql.aql_quantize_weight_int8(w, aql.AQL_WQ_SYM127, q, s, wsum)
    fn(0)
    med, _ = event_time_ms(torch, fn, 20, 1)
    nb = 4 * N * K + N * K + 8 * N
    row = {"workload": f"quantize_weight_int8 fp32 N={N} K={K}", "us": med * 1e3,
           "GB/s": nb / (med * 1e-3) / 1e9, "frac_hbm": nb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS}
    say(row)
    return [row]


def sec_calib(torch, aql, workloads, dev):
    """Static calibration: one observer call over a batch of 4096 rows of the
    W8A8 workload's width, plain and residual (the two-pass second run)."""
    rows, cols = 4096, 4096
    ncopy = copies_for(4 * rows * cols)
    g = workloads.gen(77)
    xs = [workloads.small_matrix(g, rows, cols, std=4.0).to(dev) for _ in range(ncopy)]
    st = aql.aql_minmax_state(dev)
    out = []
    for residual in (None, (0.05, 3)):
        fn = lambda i: aql.aql_minmax_observe(xs[i], st, residual=residual)
        for i in range(ncopy):
            fn(i)
        med, _ = event_time_ms(torch, fn, 40, ncopy)
        nb = 4 * rows * cols
        row = {"workload": f"calibration observe{' residual' if residual else ''} fp32 "
                           f"{rows}x{cols}", "us": med * 1e3, "GB/s": nb / (med * 1e-3) / 1e9,
               "frac_hbm": nb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS}
        say(row)
        out.append(row)
    return out


def gptq_flops(N, K, block):
    """Algorithmic fp64 operations of GPTQ int8 (one multiply and one add per
    term): the two Cholesky factors, the triangular inverse and the product
    forming H^-1 (K^3/3 each), and the column loop (per row: the block's
    in-block updates and every block's trailing update)."""
    fact = 4.0 * K ** 3 / 3.0
    loop = 0.0
    for i1 in range(0, K, block):
        bl = min(block, K - i1)
        loop += bl * (bl - 1) / 2.0 + bl * (K - i1 - bl)
    return fact + 2.0 * N * loop


def sec_gptq(torch, aql, workloads, dev):
    """GPTQ int8 (binary64, bit-exact with the oracle) of a SmolVLM-500M MLP on
    a synthetic Hessian: up and gate share their input, so they run as one
    call on [5120, 960]; down is [960, 2560]. Plus a 4096 x 4096 layer."""
    out = []
    for name, K, N in (("smolvlm up+gate", 960, 5120), ("smolvlm down", 2560, 960),
                       ("4096x4096", 4096, 4096)):
        d = workloads.gptq(K, N, seed=9)
        w = d["w"].to(dev)
        H = torch.from_numpy(d["H"]).to(dev)
        ws = torch.empty(aql.aql_workspace_bytes(aql.AQL_OP_GPTQ_INT8, 128, N, K),
                         dtype=torch.uint8, device=dev)
        q = torch.empty(N, K, dtype=torch.int8, device=dev)
        s = torch.empty(N, dtype=torch.float32, device=dev)
        wsum = torch.empty(N, dtype=torch.int32, device=dev)
        info = torch.empty(1, dtype=torch.int32, device=dev)
        fn = lambda i: aql.aql_gptq_int8(w, H, 0.01, 128, q, s, wsum, False, info, ws)
        fn(0)
        torch.cuda.synchronize()
        if int(info.cpu()[0]) != 0:
            raise RuntimeError(f"gptq {name}: info {int(info.cpu()[0])}")
        med, _ = event_time_ms(torch, fn, 3, 1, trials=3, warm_ms=40.0)
        fl = gptq_flops(N, K, 128)
        row = {"workload": f"gptq_int8 {name} K={K} N={N} block=128 (fp64)", "ms": med,
               "TFLOP/s": fl / (med * 1e-3) / 1e12,
               "frac_fp64": fl / (med * 1e-3) / 1e12 / FP64_PEAK_TFLOPS}
        say(row)
        out.append(row)
        del ws, w, H
        torch.cuda.empty_cache()
    return out


def sec_wsweep(torch, aql, workloads, dev):
    """Working-set sweep (not part of the default run): the 7B M = 1 GEMV
    (K=4096, N=14336, 58.7 MB of weights a call) rotated over 1 .. 12 weight
    copies, and the SmolVLM sweep (237 MB a grouped launch) over 1 .. 4 copies.
    Once a timed repetition touches more than the 256 MB Infinity Cache the
    rate stops depending on the copy count: that plateau is the HBM rate."""
    rows = []
    K, N = 4096, 14336
    d = workloads.llm7b(K, N, 1, seed=2)
    q, s, _ = aql.aql_quantize_weight_int8(d["w"].to(dev), aql.AQL_WQ_SYM127)
    x = d["x"].to(dev)
    y = torch.empty(1, N, dtype=torch.bfloat16, device=dev)
    qs = [q] + [q.clone() for _ in range(11)]
    nb = N * K + 4 * N + 2 * K + 2 * N
    for c in (1, 2, 3, 4, 6, 8, 12):
        fn = lambda i: aql.aql_linear_w8a16(x, qs[i % c], s, None, y)
        med, _ = event_time_ms(torch, fn, 120, c)
        row = {"workload": f"llm7b_w8a16 K={K} N={N} M=1, {c} copies", "working_set_MB": c * nb / 1e6,
               "us": med * 1e3, "GB/s": nb / (med * 1e-3) / 1e9}
        say(row)
        rows.append(row)
    del qs, q
    torch.cuda.empty_cache()
    layers = workloads.smolvlm(seed=0)
    base, xs = [], []
    for L in layers:
        for wn, xn in (("w_up", "x_up"), ("w_gate", "x_up"), ("w_down", "x_down")):
            qq, ss, _ = aql.aql_quantize_weight_int8(L[wn].to(dev), aql.AQL_WQ_SYM127)
            xx = L[xn].to(dev)
            base.append((xx, qq, ss, torch.empty(1, qq.shape[0], dtype=torch.bfloat16, device=dev)))
    del layers
    step = sum(qq.numel() + 4 * qq.shape[0] + 2 * xx.numel() + 2 * qq.shape[0]
               for xx, qq, ss, _ in base)
    sets = [base] + [[(xx, qq.clone(), ss, yy) for xx, qq, ss, yy in base] for _ in range(3)]
    plans = [aql.aql_w8a16_group_plan([(xx, qq, ss, None, yy) for xx, qq, ss, yy in st])
             for st in sets]
    for c in (1, 2, 3, 4):
        fn = lambda i: aql.aql_linear_w8a16_grouped(*plans[i % c])
        med, _ = event_time_ms(torch, fn, 200, c)
        row = {"workload": f"smolvlm500m_decode_sweep, {c} copies", "working_set_MB": c * step / 1e6,
               "us": med * 1e3, "GB/s": step / (med * 1e-3) / 1e9}
        say(row)
        rows.append(row)
    return rows


def sec_oracle(torch, aql, workloads, dev):
    """Oracle timing (not part of the default run): the CPU oracle at full size
    on each workload, OpenMP over all host cores, median of 3 (one run where a
    single run takes over 10 s), and one run on a single thread (skipped for
    8da4w M=2048, about 90 s); beside it the GPU time of the same call on one
    weight buffer (so the weights may sit in the Infinity Cache: the bench rows
    give the HBM rates)."""
    import numpy as np

    import oracle

    def cpu_ms(fn, reps=3):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append((time.perf_counter() - t0) * 1e3)
            if ts[-1] > 10e3:
                break
        return statistics.median(ts)

    def gpu_us(fn):
        fn(0)
        med, _ = event_time_ms(torch, fn, 20, 1, trials=3)
        return med * 1e3

    rows = []

    def one_thread_ms(fn):
        oracle.set_threads(1)
        try:
            return cpu_ms(fn, reps=1)
        finally:
            oracle.set_threads(None)

    def add(name, fn, g_us, outputs, single=True):
        # outputs: the (row, channel) outputs the oracle's linears split over threads
        o_ms = cpu_ms(fn)
        row = {"workload": name, "oracle_ms": o_ms, "gpu_us": g_us, "ratio": o_ms * 1e3 / g_us,
               "cores": oracle.threads(), "threads_working": min(oracle.threads(), outputs),
               "oracle_ms_1_thread": one_thread_ms(fn) if single else None}
        say(row)
        rows.append(row)

    t = workloads.tiny()
    wq, ws, _ = oracle.quantize_weight_int8(t["w"].numpy(), 0)
    xb = workloads.bf16_bits(t["x"])
    wdv = t["w"].to(dev)
    qd, sd, _ = aql.aql_quantize_weight_int8(wdv, aql.AQL_WQ_SYM127)
    xdv = t["x"].to(dev)
    add("c1 tiny quantize + GEMV", lambda: (oracle.quantize_weight_int8(t["w"].numpy(), 0),
                                            oracle.linear_w8a16(xb, wq, ws)),
        gpu_us(lambda i: (aql.aql_quantize_weight_int8(wdv, aql.AQL_WQ_SYM127, qd, sd),
                          aql.aql_linear_w8a16(xdv, qd, sd))), 256)
    for K, N in workloads.LLM7B_SHAPES:
        d = workloads.llm7b(K, N, 16, seed=2)
        q, s, _ = oracle.quantize_weight_int8(d["w"].numpy(), 0)
        qg, sg, _ = aql.aql_quantize_weight_int8(d["w"].to(dev), aql.AQL_WQ_SYM127)
        for M in (1, 4, 16):
            xm = d["x"][:M]
            xbits = workloads.bf16_bits(xm)
            xg = xm.to(dev)
            add(f"c3 7B W8A16 K={K} N={N} M={M}", lambda: oracle.linear_w8a16(xbits, q, s),
                gpu_us(lambda i: aql.aql_linear_w8a16(xg, qg, sg)), M * N)
        del d, qg
    tp = workloads.two_pass(seed=0)
    xnp = tp["x"].numpy()
    s1, z1, _ = oracle.choose_qparams_rows(np.ascontiguousarray(xnp[1:].reshape(1, -1)),
                                           quantize=False)
    s1, z1 = float(s1[0]), int(z1[0])
    s2 = float(np.float32(s1) / np.float32(255.0))
    q, ws8, wsum = oracle.quantize_weight_int8(tp["w"].numpy(), 1)
    qg, wsg, wsumg = aql.aql_quantize_weight_int8(tp["w"].to(dev), aql.AQL_WQ_SYM127_5)
    xg = tp["x"].to(dev)
    add("c4 W8A8 two-pass M=512 K=N=4096",
        lambda: oracle.linear_q8ta_q8csw(xnp, s1, z1, q, ws8, two_pass=True, s2=s2, z2=0),
        gpu_us(lambda i: aql.aql_linear_q8ta_q8csw(xg, s1, z1, qg, wsumg, wsg, two_pass=True, s2=s2,
                                                   z2=0)), 512 * 4096)
    del tp, qg, xg
    w = workloads.dyn8da4w(4, seed=1)["w"]
    q4, gs, _ = oracle.quantize_weight_q4gsw(w.numpy())
    q4g, gsg, gsumg = aql.aql_quantize_weight_q4gsw(w.to(dev))
    del w
    for M in (4, 128, 2048):
        x = workloads.dyn8da4w(M, seed=2)["x"]
        xn = x.numpy()
        xg = x.to(dev)
        add(f"c5 8da4w M={M} K=4096 N=11008",
            lambda: oracle.linear_dq8ca(xn, q4, gs, wfmt=oracle.W_Q4GSW, group=32),
            gpu_us(lambda i: aql.aql_linear_dq8ca(xg, q4g, gsg, gsumg, wfmt=aql.AQL_W_Q4GSW,
                                                  group=32)),
            M * 11008, single=M < 2048)
    return rows


# ------------------------------------------------------------- CPU baseline


def cpu_baseline(layers, seconds):
    import numpy as np

    import oracle
    import workloads

    prepared = []
    for L in layers:
        for wn, xn in (("w_up", "x_up"), ("w_gate", "x_up"), ("w_down", "x_down")):
            q, s, _ = oracle.quantize_weight_int8(L[wn].numpy(), 0)
            prepared.append((workloads.bf16_bits(L[xn]), q, s))
    done_b, t0, gemvs = 0, time.perf_counter(), 0
    while True:
        for x, q, s in prepared:
            oracle.linear_w8a16(x, q, s)
            M, K = x.shape
            N = q.shape[0]
            done_b += N * K + 4 * N + 2 * M * K + 2 * M * N
            gemvs += 1
            if time.perf_counter() - t0 >= seconds:
                break
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    # the oracle's OpenMP loops split the (row, channel) outputs over threads:
    # a decode GEMV's 960 or 2560 channels keep every thread busy
    return {"value": done_b / el / 1e9, "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{gemvs} of the decode sweep's W8A16 GEMVs (in sweep order, fp64 sums), "
                      f"{el:.1f} s on the host, outputs split over {oracle.threads()} threads"}


def sec_copy(torch, aql, workloads, dev, mib=256, reps=20):
    """Reference row: a plain device-to-device copy of `mib` MiB (torch copy_),
    the known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters."""
    n = mib << 20
    src = torch.full((n,), 7, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    med, _ = event_time_ms(torch, lambda i: dst.copy_(src), reps, 1)
    return [{"workload": f"device copy {mib} MiB (torch copy_)", "us": med * 1e3,
             "bytes_read": n, "bytes_written": n, "GB/s": 2 * n / (med * 1e-3) / 1e9}]


def ceilings(torch, aql, dev):
    """Attainable ceilings on this GPU, measured in the same run: a read-only
    HBM stream (two 512 MiB buffers rotated, so no read hits the 256 MB
    Infinity Cache), the same stream in launches of one 7B weight matrix
    (56 MiB = 14336 x 4096 int8, ten buffers rotated), and back-to-back int8
    MFMAs on all CUs."""
    n = 512 << 20
    bufs = [torch.full((n,), 1, dtype=torch.uint8, device=dev) for _ in range(2)]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    rd_ms, _ = event_time_ms(torch, lambda i: aql.aql_measure_read(bufs[i], sink), 10, 2)
    del bufs
    n7 = 56 << 20
    bufs = [torch.full((n7,), 1, dtype=torch.uint8, device=dev) for _ in range(10)]
    rd7 = raw_call(aql, torch, "aql_measure_read", [(b, n7, sink) for b in bufs])
    rd7_ms, _ = event_time_ms(torch, rd7, 50, 10)
    del bufs
    rd7 = n7 / (rd7_ms * 1e-3) / 1e9
    iters = 20000
    ops = 2048 * 32768 * 16 * iters
    mf_ms, _ = event_time_ms(torch, lambda i: aql.aql_measure_mfma_i8(iters, sink), 3, 1)
    rd = n / (rd_ms * 1e-3) / 1e9
    tops = ops / (mf_ms * 1e-3) / 1e12
    out = {"hbm_read_GBs": rd, "hbm_read_frac": rd / HBM_PEAK_GBS,
           "hbm_read_56MiB_launch_GBs": rd7, "hbm_read_56MiB_launch_frac": rd7 / HBM_PEAK_GBS,
           "mfma_i8_TOPS": tops, "mfma_i8_frac": tops / INT8_PEAK_TOPS,
           "how": "aql_measure_read over 512 MiB (2 buffers rotated) and over 56 MiB "
                  "(10 buffers rotated); aql_measure_mfma_i8 (2048 waves x 16 x 20000 MFMAs)"}
    say(out)
    return out


def sources_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(name, sources):
    """HBM bytes per launch of the headline kernel as measured by the FETCH_SIZE /
    WRITE_SIZE counter runs summarized in profiles/<name> (each scaled by the
    same counter on a plain copy of known size). The summary records a digest
    of the kernel's sources; if they have changed since, the figure no longer
    describes this kernel and None is returned."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        text = open(path).read()
    except OSError:
        return None
    m_b = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    m_d = re.search(r"^sources_sha256_16:\s*([0-9a-f]+)", text, re.M)
    if not (m_b and m_d) or m_d.group(1) != sources_digest(sources):
        return None
    return int(m_b.group(1))


def main():
    args = parse()
    _NO_SETTLE[0] = args.no_settle
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures a single GPU (got --gpus {args.gpus}, WORLD_SIZE {world}): the "
              "quantized linear here runs on one MI355X, and no multi-GPU figure is produced.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    import activation_quantized_linear_amd as aql
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    say(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    secondary = []
    if args.only is not None and args.only != "sweep":
        fn = {"llm7b": sec_llm7b, "q8ta": sec_q8ta, "dq8ca": sec_dq8ca, "quant": sec_quant,
              "chain": sec_decode_chain,
              "calib": sec_calib, "copy": sec_copy, "gptq": sec_gptq, "wsweep": sec_wsweep,
              "oracle": sec_oracle}[args.only]
        print(json.dumps({"only": args.only, "rows": fn(torch, aql, workloads, dev)}), flush=True)
        return
    calls, step_bytes, nbytes, layers = sweep_workload(torch, aql, workloads, dev)
    ms = run_sweep(torch, aql, dev, args, calls, step_bytes)
    if args.only is None and not args.no_secondary:
        secondary.append(sweep_as_graph(torch, aql, calls, step_bytes))
    del calls
    torch.cuda.empty_cache()
    if args.only is None and not args.no_secondary:
        secondary += sec_decode_chain(torch, aql, workloads, dev)
    torch.cuda.empty_cache()
    if args.only is None and not args.no_secondary:
        for fn in (sec_llm7b, sec_q8ta, sec_dq8ca, sec_quant, sec_calib, sec_gptq):
            secondary += fn(torch, aql, workloads, dev)
            torch.cuda.empty_cache()

    ceil = None
    if args.only is None and not args.no_secondary:
        ceil = ceilings(torch, aql, dev)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        say("cpu baseline ...")
        cpu = cpu_baseline(layers, args.cpu_seconds)

    value = step_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "smolvlm500m_decode_sweep: 32 layers x (up 2560x960, gate 2560x960, "
                        "down 960x2560) W8A16 GEMVs, M=1, bf16 x, int8 per-channel weights, "
                        "one grouped launch per sweep, 3 rotated weight copies (712 MB)",
            "gemvs_per_step": 96,
            "bytes_per_step": step_bytes,
            "frac_hbm": value / HBM_PEAK_GBS,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": value,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": value / HBM_PEAK_GBS,
            "traffic": traffic_from_profile(TRAFFIC_PROFILE, HEADLINE_SOURCES),
            "kernel": "k_w8a16_m1p_grouped",
            "bytes_per_launch": step_bytes,
            "avg_launch_us": ms * 1e3,
            "launches_timed": args.steps,
        },
        "cpu_baseline": cpu,
        "ceilings": ceil,
        "secondary": secondary,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
