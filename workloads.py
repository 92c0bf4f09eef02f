"""Seeded synthetic inputs for the quantized-linear workloads.

Shared by the tests, the benchmark and the smoke check, and by both sides of
every parity check (the HIP library and the CPU oracle), so that both consume
the same bytes. This module only draws random numbers and lays them out: it
holds none of the quantized linear's arithmetic (no scales, no rounding, no
calibration).

Recipe: every tensor comes from torch.Generator('cpu').manual_seed(seed) and
torch.randn / torch.rand / torch.randperm, drawn in the order written below;
bf16 activations are torch's round-to-nearest-even cast of fp32 draws. Shapes
and distributions follow the decoder layers the pages quantize:
  * tiny:       W 256x256 ~ N(0, 0.02) with row 7 all zero, x 1x256 ~ N(0, 1).
  * smolvlm:    SmolVLM-500M text decoder MLP, per layer up/gate W [2560, 960]
                and down W [960, 2560] ~ N(0, 0.02), 1% of the rows of each
                matrix (chosen by randperm) scaled by 8; decode x [1, K] ~ N(0, 1).
  * llm7b:      7B-class MLP shapes (K, N) = (4096, 14336) and (14336, 4096),
                W ~ N(0, 0.02), x [M, K] ~ N(0, 1).
  * two_pass:   x [512, 4096] ~ N(0, 4^2) whose row 0 carries the massive
                activations of an attention-sink position (8 channels at
                +-U(2500, 3500), random sign); W [4096, 4096] ~ N(0, 0.02);
                rows 1..511 are the calibration rows.
  * dyn8da4w:   x [M, 4096] ~ N(0, 1), W [11008, 4096] ~ N(0, 0.02).
  * gptq:       a SmolVLM-500M MLP weight W [N, K] ~ N(0, 0.02) with 1% outlier
                rows, and a synthetic symmetric positive (semi)definite K x K
                float64 matrix standing in for the Hessian of the layer's
                calibration inputs: the Gram matrix Z^T Z of Z [S, K] whose
                columns have log-uniform scales in [0.1, 10] and share 16
                random latent factors (so the matrix is far from diagonal), with
                chosen columns of Z set to zero (dead channels).
"""
import numpy as np
import torch


def gen(seed):
    return torch.Generator("cpu").manual_seed(int(seed))


def bf16_bits(t):
    """torch bfloat16 tensor -> numpy uint16 bit patterns (same bytes)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def randn(g, *shape, std=1.0):
    return torch.randn(*shape, generator=g, dtype=torch.float32) * std


def tiny(seed=0):
    """256x256 weight with one all-zero row, one bf16 decode row."""
    g = gen(seed)
    w = randn(g, 256, 256, std=0.02)
    w[7, :] = 0.0
    x = randn(g, 1, 256).to(torch.bfloat16)
    return {"w": w, "x": x}


def outlier_rows(g, w, frac=0.01, factor=8.0):
    """Scale floor(frac * N) randomly chosen rows of w by `factor` in place."""
    n = w.shape[0]
    k = int(frac * n)
    idx = torch.randperm(n, generator=g)[:k]
    w[idx] *= factor
    return idx


SMOLVLM_HIDDEN = 960
SMOLVLM_FFN = 2560
SMOLVLM_LAYERS = 32


def smolvlm_layer(g):
    """One SmolVLM-500M text-decoder MLP: up, gate [2560, 960], down [960, 2560]."""
    H, F = SMOLVLM_HIDDEN, SMOLVLM_FFN
    w_up = randn(g, F, H, std=0.02)
    outlier_rows(g, w_up)
    w_gate = randn(g, F, H, std=0.02)
    outlier_rows(g, w_gate)
    w_down = randn(g, H, F, std=0.02)
    outlier_rows(g, w_down)
    x_up = randn(g, 1, H).to(torch.bfloat16)
    x_down = randn(g, 1, F).to(torch.bfloat16)
    return {"w_up": w_up, "w_gate": w_gate, "w_down": w_down, "x_up": x_up, "x_down": x_down}


def smolvlm(seed=0, layers=SMOLVLM_LAYERS):
    """`layers` independent decoder MLPs (the 32-layer decode sweep)."""
    g = gen(seed)
    return [smolvlm_layer(g) for _ in range(layers)]


LLM7B_SHAPES = ((4096, 14336), (14336, 4096))  # (K, N)


def llm7b(K, N, M, seed=0):
    g = gen(seed)
    w = randn(g, N, K, std=0.02)
    x = randn(g, M, K).to(torch.bfloat16)
    return {"w": w, "x": x}


def two_pass(seed=0, M=512, K=4096, N=4096, n_outliers=8):
    """Static-activation workload with an attention-sink outlier row 0."""
    g = gen(seed)
    x = randn(g, M, K, std=4.0)
    n_outliers = min(n_outliers, K)
    ch = torch.randperm(K, generator=g)[:n_outliers]
    mag = 2500.0 + 1000.0 * torch.rand(n_outliers, generator=g)
    sign = torch.where(torch.rand(n_outliers, generator=g) < 0.5, -1.0, 1.0)
    x[0, ch] = sign * mag
    w = randn(g, N, K, std=0.02)
    return {"x": x, "w": w, "calib_rows": slice(1, M), "outlier_channels": ch}


DYN_K = 4096
DYN_N = 11008
DYN_MS = (4, 128, 2048)


def dyn8da4w(M, seed=0, K=DYN_K, N=DYN_N):
    g = gen(seed)
    x = randn(g, M, K)
    w = randn(g, N, K, std=0.02)
    return {"x": x, "w": w}


def small_matrix(g, rows, cols, std=1.0):
    return randn(g, rows, cols, std=std)


def gptq(K, N, samples=None, seed=0, dead=()):
    """Weight [N, K] float32 and a synthetic Hessian stand-in [K, K] float64."""
    g = gen(seed)
    w = randn(g, N, K, std=0.02)
    outlier_rows(g, w)
    S = samples if samples is not None else 2 * K
    scale = torch.exp(torch.empty(K).uniform_(np.log(0.1), np.log(10.0), generator=g))
    factors = randn(g, S, 16) @ randn(g, 16, K)
    z = (randn(g, S, K) + 0.5 * factors) * scale
    z = z.double()
    for d in dead:
        z[:, d] = 0.0
    H = (z.T @ z).numpy()
    return {"w": w, "H": np.ascontiguousarray(H)}
