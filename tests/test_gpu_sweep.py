"""Seeded sweep of random shapes against the oracle, across every launch path of the forward.

Each case draws a token count from one of five bands (one to four tokens: the one-kernel
quantize-and-multiply step; five to sixteen: the int8 GEMV; 17 to 96: 64-token GEMM tiles split
over K; 97 to 700: 64- or 128-token tiles; 2000 to 2600: the 512-row tiles when N is wide), an
n:m pattern of any supported form (2-bit positional codes, the structured 2:4 form, the kept form),
K a multiple of m that is mostly not a multiple of 256, N ragged, and sometimes padded leading
dimensions (element-wise loads). Every stage is compared with the oracle: a', x_q, gamma, the keep
mask and codes exactly (codes and x_q up to counted rounding-boundary elements), the packed RPF
bytes, the int32 accumulators exactly and y within the forward's fp32 tolerance; the one-kernel
bf16 entry must equal the two-call path bit for bit. Inputs: Student-t activations (nu = 4) with a
few channels scaled x20, latent weights N(0, 0.02) with per-row scales U(0.5, 2), as the decode and
prefill workloads."""

import numpy as np
import pytest

from tests import gpu_util as gu
from sparsity_sbn_quantize_amd import inputs

pytestmark = pytest.mark.gpu

PATTERNS = [(2, 4), (4, 4), (1, 4), (3, 4), (4, 8), (6, 8), (8, 8), (3, 8), (5, 8), (1, 8),
            (8, 16), (16, 16), (5, 16), (12, 16)]
BANDS = [(1, 4), (5, 16), (17, 96), (97, 700), (2000, 2600)]


def _draw(case):
    rng = np.random.default_rng(90_000 + case)
    n, m = PATTERNS[case % len(PATTERNS)]
    lo, hi = BANDS[case % len(BANDS)]
    T = int(rng.integers(lo, hi + 1))
    if lo >= 2000:
        # wide enough for 512-row tiles, small K so the oracle stays quick
        N = int(rng.integers(2300, 4400))
        K = int(rng.integers(2, 24)) * 16
    else:
        N = int(rng.integers(1, 700))
        K = int(rng.integers(1, 3000 // m + 1)) * m
    pad = case % 4 == 3  # odd leading dimensions: element-wise loads
    return T, K, N, n, m, pad, rng


@pytest.mark.parametrize("case", range(120))
def test_random_shape_sweep(case):
    T, K, N, n, m, pad, rng = _draw(case)
    x = rng.standard_t(4, (T, K)).astype(np.float32)
    hot = rng.choice(K, size=max(1, K // 1000), replace=False)
    x[:, hot] *= 20.0
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w *= rng.uniform(0.5, 2.0, (N, 1)).astype(np.float32)
    xb = inputs.f32_to_bf16_bits(x)
    kw = dict(ld_x=K + 3, ld_w=K + 1, ld_q=K + 5) if pad else {}
    g = gu.gpu_forward(xb, w, n, m, bf16_step=T <= 16, **kw)
    gu.check_stages(g, xb, w, n, m)
