"""Seeded random-shape sweeps of the forward's options against the oracle.

- The parameter-free LayerNorm in front of the quantizer ("Microsoft BitNet 1.58: The Era of 1-Bit
  Large Language Models", "The BitLinear Layer", operation 1) through sbn_bitlinear_fwd_ln_bf16:
  one kernel for one to four tokens, two kernels above; x_q and a' exactly the oracle's, the int32
  accumulators exact, y within the forward's fp32 tolerance.
- Structured k:256 outliers ("From 2:4 to 8:16 sparsity patterns in LLMs for Outliers and Weights
  with Variance Correction", summary), with and without the compact plane: the ternary codes of
  the remaining weights exactly the oracle's, the ternary accumulators exact, y within the bound of
  the fp32 evaluation of (gamma acc + o) a'/127."""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
PATTERNS = [(2, 4), (6, 8), (8, 16), (4, 8), (8, 8), (3, 8), (12, 16)]


@pytest.mark.parametrize("case", range(42))
def test_layernorm_forward_random(case):
    import torch
    n, m = PATTERNS[case % len(PATTERNS)]
    rng = np.random.default_rng(80_000 + case)
    T = int(rng.choice([int(rng.integers(1, 5)), int(rng.integers(5, 17)),
                        int(rng.integers(17, 65))]))
    K = int(rng.integers(1, 4000 // m + 1)) * m
    N = int(rng.integers(1, 500))
    eps = float(rng.choice([1e-5, 1e-6, 1e-3]))
    x = inputs.f32_to_bf16_bits((rng.standard_t(4, (T, K)) * 2 + rng.uniform(-1, 1)).astype(
        np.float32))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xd = gu.to_dev_bf16(x)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
    y, q, a = binding.bitlinear_bf16(xd, pw, out="f32", ln_eps=eps)
    acc, _, _ = binding.bitlinear_bf16(xd, pw, out="i32", ln_eps=eps)
    codes, _, gamma = pw.export()
    torch.cuda.synchronize()
    q_ref, a_ref = oracle.layernorm_quantize_act(x, eps)
    assert np.array_equal(q.cpu().numpy(), q_ref), "x_q after the LayerNorm"
    assert np.array_equal(a.cpu().numpy(), a_ref), "a' after the LayerNorm"
    acc_ref = oracle.int_matmul(q_ref, codes.cpu().numpy())
    assert np.array_equal(acc.cpu().numpy(), acc_ref), "int32 accumulators"
    gu.assert_y_close(y.cpu().numpy(),
                      oracle.dequantize(acc_ref, np.float32(gamma.cpu().numpy()[0]), a_ref))
    pw.free()


@pytest.mark.parametrize("case", range(24))
def test_outliers_random(case):
    import torch
    n, m = [(2, 4), (6, 8), (8, 16), (4, 8)][case % 4]
    compact = case % 3 == 2
    rng = np.random.default_rng(81_000 + case)
    k = int(rng.choice([4, 8, 16]))
    K = int(rng.integers(1, 13)) * 256
    N = int(rng.integers(1, 400))
    T = int(rng.choice([1, 2, 4, int(rng.integers(5, 17)), int(rng.integers(17, 80))]))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w *= rng.uniform(0.5, 2.0, (N, 1)).astype(np.float32)
    x = inputs.f32_to_bf16_bits(rng.standard_t(4, (T, K)).astype(np.float32))
    xd = gu.to_dev_bf16(x)
    q, a = binding.quantize_act(xd)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, compact=compact, outliers=k)
    y = binding.bitlinear(q, a, pw, out="f32")
    acc = binding.bitlinear(q, a, pw, out="i32")
    yb = binding.bitlinear_bf16(xd, pw, out="f32")[0]
    codes, _, g = pw.export()
    pos, val = pw.export_outliers()
    torch.cuda.synchronize()
    ref = oracle.pack_with_outliers(w, n, m, k)
    codes_h = codes.cpu().numpy()
    assert np.array_equal(codes_h, ref["codes"]), "ternary codes of the remaining weights"
    qh, ah = q.cpu().numpy(), a.cpu().numpy()
    f = oracle.forward_with_outliers(qh, ah, codes_h, np.float32(g.cpu().numpy()[0]),
                                     pos.cpu().numpy(), val.cpu().numpy().view(np.uint16))
    assert np.array_equal(acc.cpu().numpy(), f["acc"]), "int32 accumulators (ternary part)"
    bound = ((K // 256) * k + 8) * U * f["mag"] + 1e-30
    for what, got in (("y", y.cpu().numpy()), ("y (bf16 entry)", yb.cpu().numpy())):
        err = np.abs(got.astype(np.float64) - f["y"])
        assert np.all(err <= bound), f"{what}: max err/bound {np.max(err / bound):.3g}"
    pw.free()
