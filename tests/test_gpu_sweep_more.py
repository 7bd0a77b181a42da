"""Seeded random-shape sweeps of the other entries against the oracle.

- The straight-through data gradient (sbn_bitlinear_bwd_dx; "Sparse-BitNet", the gradient flows to
  the latent weights through the quantizer as if it were the identity): random T, n_out and K
  (tiles of 256 columns, and of 512 columns on 8 waves in every sixth case, ragged rows and
  columns), within the fp32 summation bound
  (n_out + 2) u gamma sum |dY code| of the oracle's fp64 values.
- Grouped forwards over weights that share an input (sbn_bitlinear_fwd_group and its bf16 entry):
  two to five members of random n_out, every member equal to its own forward bit for bit and its
  int32 accumulators equal to the oracle's on the GPU's x_q and codes.
- The int8 GEMV past one batch of quads (K from 12544 to 32768): one to sixteen tokens, positional
  and 2:4 codes, the accumulators exact."""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
PATTERNS = [(2, 4), (6, 8), (8, 16), (4, 8), (8, 8), (3, 8), (12, 16), (1, 4)]


@pytest.mark.parametrize("case", range(48))
def test_bwd_dx_random(case):
    import torch
    n, m = PATTERNS[case % len(PATTERNS)]
    rng = np.random.default_rng(60_000 + case)
    if case % 6 == 5:
        # at least 200 tiles of 512 columns x 128 tokens: the 8-wave workgroups
        T = int(rng.integers(1700, 2101))
        N = int(rng.integers(16, 200))
        K = int(rng.integers(7680 // m, 8192 // m + 1)) * m
        assert -(-K // 512) * -(-T // 128) >= 200
    else:
        T = int(rng.integers(1, 700))
        N = int(rng.integers(1, 1200))
        K = int(rng.integers(1, 4000 // m + 1)) * m
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    dy = inputs.f32_to_bf16_bits((rng.standard_normal((T, N)) * 0.5).astype(np.float32))
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
    dx = binding.bitlinear_bwd_dx(gu.to_dev_bf16(dy), pw)
    codes, _, gamma = pw.export()
    torch.cuda.synchronize()
    codes, gamma, got = codes.cpu().numpy(), np.float32(gamma.cpu().numpy()[0]), dx.cpu().numpy()
    pw.free()
    ref = oracle.ste_dx(dy, codes, gamma).astype(np.float64)
    bound = (N + 2) * U * oracle.ste_dx_abs(dy, codes, gamma) + 1e-30
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(np.isfinite(got)), "non-finite dX"
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"


@pytest.mark.parametrize("case", range(48))
def test_group_random(case):
    import torch
    n, m = PATTERNS[case % len(PATTERNS)]
    rng = np.random.default_rng(61_000 + case)
    T = int(rng.choice([1, 2, 3, 4, int(rng.integers(5, 17)), int(rng.integers(17, 200))]))
    K = int(rng.integers(1, 6000 // m + 1)) * m
    members = int(rng.integers(2, 6))
    ws = [(rng.standard_normal((int(rng.integers(1, 900)), K)) * 0.02).astype(np.float32)
          for _ in range(members)]
    x = inputs.f32_to_bf16_bits(rng.standard_t(4, (T, K)).astype(np.float32))
    xd = gu.to_dev_bf16(x)
    pws = [binding.PackedWeight(gu.to_dev_f32(w), n, m) for w in ws]
    ys_b, q, a = binding.bitlinear_group_bf16(xd, pws, out="f32")
    acc_g = binding.bitlinear_group(q, a, pws, out="i32")
    torch.cuda.synchronize()
    q_ref, a_ref = oracle.quantize_act(x)
    assert np.array_equal(a.cpu().numpy(), a_ref), "absmax"
    qh = q.cpu().numpy()
    gu.assert_int_exact_except_boundary(qh, q_ref, oracle.boundary_elements_act(x, a_ref),
                                        "int8 activations")
    for pw, yb, ag in zip(pws, ys_b, acc_g):
        ys = binding.bitlinear(q, a, pw, out="f32")
        codes, _, gamma = pw.export()
        torch.cuda.synchronize()
        assert np.array_equal(yb.cpu().numpy(), ys.cpu().numpy()), "grouped y vs single forward"
        acc_ref = oracle.int_matmul(qh, codes.cpu().numpy())
        assert np.array_equal(ag.cpu().numpy(), acc_ref), "grouped int32 accumulators"
        gu.assert_y_close(yb.cpu().numpy(),
                          oracle.dequantize(acc_ref, np.float32(gamma.cpu().numpy()[0]),
                                            a.cpu().numpy()))
    for pw in pws:
        pw.free()


@pytest.mark.parametrize("case", range(32))
def test_large_k_random(case):
    import torch
    n, m = [(2, 4), (6, 8), (8, 16), (4, 8)][case % 4]
    rng = np.random.default_rng(62_000 + case)
    T = int(rng.integers(1, 17))
    K = int(rng.integers(12544 // m, 32768 // m + 1)) * m
    N = int(rng.integers(1, 300))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = inputs.f32_to_bf16_bits(rng.standard_t(4, (T, K)).astype(np.float32))
    q, a = binding.quantize_act(gu.to_dev_bf16(x))
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
    acc = binding.bitlinear(q, a, pw, out="i32")
    y = binding.bitlinear(q, a, pw, out="f32")
    codes, _, gamma = pw.export()
    torch.cuda.synchronize()
    acc_ref = oracle.int_matmul(q.cpu().numpy(), codes.cpu().numpy())
    assert np.array_equal(acc.cpu().numpy(), acc_ref), "int32 accumulators"
    gu.assert_y_close(y.cpu().numpy(),
                      oracle.dequantize(acc_ref, np.float32(gamma.cpu().numpy()[0]),
                                        a.cpu().numpy()))
    pw.free()
