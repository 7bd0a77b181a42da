"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, stage by stage.

Integer results (int8 activations, keep masks, ternary codes, packed bytes, int32 accumulators)
must be bit-exact (codes and int8 values may differ only at counted rounding boundaries); fp32
outputs within 1e-5 relative.
"""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

FAST_PATTERNS = [(2, 4), (4, 4), (4, 8), (6, 8), (8, 8), (8, 16), (16, 16)]
GENERIC_PATTERNS = [(1, 4), (3, 4), (1, 8), (3, 8), (5, 8), (7, 8), (2, 8), (1, 16), (5, 16),
                    (12, 16), (15, 16)]


def _rand_case(seed, T, K, N, scale=0.02, ties=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, K)).astype(np.float32) * 2
    if ties:
        w = (rng.integers(-4, 5, (N, K)) * 0.01).astype(np.float32)
    else:
        w = (rng.standard_normal((N, K)) * scale).astype(np.float32)
    return inputs.f32_to_bf16_bits(x), w


def test_small_workload_2of4():
    """Single BitLinear, 2:4, T=8, K=256, N=256, seed 0."""
    wl = inputs.W_SMALL
    x, w = inputs.layer_inputs(wl, 0, 8)
    g = gu.gpu_forward(x, w, 2, 4)
    gu.check_stages(g, x, w, 2, 4)


def test_worked_example():
    import json, os
    from tests.conftest import GOLDEN
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_2of4.json")))
    # pad to 64 positions per row so the brick is exercised with the example in its first group
    w = np.zeros((1, 8), np.float32)
    w[0] = ex["w"]
    x = inputs.f32_to_bf16_bits(np.array([ex["x"]], np.float32))
    g = gu.gpu_forward(x, w, 2, 4)
    e = ex["expected"]
    assert g["gamma"] == np.float32(e["gamma"])
    assert g["q"][0].tolist() == e["q"]
    assert g["codes"][0].tolist() == e["codes_2of4"]
    assert g["code_bytes"][0].tolist() == e["code_bytes_2of4"]
    assert g["mask_bytes"][0].tolist() == e["mask_bytes_2of4"]
    assert int(g["acc"][0, 0]) == e["acc_2of4"]
    assert g["y"][0, 0] == np.float32(e["y_2of4"])


@pytest.mark.parametrize("n,m", FAST_PATTERNS + GENERIC_PATTERNS)
@pytest.mark.parametrize("T", [1, 7, 16, 150])
def test_patterns_ragged(n, m, T):
    """Several tiles with ragged tails: n_out not a multiple of 16 or 256, K not a multiple of
    64 or 256, T not a multiple of 16 or 128."""
    K = {4: 4 * 85, 8: 8 * 43, 16: 16 * 21}[m]
    N = 300
    x, w = _rand_case(n * 1000 + m * 10 + T, T, K, N, ties=(T == 7))
    g = gu.gpu_forward(x, w, n, m)
    gu.check_stages(g, x, w, n, m)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 16), (3, 8)])
def test_unaligned_leading_dims(n, m):
    T, K, N = 37, 5 * m * 4, 45
    x, w = _rand_case(5, T, K, N)
    g = gu.gpu_forward(x, w, n, m, ld_x=K + 3, ld_w=K + 1, ld_q=K + 5)
    gu.check_stages(g, x, w, n, m)
    assert np.all(g["q_pad"][:, K:] == 77), "int8 output written beyond K"


def test_output_leading_dim_canaries():
    import torch
    T, K, N = 20, 256, 40
    x, w = _rand_case(9, T, K, N)
    xd = gu.to_dev_bf16(x)
    q, a = binding.quantize_act(xd)
    pw = binding.PackedWeight(gu.to_dev_f32(w), 6, 8)
    ybuf = torch.full((T, N + 9), -7.0, dtype=torch.float32, device="cuda")
    binding.bitlinear(q, a, pw, out="f32", y=ybuf[:, :N])
    yb = ybuf.cpu().numpy()
    assert np.all(yb[:, N:] == -7.0)
    acc_ref = oracle.int_matmul(q.cpu().numpy(), pw.export()[0].cpu().numpy())
    gu.assert_y_close(yb[:, :N], oracle.dequantize(acc_ref, pw.export()[2].cpu().numpy()[0],
                                                   a.cpu().numpy()))


def test_edge_cases():
    import torch
    # zero activation rows, a tiny row, all-zero weights (gamma = 0)
    T, K, N = 5, 128, 32
    xf = np.random.default_rng(1).standard_normal((T, K)).astype(np.float32)
    xf[1] = 0.0
    xf[2] = 0.0
    xf[2, 5] = 1e-30
    x = inputs.f32_to_bf16_bits(xf)
    w = np.zeros((N, K), np.float32)
    g = gu.gpu_forward(x, w, 2, 4)
    gu.check_stages(g, x, w, 2, 4)
    assert g["gamma"] == 0 and np.all(g["codes"] == 0) and np.all(g["acc"] == 0)
    assert g["a_prime"][1] == np.float32(1e-5) and np.all(g["q"][1] == 0)
    # exact ties everywhere: equal magnitudes keep the lowest positions
    w = np.full((N, K), 0.01, np.float32)
    w[:, ::3] *= -1
    g = gu.gpu_forward(x, w, 2, 4)
    gu.check_stages(g, x, w, 2, 4)
    # T = 0 is a no-op; n_out smaller than one fragment; K = m
    q = torch.empty((0, K), dtype=torch.int8, device="cuda")
    a = torch.empty((0,), dtype=torch.float32, device="cuda")
    binding.quantize_act(gu.to_dev_bf16(np.zeros((0, K), np.uint16)), out_q=q, out_absmax=a)
    x1, w1 = _rand_case(3, 3, 16, 3)
    g = gu.gpu_forward(x1, w1, 8, 16)
    gu.check_stages(g, x1, w1, 8, 16)


def test_repack_in_place_and_shape_errors():
    import torch
    T, K, N = 16, 512, 64
    x, w = _rand_case(11, T, K, N)
    xd = gu.to_dev_bf16(x)
    q, a = binding.quantize_act(xd)
    pw = binding.PackedWeight(gu.to_dev_f32(w), 8, 16)
    h0 = pw.handle.value
    for step in range(3):
        w2 = (w + np.float32(0.003) * step * np.sign(w)).astype(np.float32)
        pw.pack(gu.to_dev_f32(w2))
        assert pw.handle.value == h0, "re-pack must reuse the handle"
        codes, keep, gamma = pw.export()
        p = oracle.pack_nm_ternary(w2, 8, 16)
        assert np.array_equal(keep.cpu().numpy().astype(bool), p["keep"])
        assert np.array_equal(codes.cpu().numpy(), p["codes"])
        acc = binding.bitlinear(q, a, pw, out="i32").cpu().numpy()
        assert np.array_equal(acc, oracle.int_matmul(q.cpu().numpy(), p["codes"]))
    with pytest.raises(binding.SbnError) as e:
        pw.pack(gu.to_dev_f32(w[:, :256]))
    assert e.value.status == -3
    pw.free()


def test_determinism_of_gamma():
    w = inputs.latent_weights(inputs.W_PREFILL, 0, n_out=2048, k=2560)
    wd = gu.to_dev_f32(w)
    gs = set()
    for _ in range(3):
        pw = binding.PackedWeight(wd, 8, 16)
        gs.add(float(pw.export()[2].cpu().numpy()[0]))
        pw.free()
    assert len(gs) == 1
    assert gs.pop() == float(oracle.absmean_gamma(w))
