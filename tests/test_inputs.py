"""Seeded input generators: determinism, shapes, distributions, bf16 rounding (CPU only)."""

import numpy as np
import pytest

from sparsity_sbn_quantize_amd import inputs


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40],
                                 np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(inputs.f32_to_bf16_bits(x), ref)
    back = inputs.bf16_bits_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                          .float().numpy())


def test_generators_are_deterministic_and_shaped():
    wl = inputs.W_SMALL
    x1, w1 = inputs.layer_inputs(wl, 0, 8)
    x2, w2 = inputs.layer_inputs(wl, 0, 8)
    assert x1.dtype == np.uint16 and x1.shape == (8, 256)
    assert w1.dtype == np.float32 and w1.shape == (256, 256)
    assert np.array_equal(x1, x2) and np.array_equal(w1, w2)
    assert abs(float(w1.std()) - 0.02) < 0.001


def test_distributions():
    xw = inputs.activations(inputs.W_PREFILL, 0, 256, 2560)
    x = inputs.bf16_bits_to_f32(xw)
    ch = inputs.outlier_channels(2560, inputs.W_PREFILL.index, 0)
    assert ch.size == 3 and len(set(ch.tolist())) == 3
    assert np.abs(x[:, ch]).std() > 10 * np.abs(np.delete(x, ch, axis=1)).std()
    w = inputs.latent_weights(inputs.W_PREFILL, 0, n_out=512, k=512)
    # Laplace(0, b): E|w| = b
    assert abs(float(np.abs(w).mean()) - 0.015) < 0.0005
    wd = inputs.latent_weights(inputs.W_DECODE, 0, n_out=2048, k=256)
    rs = wd.std(axis=1) / 0.02
    assert 0.45 < rs.min() and rs.max() < 2.2
    xt = inputs.bf16_bits_to_f32(inputs.activations(inputs.W_DECODE, 0, 16, 2560))
    # Student-t(4) has heavier tails than N(0,1)
    assert np.abs(xt).max() > 6


def test_workload_shapes():
    assert [(l.n_out, l.k) for l in inputs.W_BLOCK.layers] == [
        (2560, 2560)] * 4 + [(6912, 2560)] * 2 + [(2560, 6912)]
    assert sum(l.n_out * l.k for l in inputs.W_BLOCK.layers) == 79_298_560
    assert [(l.n_out, l.k) for l in inputs.W_TRAIN.layers] == [(11008, 4096), (4096, 11008)]
