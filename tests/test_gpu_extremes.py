"""Extreme magnitudes against the oracle (absmean gamma, n:m keep mask and ternary codes of
"Sparse-BitNet" and of "The BitLinear Layer", operation 3; per-token absmax int8 activations,
operation 2).

- Latent weights at scales from 1e30 down into the fp32 subnormal range: gamma subnormal, and gamma
  rounding to zero (every kept nonzero weight then ternarizes to its sign). Each goes through
  quantize -> pack -> forward with every stage compared, across the launch paths (one token, the
  GEMV, the GEMM).
- Activations at the top of the bf16 range, in its subnormal range (under the absmax floor of
  1e-5), all-zero rows and one-hot rows.
- Re-packs of one handle across scale jumps: x1e6 (outside the single-read re-pack's bracket, and
  its fixed-point gamma sum overflows), x1.001 at that scale (inside the bracket), x1e-6, all-zero
  weights (gamma 0), a re-pack from that zero gamma, and rows of 1e30 mixed with rows of 1e-30.
  After every pack gamma, the keep mask and the codes must equal the oracle's."""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

PATTERNS = [(2, 4), (8, 16), (6, 8), (3, 8), (4, 8), (1, 4)]
TOKENS = [1, 5, 12, 40, 300]
TINY = np.float32(2.0 ** -149)  # the smallest fp32 subnormal


def _weights(kind, rng, N, K):
    if kind == "huge":
        return (rng.standard_normal((N, K)) * 1e30).astype(np.float32)
    if kind == "tiny":
        return (rng.standard_normal((N, K)) * 1e-30).astype(np.float32)
    if kind == "subnormal":  # mostly below 2^-126; gamma subnormal
        return (rng.standard_normal((N, K)) * 4e-39).astype(np.float32)
    if kind == "ulps":  # integer multiples of 2^-149: gamma a small multiple of it
        return rng.integers(-3, 4, (N, K)).astype(np.float32) * TINY
    # "zero_gamma": a few +-2^-149 among zeros; the mean rounds to zero
    w = np.zeros((N, K), np.float32)
    idx = rng.choice(N * K, size=max(1, N * K // 8), replace=False)
    w.flat[idx] = np.where(rng.random(idx.size) < 0.5, -TINY, TINY)
    return w


WEIGHT_KINDS = ["huge", "tiny", "subnormal", "ulps", "zero_gamma"]


@pytest.mark.parametrize("case", range(25))
def test_extreme_weight_scales(case):
    kind = WEIGHT_KINDS[case % len(WEIGHT_KINDS)]
    n, m = PATTERNS[case % len(PATTERNS)]
    rng = np.random.default_rng(95_000 + case)
    T = TOKENS[(case // len(WEIGHT_KINDS)) % len(TOKENS)]
    K = int(rng.integers(1, 2000 // m + 1)) * m
    N = int(rng.integers(1, 500))
    w = _weights(kind, rng, N, K)
    if kind == "zero_gamma":
        assert oracle.absmean_gamma(w) == 0.0
    x = inputs.f32_to_bf16_bits(rng.standard_t(4, (T, K)).astype(np.float32))
    g = gu.gpu_forward(x, w, n, m, bf16_step=T <= 16)
    gu.check_stages(g, x, w, n, m)


def _activation_rows(rng, T, K):
    """T rows cycling through: near the bf16 maximum (random signs), bf16 subnormals, the maximum
    and subnormals mixed, all zeros, one nonzero element, ordinary Student-t."""
    rows = []
    for t in range(T):
        kind = t % 6
        if kind == 0:
            mag = rng.integers(0x7F00, 0x7F80, K).astype(np.uint16)
        elif kind == 1:
            mag = rng.integers(1, 0x80, K).astype(np.uint16)
        elif kind == 2:
            mag = np.where(rng.random(K) < 0.1, 0x7F7F, rng.integers(1, 0x80, K)).astype(np.uint16)
        elif kind == 3:
            mag = np.zeros(K, np.uint16)
        elif kind == 4:
            mag = np.zeros(K, np.uint16)
            mag[int(rng.integers(0, K))] = inputs.f32_to_bf16_bits(
                np.float32([rng.uniform(1e-3, 1e3)]))[0]
        else:
            mag = inputs.f32_to_bf16_bits(np.abs(rng.standard_t(4, K)).astype(np.float32))
        sign = np.where(rng.random(K) < 0.5, 0x8000, 0).astype(np.uint16)
        rows.append(mag | sign)
    return np.stack(rows).astype(np.uint16)


@pytest.mark.parametrize("case", range(15))
def test_extreme_activations(case):
    n, m = PATTERNS[case % len(PATTERNS)]
    rng = np.random.default_rng(96_000 + case)
    T = TOKENS[case % len(TOKENS)]
    K = int(rng.integers(1, 2000 // m + 1)) * m
    N = int(rng.integers(1, 500))
    x = _activation_rows(rng, T, K)
    # weights small enough that y stays finite for a' near the bf16 maximum
    w = (rng.standard_normal((N, K)) * 1e-12).astype(np.float32)
    g = gu.gpu_forward(x, w, n, m, bf16_step=T <= 16)
    assert np.all(np.isfinite(g["y"]))
    gu.check_stages(g, x, w, n, m)


def _check(pw, w, n, m, what):
    codes_d, keep_d, gamma_d = pw.export()
    g = np.float32(gamma_d.cpu().numpy()[0])
    assert gu.gamma_matches(g, w), f"{what}: gamma {g} vs {oracle.absmean_gamma(w)}"
    keep_ref = oracle.nm_keep_mask(w, n, m)
    assert np.array_equal(keep_d.cpu().numpy().astype(bool), keep_ref), f"{what}: keep mask"
    codes_ref = oracle.ternary_codes(w, keep_ref, g)
    bad = int((codes_d.cpu().numpy() != codes_ref).sum())
    assert bad == 0, f"{what}: {bad} codes differ"


@pytest.mark.parametrize("case", range(12))
def test_repack_scale_jumps(case):
    n, m = PATTERNS[case % len(PATTERNS)]
    rng = np.random.default_rng(97_000 + case)
    N = int(rng.integers(1, 600))
    K = int(rng.integers(1, 3000 // m + 1)) * m
    w0 = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    mixed = w0 * np.where(rng.random((N, 1)) < 0.3, np.float32(1e30), np.float32(1e-30))
    steps = [("x1e6", w0 * np.float32(1e6)),
             ("x1e6 then x1.001", w0 * np.float32(1e6) * np.float32(1.001)),
             ("x1e-6", w0 * np.float32(1e-6)),
             ("zeros", np.zeros_like(w0)),
             ("back from zero gamma", w0),
             ("x1.003", w0 * np.float32(1.003)),
             ("rows of 1e30 and 1e-30", mixed.astype(np.float32)),
             ("mixed x0.999", (mixed * np.float32(0.999)).astype(np.float32)),
             ("back", w0)]
    pw = binding.PackedWeight(gu.to_dev_f32(w0), n, m)
    _check(pw, w0, n, m, "first pack")
    for what, w in steps:
        pw.pack(gu.to_dev_f32(w))
        _check(pw, w, n, m, what)
    x = inputs.f32_to_bf16_bits(rng.standard_normal((3, K)).astype(np.float32))
    y, _, _ = binding.bitlinear_bf16(gu.to_dev_bf16(x), pw)
    xq, a = oracle.quantize_act(x)
    p = oracle.pack_nm_ternary(w0, n, m)
    y_ref = oracle.dequantize(oracle.int_matmul(xq, p["codes"]), p["gamma"], a)
    gu.assert_y_close(y.cpu().numpy(), y_ref, "y after the walk")
    pw.free()
