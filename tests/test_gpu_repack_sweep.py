"""Seeded random walks of re-packs against the oracle (the dynamic mask of "Sparse-BitNet",
re-derived every step from the latent weights, Figure 6; gamma from "The BitLinear Layer",
operation 3).

Each case packs random latent weights once and then re-packs the same handle eight times, every
step applying an update drawn at random: gamma scaled by up to 1% either way (inside or past the
2^-7 bracket of the single-read re-pack), additive noise of four magnitudes, a row block replaced
by a fresh draw, a row block set to exact magnitude ties, rows set to zero, or whole m-groups
permuted along K (the masks move, gamma stays). After every pack
gamma, the keep mask and the codes must equal the oracle's for the current weights (codes at the
gamma the kernels used, which equals the oracle's except at an fp32 rounding midpoint of the mean);
at the end a forward on the handle must match the oracle. Mostly the lean patterns (single-read
re-pack), also patterns outside that set and 2:4 on both MFMA forms. Also walks on padded rows
(NaN canaries past K) and on a base address 4 bytes off 16 (element-wise loads)."""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

PATTERNS = [(2, 4, "0"), (2, 4, "1"), (4, 8, "0"), (6, 8, "0"), (8, 16, "0"), (8, 8, "0"),
            (4, 4, "0"), (8, 16, "0"), (6, 8, "0"), (3, 8, "0"), (5, 16, "0"), (1, 4, "0")]


def _check(pw, w, n, m, what):
    codes_d, keep_d, gamma_d = pw.export()
    g = np.float32(gamma_d.cpu().numpy()[0])
    assert gu.gamma_matches(g, w), f"{what}: gamma {g} vs {oracle.absmean_gamma(w)}"
    keep_ref = oracle.nm_keep_mask(w, n, m)
    assert np.array_equal(keep_d.cpu().numpy().astype(bool), keep_ref), f"{what}: keep mask"
    codes_ref = oracle.ternary_codes(w, keep_ref, g)
    bad = int((codes_d.cpu().numpy() != codes_ref).sum())
    assert bad == 0, f"{what}: {bad} codes differ"


def _update(rng, w, m):
    N, K = w.shape
    kind = int(rng.integers(0, 6))
    w = w.copy()
    if kind == 0:
        w *= np.float32(1.0 + rng.uniform(-0.01, 0.01))
        what = "scaled"
    elif kind == 1:
        sigma = float(rng.choice([1e-5, 1e-4, 1e-3, 5e-3]))
        w += (sigma * rng.standard_normal((N, K))).astype(np.float32)
        what = f"noise {sigma:g}"
    elif kind == 2:
        r0 = int(rng.integers(0, N))
        r1 = min(N, r0 + int(rng.integers(1, 33)))
        w[r0:r1] = (0.02 * rng.standard_normal((r1 - r0, K))).astype(np.float32)
        what = f"rows {r0}..{r1} redrawn"
    elif kind == 3:
        r0 = int(rng.integers(0, N))
        r1 = min(N, r0 + int(rng.integers(1, 17)))
        mag = np.float32(abs(w).mean())
        sign = np.where(rng.random((r1 - r0, K)) < 0.5, -1.0, 1.0).astype(np.float32)
        w[r0:r1] = sign * mag
        what = f"rows {r0}..{r1} tied"
    elif kind == 4:
        rows = rng.choice(N, size=max(1, N // 10), replace=False)
        w[rows] = 0.0
        what = "rows zeroed"
    else:
        w = w[:, rng.permutation(K // m).repeat(m) * m + np.tile(np.arange(m), K // m)]
        w = np.ascontiguousarray(w)
        what = "groups permuted"
    return w.astype(np.float32), what


@pytest.mark.parametrize("case", range(72))
def test_random_repack_walk(case, monkeypatch):
    n, m, no_sp = PATTERNS[case % len(PATTERNS)]
    monkeypatch.setenv("SBN_NO_SMFMAC", no_sp)
    rng = np.random.default_rng(70_000 + case)
    N = int(rng.integers(1, 600))
    K = int(rng.integers(1, 3000 // m + 1)) * m
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    w *= rng.uniform(0.5, 2.0, (N, 1)).astype(np.float32)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
    _check(pw, w, n, m, "first pack")
    for step in range(8):
        w, what = _update(rng, w, m)
        pw.pack(gu.to_dev_f32(w))
        _check(pw, w, n, m, f"step {step}: {what}")
    x = inputs.f32_to_bf16_bits(rng.standard_normal((3, K)).astype(np.float32))
    y, _, _ = binding.bitlinear_bf16(gu.to_dev_bf16(x), pw)
    xq, a = oracle.quantize_act(x)
    p = oracle.pack_nm_ternary(w, n, m)
    y_ref = oracle.dequantize(oracle.int_matmul(xq, p["codes"]), p["gamma"], a)
    gu.assert_y_close(y.cpu().numpy(), y_ref, "y after the walk")
    pw.free()


@pytest.mark.parametrize("case", range(24))
def test_random_repack_walk_padded(case):
    """The same walks on weights whose rows are padded (NaN canaries past K: a read beyond the row
    would make gamma NaN) or whose base address is 4 bytes off 16: the single-read pass and its
    fix-up on element-wise loads, and on 16-byte loads over padded rows."""
    import torch
    n, m, _ = PATTERNS[case % len(PATTERNS)]
    rng = np.random.default_rng(71_000 + case)
    N = int(rng.integers(1, 500))
    K = int(rng.integers(1, 2500 // m + 1)) * m
    layout = ["pad1", "pad4", "offset"][case % 3]

    def dev(w):
        if layout == "pad1":
            return gu.to_dev_f32(w, ld=K + 1)
        if layout == "pad4":
            return gu.to_dev_f32(w, ld=K + 4)
        flat = torch.full((N * K + 1,), float("nan"), dtype=torch.float32, device="cuda")
        flat[1:].copy_(torch.from_numpy(np.ascontiguousarray(w)).reshape(-1))
        return flat[1:].view(N, K)

    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    pw = binding.PackedWeight(dev(w), n, m)
    _check(pw, w, n, m, f"{layout}: first pack")
    for step in range(6):
        w, what = _update(rng, w, m)
        pw.pack(dev(w))
        _check(pw, w, n, m, f"{layout} step {step}: {what}")
    pw.free()
