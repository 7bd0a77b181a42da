"""GPU parity of re-packing a handle (sbn_pack_nm_ternary on a handle that already holds a pack).

The first pack of a handle reads the latent weights twice: the absmean ("The BitLinear Layer",
operation 3) must be known before a code (Sparse-BitNet, Figure 6: keep the n largest of each
m-group, then the ternary value) can be written. A re-pack of the lean patterns reads them once:
the previous gamma brackets the new threshold, the pieces with a kept magnitude inside the bracket
are finished by a fix-up kernel once the new gamma is known, and the codes are rewritten from the
weights where the bracket does not hold (a fragment that listed too many pieces, or every fragment
when gamma moved by more than 2^-7). Every case must give the oracle's gamma, keep mask and codes
for the current weights exactly, and a forward on the re-packed handle must match the oracle.

The sequences below reach each path: an identical re-pack, gamma scaled by 0.996 and 1.004 (the
threshold moves inside the bracket, so listed pieces change value), a small perturbation (the
masks change), a fragment row block whose kept magnitudes all sit inside the bracket (more listed
pieces than a fragment holds), and gamma scaled by 1.5 (the threshold leaves the bracket)."""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# (n, m, SBN_NO_SMFMAC): 2:4 in the structured-sparse form and in the positional form; the other
# lean patterns; and patterns outside the lean set (always two reads).
PATTERNS = [(2, 4, "0"), (2, 4, "1"), (4, 8, "0"), (6, 8, "0"), (8, 16, "0"), (8, 8, "0"),
            (4, 4, "0"), (1, 4, "0"), (3, 8, "0"), (12, 16, "0")]
LEAN = {(2, 4), (4, 8), (6, 8), (8, 16), (8, 8), (4, 4)}


def _check(pw, w, n, m, what):
    codes_d, keep_d, gamma_d = pw.export()
    g = np.float32(gamma_d.cpu().numpy()[0])
    assert gu.gamma_matches(g, w), f"{what}: gamma {g} vs {oracle.absmean_gamma(w)}"
    keep_ref = oracle.nm_keep_mask(w, n, m)
    assert np.array_equal(keep_d.cpu().numpy().astype(bool), keep_ref), f"{what}: keep mask"
    # the oracle's codes at the gamma the kernels used (equal to the oracle's own gamma except at
    # an fp32 rounding midpoint of the mean)
    codes_ref = oracle.ternary_codes(w, keep_ref, g)
    got = codes_d.cpu().numpy()
    bad = int((got != codes_ref).sum())
    assert bad == 0, f"{what}: {bad} codes differ"


def _sequence(rng, N, K):
    w0 = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    steps = [("identical", w0),
             ("gamma x 0.996", (w0 * np.float32(0.996)).astype(np.float32)),
             ("gamma x 1.004", (w0 * np.float32(1.004)).astype(np.float32)),
             ("perturbed", (w0 + 0.0005 * rng.standard_normal((N, K))).astype(np.float32))]
    return w0, steps


def _crowded(rng, w_prev, N, K):
    """Rows 0..11 with every |w| within 0.2% of the previous threshold gamma/2, rows 12..15 at
    2.5 gamma (so the block's mean, and gamma, stay put): every piece of rows 0..11 holds a kept
    magnitude inside the bracket, 192 listed pieces per fragment of the first row block."""
    gamma = float(oracle.absmean_gamma(w_prev))
    w = w_prev.copy()
    sign = np.where(rng.random((16, K)) < 0.5, -1.0, 1.0)
    mag = np.empty((16, K))
    mag[:12] = 0.5 * gamma * (1.0 + rng.uniform(-0.002, 0.002, (12, K)))
    mag[12:] = 2.5 * gamma * (1.0 + rng.uniform(-0.05, 0.05, (4, K)))
    w[:16] = (sign * mag).astype(np.float32)
    return w


@pytest.mark.parametrize("n,m,no_sp", PATTERNS)
@pytest.mark.parametrize("N,K", [(300, 2560), (70, 1040), (16, 256)])
def test_repack_sequence(n, m, no_sp, N, K, monkeypatch):
    monkeypatch.setenv("SBN_NO_SMFMAC", no_sp)
    K += (-K) % m
    rng = np.random.default_rng(1000 * n + 100 * m + N + K + int(no_sp))
    w0, steps = _sequence(rng, N, K)
    pw = binding.PackedWeight(gu.to_dev_f32(w0), n, m)
    assert pw.query().single_pass == 0
    _check(pw, w0, n, m, "first pack")
    cur = w0
    for what, w in steps:
        pw.pack(gu.to_dev_f32(w))
        assert pw.query().single_pass == (1 if (n, m) in LEAN else 0), what
        _check(pw, w, n, m, what)
        cur = w
    if N >= 16:
        w = _crowded(rng, cur, N, K)
        pw.pack(gu.to_dev_f32(w))
        _check(pw, w, n, m, "crowded row block")
        cur = w
    w = (cur * np.float32(1.5)).astype(np.float32)
    pw.pack(gu.to_dev_f32(w))
    _check(pw, w, n, m, "gamma x 1.5")
    cur = w
    # the forward reads the re-packed planes
    x = inputs.f32_to_bf16_bits(rng.standard_normal((5, K)).astype(np.float32))
    y, _, _ = binding.bitlinear_bf16(gu.to_dev_bf16(x), pw)
    xq, a = oracle.quantize_act(x)
    p = oracle.pack_nm_ternary(cur, n, m)
    y_ref = oracle.dequantize(oracle.int_matmul(xq, p["codes"]), p["gamma"], a)
    gu.assert_y_close(y.cpu().numpy(), y_ref, "y after re-packs")
    pw.free()


def test_repack_flips_and_options(monkeypatch):
    """The single-read re-pack counts mask flips like the two-pass one; a re-pack with variance
    correction or outliers takes the two-read path, and the next plain re-pack reads once again."""
    monkeypatch.setenv("SBN_NO_SMFMAC", "0")
    rng = np.random.default_rng(5)
    N, K = 256, 2048
    w0 = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    w1 = (w0 + 0.002 * rng.standard_normal((N, K))).astype(np.float32)
    pw = binding.PackedWeight(gu.to_dev_f32(w0), 8, 16)
    pw.pack(gu.to_dev_f32(w1))
    assert pw.query().single_pass == 1
    import torch
    f = pw.mask_flips()
    torch.cuda.synchronize()
    assert int(f.cpu().numpy()[0]) == oracle.mask_flips(oracle.nm_keep_mask(w0, 8, 16),
                                                         oracle.nm_keep_mask(w1, 8, 16))
    pw.pack(gu.to_dev_f32(w0), variance_correction=True)
    assert pw.query().single_pass == 0
    pw.pack(gu.to_dev_f32(w1), variance_correction=False)
    assert pw.query().single_pass == 1
    _check(pw, w1, 8, 16, "after the variance-corrected pack")
    pw.free()


def test_repack_7b_ffn_shapes():
    """The training workload's shapes (4096 -> 11008 at 2:4, 11008 -> 4096 at 8:16), re-packed
    from a small latent update: bit-equal keep masks and codes."""
    wl = inputs.W_TRAIN
    for li, (n, m) in ((0, (2, 4)), (1, (8, 16))):
        w = inputs.latent_weights(wl, li)
        rng = np.random.default_rng(li)
        pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
        w2 = (w + 1e-4 * rng.standard_normal(w.shape)).astype(np.float32)
        pw.pack(gu.to_dev_f32(w2))
        assert pw.query().single_pass == 1
        _check(pw, w2, n, m, f"layer {li}")
        pw.free()
