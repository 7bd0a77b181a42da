"""GPU parity of the variance-corrected scale (sbn_pack_nm_ternary_ex with
SBN_PACK_VARIANCE_CORRECTION; "From 2:4 to 8:16 sparsity patterns in LLMs for Outliers and Weights
with Variance Correction", method summary).

The pack counts the nonzero dense and n:m ternary codes and writes gamma_out = fl32(gamma *
sqrt(nd / ns)) with the same fp64 steps as the oracle (correctly rounded division and square root),
so the exported scale must equal the oracle's exactly. Codes and the keep mask do not change, so
the int32 accumulators equal the uncorrected ones, and every scaled output (fp32 forward, bf16 and
LayerNorm forwards, the data gradient) follows the oracle with gamma_out in place of gamma.
"""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
PATTERNS = [(2, 4), (6, 8), (8, 16), (3, 8), (8, 8), (1, 4), (12, 16)]


def _w(seed, N, K, kind="normal"):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if kind == "laplace":
        return rng.laplace(0, 0.01, (N, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)  # outlier channels
    w[:, rng.choice(K, max(1, K // 64), replace=False)] *= 30
    return w


def _export(pw):
    import torch
    codes, keep, gamma = pw.export()
    torch.cuda.synchronize()
    return codes.cpu().numpy(), keep.cpu().numpy().astype(bool), np.float32(gamma.cpu().numpy()[0])


@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("N,K,kind", [(70, 1040, "normal"), (300, 2560, "laplace"),
                                      (16, 256, "outliers"), (129, 4096, "normal")])
def test_vc_scale_and_codes(n, m, N, K, kind):
    """Exported gamma_out equals the oracle's bit for bit; codes and keep mask are the uncorrected
    ones; every code form, ragged n_out, several row blocks."""
    K += (-K) % m
    w = _w(N * 13 + K + n * 7 + m, N, K, kind)
    ref = oracle.variance_correction(w, n, m)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, variance_correction=True)
    codes, keep, g = _export(pw)
    pw.free()
    assert g == ref["gamma_out"], f"gamma_out {g!r} vs {ref['gamma_out']!r}"
    keep_ref = oracle.nm_keep_mask(w, n, m)
    assert np.array_equal(keep, keep_ref)
    assert np.array_equal(codes, oracle.ternary_codes(w, keep_ref, ref["gamma"]))
    if n == m:
        assert g == ref["gamma"]
    else:
        assert g >= ref["gamma"]


def test_vc_zero_and_tiny():
    """All-zero weights (no nonzero codes: gamma_out = gamma) and a single row block."""
    import torch
    w = np.zeros((5, 64), np.float32)
    pw = binding.PackedWeight(torch.zeros((5, 64), device="cuda"), 2, 4, variance_correction=True)
    _, _, g = _export(pw)
    pw.free()
    assert g == oracle.variance_correction(w, 2, 4)["gamma_out"]
    w = _w(3, 1, 16)
    pw = binding.PackedWeight(gu.to_dev_f32(w), 2, 4, variance_correction=True)
    _, _, g = _export(pw)
    pw.free()
    assert g == oracle.variance_correction(w, 2, 4)["gamma_out"]


def _forwards(x, w, n, m, T):
    """fp32 and int32 forwards from sbn_quantize_act, the bf16 forward and the LayerNorm forward,
    all through one variance-corrected handle."""
    import torch
    xd = gu.to_dev_bf16(x)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, variance_correction=True)
    q, a = binding.quantize_act(xd)
    y = binding.bitlinear(q, a, pw, out="f32")
    acc = binding.bitlinear(q, a, pw, out="i32")
    yb, _, _ = binding.bitlinear_bf16(xd, pw)
    yl, ql, al = binding.bitlinear_bf16(xd, pw, ln_eps=1e-5)
    codes, _, g = pw.export()
    torch.cuda.synchronize()
    pw.free()
    return dict(q=q.cpu().numpy(), a=a.cpu().numpy(), y=y.cpu().numpy(), acc=acc.cpu().numpy(),
                yb=yb.cpu().numpy(), yl=yl.cpu().numpy(), ql=ql.cpu().numpy(),
                al=al.cpu().numpy(), codes=codes.cpu().numpy(), g=np.float32(g.cpu().numpy()[0]))


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 16), (3, 8)])
@pytest.mark.parametrize("T", [1, 4, 16, 300])
def test_vc_forward(n, m, T):
    """GEMV (T <= 16) and GEMM (T = 300) launches, fused and LayerNorm-fused variants, all scaled
    by gamma_out."""
    K, N = 2560, 264
    rng = np.random.default_rng(T * 31 + n + m)
    x = inputs.f32_to_bf16_bits(rng.standard_t(4, (T, K)).astype(np.float32))
    w = _w(T + 5 * n + m, N, K)
    r = _forwards(x, w, n, m, T)
    ref = oracle.variance_correction(w, n, m)
    assert r["g"] == ref["gamma_out"]
    q_ref, a_ref = oracle.quantize_act(x)
    assert np.array_equal(r["q"], q_ref) and np.array_equal(r["a"], a_ref)
    acc_ref = oracle.int_matmul(q_ref, r["codes"])
    assert np.array_equal(r["acc"], acc_ref)
    y_ref = oracle.dequantize(acc_ref, ref["gamma_out"], a_ref)
    gu.assert_y_close(r["y"], y_ref)
    assert np.array_equal(r["yb"], r["y"])
    ql_ref, al_ref = oracle.layernorm_quantize_act(x, 1e-5)
    assert np.array_equal(r["ql"], ql_ref) and np.array_equal(r["al"], al_ref)
    gu.assert_y_close(r["yl"], oracle.dequantize(oracle.int_matmul(ql_ref, r["codes"]),
                                                 ref["gamma_out"], al_ref), "y (LayerNorm)")
    # the correction is visible: the uncorrected scale would give other outputs (n < m)
    if n < m and ref["gamma_out"] != ref["gamma"]:
        assert not np.array_equal(r["y"], oracle.dequantize(acc_ref, ref["gamma"], a_ref))


@pytest.mark.parametrize("n,m", [(2, 4), (8, 16)])
def test_vc_bwd_dx(n, m):
    """The data gradient uses gamma_out (recursive-summation bound as for the plain gradient)."""
    import torch
    T, N, K = 130, 520, 1024
    rng = np.random.default_rng(77 + n)
    dy = inputs.f32_to_bf16_bits((rng.standard_normal((T, N)) * 0.5).astype(np.float32))
    w = _w(78 + m, N, K)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, variance_correction=True)
    dx = binding.bitlinear_bwd_dx(gu.to_dev_bf16(dy), pw).cpu().numpy().astype(np.float64)
    codes, _, g = _export(pw)
    pw.free()
    torch.cuda.synchronize()
    g_ref = oracle.variance_correction(w, n, m)["gamma_out"]
    assert g == g_ref
    ref = oracle.ste_dx(dy, codes, g_ref).astype(np.float64)
    bound = (N + 2) * U * oracle.ste_dx_abs(dy, codes, g_ref) + 1e-30
    assert np.all(np.abs(dx - ref) <= bound)


def test_vc_toggle_across_repacks():
    """A handle's flag follows each pack: on, off, on with new weights; flips are unaffected."""
    import torch
    N, K, n, m = 300, 1040, 6, 8
    w1 = _w(1, N, K)
    w2 = (w1 + 0.003 * np.random.default_rng(2).standard_normal((N, K))).astype(np.float32)
    pw = binding.PackedWeight(gu.to_dev_f32(w1), n, m, variance_correction=True)
    _, _, g1 = _export(pw)
    assert g1 == oracle.variance_correction(w1, n, m)["gamma_out"]
    pw.pack(gu.to_dev_f32(w1), variance_correction=False)
    _, _, g0 = _export(pw)
    assert g0 == oracle.absmean_gamma(w1)
    f = pw.mask_flips()
    torch.cuda.synchronize()
    assert int(f.cpu().numpy()[0]) == 0
    pw.pack(gu.to_dev_f32(w2), variance_correction=True)
    _, keep2, g2 = _export(pw)
    assert g2 == oracle.variance_correction(w2, n, m)["gamma_out"]
    f = pw.mask_flips()
    torch.cuda.synchronize()
    assert int(f.cpu().numpy()[0]) == oracle.mask_flips(oracle.nm_keep_mask(w1, n, m), keep2)
    pw.free()


def test_vc_7b_ffn_shapes():
    """The 7B FFN projections (11008 x 4096 up at 2:4, 4096 x 11008 down at 8:16) and the
    6912 x 2560 decode projection at 6:8: exact gamma_out."""
    for wl, li, (n, m) in ((inputs.W_TRAIN, 0, (2, 4)), (inputs.W_TRAIN, 1, (8, 16)),
                           (inputs.W_DECODE, 0, (6, 8))):
        w = inputs.latent_weights(wl, li)
        pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, variance_correction=True)
        _, _, g = _export(pw)
        pw.free()
        assert g == oracle.variance_correction(w, n, m)["gamma_out"]
