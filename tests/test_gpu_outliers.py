"""GPU parity of the structured k:256 outliers (sbn_pack_nm_ternary_ex with SBN_PACK_OUTLIERS(k);
"From 2:4 to 8:16 sparsity patterns in LLMs for Outliers and Weights with Variance Correction",
summary: salient weights kept in structured 4:256, 8:256 or 16:256 patterns).

Integer and selection work is bit-exact: outlier positions and bf16 values, codes and keep mask of
the remaining weights, int32 accumulators. gamma is the absmean of the remaining weights; the GPU
takes the outliers' |w| off its blocked fp64 sum, so the fp64 mean can differ from the oracle's in
its last bits, and gamma is compared exactly unless that mean lies within 1e-9 of an fp32 rounding
midpoint (one ulp then). The fp32 output adds fl32(o * step) with o an fp32 sum of exact products:
its error is below (n_o + 8) * 2^-24 * (|gamma acc| + |x_q| |O|) * a'/127, n_o outliers per row.
"""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _w(seed, N, K):
    rng = np.random.default_rng(seed)
    return rng.laplace(0, 0.015, (N, K)).astype(np.float32)


def _x(seed, T, K):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 1000), replace=False)] *= 20
    return inputs.f32_to_bf16_bits(x)


def _gamma_ok(g, ref_w_rest):
    mean = np.abs(ref_w_rest.astype(np.float64)).sum() / ref_w_rest.size
    exact = np.float32(mean)
    if g == exact:
        return True
    lo, hi = sorted((np.float64(exact), np.float64(g)))
    mid = (lo + hi) / 2
    return abs(mean - mid) <= 1e-9 * mean and abs(int(np.float32(g).view(np.int32)) -
                                                    int(exact.view(np.int32))) == 1


def _pack_export(w, n, m, k, **kw):
    import torch
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, outliers=k, **kw)
    pos, val = pw.export_outliers()
    codes, keep, g = pw.export()
    torch.cuda.synchronize()
    r = dict(pos=pos.cpu().numpy(), val=val.cpu().numpy().view(np.uint16),
             codes=codes.cpu().numpy(), keep=keep.cpu().numpy().astype(bool),
             gamma=np.float32(g.cpu().numpy()[0]), desc=pw.query())
    return pw, r


@pytest.mark.parametrize("k", [4, 8, 16])
@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 16), (3, 8), (8, 8)])
@pytest.mark.parametrize("N,K", [(70, 1024), (300, 2560), (16, 256)])
def test_outlier_pack(k, n, m, N, K):
    """Positions and bf16 values of the outliers, and the codes, keep mask and gamma of the
    remaining weights, against the oracle."""
    w = _w(N + K + 7 * k + n + m, N, K)
    pw, r = _pack_export(w, n, m, k)
    pw.free()
    ref = oracle.pack_with_outliers(w, n, m, k)
    assert r["desc"].outlier_k == k
    assert np.array_equal(r["pos"], ref["opos"]) and np.array_equal(r["val"], ref["oval"])
    assert np.array_equal(r["keep"], ref["keep"])
    assert np.array_equal(r["codes"], ref["codes"])
    assert _gamma_ok(r["gamma"], ref["w_rest"])


def test_outlier_ties_and_zeros():
    """Equal magnitudes go to the lower positions; all-zero groups keep positions 0..k-1."""
    w = np.zeros((20, 512), np.float32)
    w[3, :256] = 0.5             # a whole group tied
    w[4, 256:] = -0.25
    w[4, 300] = 1.0
    w[5] = np.tile(np.float32([1.0, -1.0]), 256)
    pw, r = _pack_export(w, 2, 4, 8)
    pw.free()
    ref = oracle.pack_with_outliers(w, 2, 4, 8)
    assert np.array_equal(r["pos"], ref["opos"]) and np.array_equal(r["val"], ref["oval"])
    assert r["pos"][0, 0].tolist() == list(range(8)) and r["pos"][3, 0].tolist() == list(range(8))
    assert np.array_equal(r["codes"], ref["codes"])


def _fwd(w, x, n, m, k, T, **kw):
    import torch
    xd = gu.to_dev_bf16(x)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, outliers=k, **kw)
    q, a = binding.quantize_act(xd)
    y = binding.bitlinear(q, a, pw, out="f32")
    acc = binding.bitlinear(q, a, pw, out="i32")
    res = dict(y=y, acc=acc, q=q, a=a)
    if T <= 16:
        res["yb"] = binding.bitlinear_bf16(xd, pw)[0]
    codes, _, g = pw.export()
    pos, val = pw.export_outliers()
    torch.cuda.synchronize()
    out = {kk: v.cpu().numpy() for kk, v in res.items()}
    out.update(codes=codes.cpu().numpy(), gamma=np.float32(g.cpu().numpy()[0]),
               pos=pos.cpu().numpy(), val=val.cpu().numpy().view(np.uint16))
    pw.free()
    return out


def _check_y(r, k, K):
    f = oracle.forward_with_outliers(r["q"], r["a"], r["codes"], r["gamma"], r["pos"], r["val"])
    assert np.array_equal(r["acc"], f["acc"]), "int32 accumulators (ternary part)"
    n_o = (K // 256) * k
    bound = (n_o + 8) * U * f["mag"] + 1e-30
    err = np.abs(r["y"].astype(np.float64) - f["y"])
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"
    return f


@pytest.mark.parametrize("k", [4, 16])
@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 16)])
@pytest.mark.parametrize("T", [1, 3, 16, 40])
def test_outlier_forward(k, n, m, T):
    """GEMV and GEMM launches plus the outlier term, within the fp32 bound; the bf16-input path
    (one kernel for T <= 4) gives the same bits."""
    K, N = 2560, 300
    w = _w(T * 5 + k + n, N, K)
    x = _x(T + 31, T, K)
    r = _fwd(w, x, n, m, k, T)
    q_ref, a_ref = oracle.quantize_act(x)
    assert np.array_equal(r["q"], q_ref) and np.array_equal(r["a"], a_ref)
    ref = oracle.pack_with_outliers(w, n, m, k)
    assert np.array_equal(r["codes"], ref["codes"])
    f = _check_y(r, k, K)
    assert np.max(np.abs(f["o"])) > 0  # the outlier term is present
    if T <= 16:
        assert np.array_equal(r["yb"], r["y"])


def test_outlier_with_variance_correction_and_compact():
    """VC counts the remaining weights' codes; the compact GEMV reads their codes."""
    K, N, n, m, k = 1024, 96, 6, 8, 8
    w = _w(41, N, K)
    x = _x(42, 2, K)
    r = _fwd(w, x, n, m, k, 2, variance_correction=True, compact=True)
    vc = oracle.variance_correction(oracle.pack_with_outliers(w, n, m, k)["w_rest"], n, m)
    assert r["gamma"] == vc["gamma_out"] or _gamma_ok(
        r["gamma"] / np.float32(np.sqrt(vc["nd"] / vc["ns"])),
        oracle.pack_with_outliers(w, n, m, k)["w_rest"])
    _check_y(r, k, K)


def test_outlier_repack_toggle_and_backward_rejected():
    import torch
    K, N = 512, 64
    w = _w(50, N, K)
    pw = binding.PackedWeight(gu.to_dev_f32(w), 2, 4, outliers=4)
    dy = torch.zeros((2, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.SbnError) as e:
        binding.bitlinear_bwd_dx(dy, pw)
    assert e.value.status == -2
    pw.pack(gu.to_dev_f32(w), outliers=0)
    assert pw.query().outlier_k == 0
    with pytest.raises(binding.SbnError):
        pw.export_outliers()
    codes, _, _ = pw.export()
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), oracle.pack_nm_ternary(w, 2, 4)["codes"])
    binding.bitlinear_bwd_dx(dy, pw)  # allowed again
    pw.free()


def test_outlier_decode_shape():
    """The 2560 -> 6912 decode projection at 6:8 with 16:256 outliers, T = 1 (one-kernel step
    plus the outlier term)."""
    wl = inputs.W_DECODE
    w = inputs.latent_weights(wl, 0)
    x = inputs.activations(wl, 0, 1, w.shape[1])
    r = _fwd(w, x, 6, 8, 16, 1)
    ref = oracle.pack_with_outliers(w, 6, 8, 16)
    assert np.array_equal(r["pos"], ref["opos"]) and np.array_equal(r["val"], ref["oval"])
    assert np.array_equal(r["codes"], ref["codes"])
    _check_y(r, 16, w.shape[1])
    assert np.array_equal(r["yb"], r["y"])


@pytest.mark.parametrize("k", [4, 8, 16])
@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (3, 8), (8, 16)])
@pytest.mark.parametrize("N,K", [(64, 256), (304, 2560), (96, 12288), (48, 4096), (64, 6912)])
def test_outlier_term_in_the_one_token_step(k, n, m, N, K):
    """One token, n_out a multiple of 16: both the bf16-input step and the int8 forward add the
    outlier term in the GEMV's launch (one to 48 quads, 1 to 16 waves, one to three quads per
    wave: K = 6912 has 27 quads, two per wave; every code form). Both stay within the fp32 bound
    and give the same bits."""
    w = _w(N * 3 + K + 7 * k + n, N, K)
    x = _x(K + k, 1, K)
    r = _fwd(w, x, n, m, k, 1)
    q_ref, a_ref = oracle.quantize_act(x)
    assert np.array_equal(r["q"], q_ref) and np.array_equal(r["a"], a_ref)
    _check_y(r, k, K)
    assert np.array_equal(r["yb"], r["y"])


@pytest.mark.parametrize("k", [4, 16])
@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (3, 8), (8, 16)])
@pytest.mark.parametrize("K", [2560, 12288])
def test_one_token_outlier_launch_equals_two_launch_order(k, n, m, K):
    """The one-token launches sum the outlier term in the order of the separate outlier kernel
    (eight partial sums per row over groups c, c + 8, ..., added in order c = 0 .. 7). The same
    token as row 0 of a two-token call (GEMV, then the outlier kernel) must give row 0 of the
    one-token output bit for bit, here with G = 10 and 48 groups of 256, more than the eight
    partial sums, so the cross-group order is exercised."""
    import torch
    N = 96
    w = _w(K + 11 * k + n, N, K)
    x2 = _x(K + 3 * k + m, 2, K)
    xd2 = gu.to_dev_bf16(x2)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, outliers=k)
    q2, a2 = binding.quantize_act(xd2)
    y2 = binding.bitlinear(q2, a2, pw, out="f32")          # GEMV + outlier kernel
    y1 = binding.bitlinear(q2[:1], a2[:1], pw, out="f32")  # one launch, int8 input
    yb = binding.bitlinear_bf16(xd2[:1], pw)[0]            # one launch, bf16 input
    torch.cuda.synchronize()
    assert np.array_equal(y1.cpu().numpy()[0], y2.cpu().numpy()[0])
    assert np.array_equal(yb.cpu().numpy()[0], y2.cpu().numpy()[0])
    pw.free()


def test_outlier_term_in_the_one_token_step_unaligned_y_and_fallbacks():
    """An output row 4 bytes off 16-byte alignment (element-wise stores in the one-kernel step),
    n_out not a multiple of 16 and the LayerNorm step (both: forward, then the outlier kernel)."""
    import torch
    K, N, n, m, k = 1024, 160, 6, 8, 16
    w = _w(77, N, K)
    x = _x(78, 1, K)
    xd = gu.to_dev_bf16(x)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, outliers=k)
    q, a = binding.quantize_act(xd)
    y_ref = binding.bitlinear(q, a, pw, out="f32")
    ybuf = torch.full((N + 1,), -7.0, dtype=torch.float32, device="cuda")
    binding.bitlinear_bf16(xd, pw, y=ybuf[1:].view(1, N))
    yl, ql, al = binding.bitlinear_bf16(xd, pw, ln_eps=1e-5)
    yl_ref = binding.bitlinear(ql, al, pw, out="f32")
    torch.cuda.synchronize()
    assert ybuf[0].item() == -7.0
    assert np.array_equal(ybuf[1:].cpu().numpy(), y_ref.cpu().numpy()[0])
    assert np.array_equal(yl.cpu().numpy(), yl_ref.cpu().numpy())
    pw.free()
    w2 = _w(79, 72, K)
    r = _fwd(w2, x, n, m, k, 1)
    _check_y(r, k, K)
    assert np.array_equal(r["yb"], r["y"])
