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
  After every pack gamma, the keep mask and the codes must equal the oracle's. Also walks whose
  previous gamma is subnormal (the single-read pass's bracket in the subnormal range), and the
  jumps with variance correction, the compact plane or k:256 outliers on, where gamma_out, the
  compact bytes, the outlier positions and values and the mask flip count are checked as well.
- The parameter-free LayerNorm ("The BitLinear Layer", operation 1) on rows of large, subnormal,
  zero, constant and one-hot activations: x_q and a' exactly the oracle's.
- Structured k:256 outliers ("From 2:4 to 8:16 sparsity patterns in LLMs for Outliers and Weights
  with Variance Correction", summary) of huge and of subnormal weights: positions and bf16 values
  exactly the oracle's, the ternary codes and accumulators exact, y within the fp32 bound.
- The straight-through data gradient with gamma near 1e30, or dY near 1e34, within the fp32
  summation bound; grouped forwards whose members range from 1e30 to subnormal and all-zero
  weights, each member equal to its own forward."""

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


def _ln_rows(rng, T, K):
    """T rows cycling through: large magnitudes (up to 8.5e37, random signs, so that fp32 x - mu
    stays finite), bf16 subnormals, all zeros, one constant, one nonzero element, Student-t."""
    rows = []
    for t in range(T):
        kind = t % 6
        sign = np.where(rng.random(K) < 0.5, 0x8000, 0).astype(np.uint16)
        if kind == 0:
            row = rng.integers(0x7E00, 0x7E80, K).astype(np.uint16) | sign
        elif kind == 1:
            row = rng.integers(1, 0x80, K).astype(np.uint16) | sign
        elif kind == 2:
            row = np.zeros(K, np.uint16)
        elif kind == 3:
            row = np.full(K, inputs.f32_to_bf16_bits(np.float32([rng.uniform(-50, 50)]))[0],
                          np.uint16)
        elif kind == 4:
            row = np.zeros(K, np.uint16)
            row[int(rng.integers(0, K))] = 0x4120  # 10.0
        else:
            row = inputs.f32_to_bf16_bits(rng.standard_t(4, K).astype(np.float32))
        rows.append(row)
    return np.stack(rows).astype(np.uint16)


@pytest.mark.parametrize("case", range(10))
def test_extreme_layernorm(case):
    import torch
    n, m = PATTERNS[case % len(PATTERNS)]
    rng = np.random.default_rng(98_000 + case)
    T = [1, 3, 4, 5, 12, 40][case % 6]
    K = int(rng.integers(1, 2000 // m + 1)) * m
    N = int(rng.integers(1, 400))
    eps = float(rng.choice([1e-5, 1e-6]))
    x = _ln_rows(rng, T, K)
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


@pytest.mark.parametrize("case", range(8))
def test_extreme_outliers(case):
    import torch
    n, m = [(2, 4), (8, 16), (6, 8), (4, 8)][case % 4]
    scale = [1e30, 4e-39][case % 2]  # huge weights, or mostly fp32 subnormals
    rng = np.random.default_rng(99_000 + case)
    k = int(rng.choice([4, 16]))
    K = int(rng.integers(1, 7)) * 256
    N = int(rng.integers(1, 300))
    T = [1, 5, 40, 3][case % 4]
    w = (rng.standard_normal((N, K)) * scale).astype(np.float32)
    x = inputs.f32_to_bf16_bits(rng.standard_t(4, (T, K)).astype(np.float32))
    q, a = binding.quantize_act(gu.to_dev_bf16(x))
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, outliers=k)
    y = binding.bitlinear(q, a, pw, out="f32")
    acc = binding.bitlinear(q, a, pw, out="i32")
    codes, _, g = pw.export()
    pos, val = pw.export_outliers()
    torch.cuda.synchronize()
    ref = oracle.pack_with_outliers(w, n, m, k)
    codes_h = codes.cpu().numpy()
    assert np.array_equal(codes_h, ref["codes"]), "ternary codes of the remaining weights"
    assert np.array_equal(pos.cpu().numpy(), ref["opos"]), "outlier positions"
    assert np.array_equal(val.cpu().numpy().view(np.uint16), ref["oval"]), "bf16 outlier values"
    qh, ah = q.cpu().numpy(), a.cpu().numpy()
    f = oracle.forward_with_outliers(qh, ah, codes_h, np.float32(g.cpu().numpy()[0]),
                                     pos.cpu().numpy(), val.cpu().numpy().view(np.uint16))
    assert np.array_equal(acc.cpu().numpy(), f["acc"]), "int32 accumulators (ternary part)"
    # relative fp32 rounding, plus an absolute 2^-150 per operation whose result is subnormal
    bound = ((K // 256) * k + 8) * (2.0 ** -24 * f["mag"] + 2.0 ** -150)
    err = np.abs(y.cpu().numpy().astype(np.float64) - f["y"])
    assert np.all(err <= bound), f"y: max err/bound {np.max(err / bound):.3g}"
    pw.free()


@pytest.mark.parametrize("case", range(12))
def test_repack_subnormal_walk(case):
    """Re-packs whose previous gamma is subnormal: the single-read pass brackets a subnormal
    gamma / 2, and its fixed-point scale comes from a total near 1e-33."""
    n, m = PATTERNS[case % len(PATTERNS)]
    rng = np.random.default_rng(97_500 + case)
    N = int(rng.integers(1, 600))
    K = int(rng.integers(1, 3000 // m + 1)) * m
    w0 = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    sub = (w0 * np.float32(3e-37)).astype(np.float32)  # mostly below 2^-126; gamma too
    ulps = rng.integers(-3, 4, (N, K)).astype(np.float32) * TINY
    flip = ulps.copy()
    idx = rng.choice(N * K, size=max(1, N * K // 50), replace=False)
    flip.flat[idx] = -flip.flat[idx]
    steps = [("to subnormal", sub),
             ("subnormal x1.001", (sub * np.float32(1.001)).astype(np.float32)),
             ("subnormal + noise", (sub + np.float32(1e-40) * rng.standard_normal((N, K)))
              .astype(np.float32)),
             ("multiples of 2^-149", ulps),
             ("signs flipped", flip),
             ("back", w0)]
    pw = binding.PackedWeight(gu.to_dev_f32(w0), n, m)
    _check(pw, w0, n, m, "first pack")
    for what, w in steps:
        pw.pack(gu.to_dev_f32(w))
        _check(pw, w, n, m, what)
    pw.free()


@pytest.mark.parametrize("case", range(12))
def test_repack_options_scale_jumps(case):
    """The same scale jumps with a pack option on: variance correction (the exported scale is
    gamma_out, the codes use gamma), the compact plane (its bytes), or k:256 outliers (positions,
    values and the codes of the other weights). The mask flip count of every pack is checked too."""
    import torch
    option = ["vc", "compact", "outliers"][case % 3]
    n, m = [(2, 4), (8, 16), (6, 8), (4, 8)][case % 4]
    rng = np.random.default_rng(97_800 + case)
    N = int(rng.integers(1, 400))
    K = int(rng.integers(1, 9)) * 256
    k = int(rng.choice([4, 8, 16]))
    w0 = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    mixed = w0 * np.where(rng.random((N, 1)) < 0.3, np.float32(1e30), np.float32(1e-30))
    steps = [("first pack", w0),
             ("x1e6", w0 * np.float32(1e6)),
             ("x1e6 then x1.001", w0 * np.float32(1e6) * np.float32(1.001)),
             ("x1e-6", w0 * np.float32(1e-6)),
             ("zeros", np.zeros_like(w0)),
             ("back from zero gamma", w0),
             ("subnormal", (w0 * np.float32(3e-37)).astype(np.float32)),
             ("rows of 1e30 and 1e-30", mixed.astype(np.float32)),
             ("back", w0)]
    kw = {"vc": dict(variance_correction=True), "compact": dict(compact=True),
          "outliers": dict(outliers=k)}[option]
    pw = None
    keep_prev = None
    for what, w in steps:
        if pw is None:
            pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, **kw)
        else:
            pw.pack(gu.to_dev_f32(w))
        codes_d, keep_d, gamma_d = pw.export()
        flips = pw.mask_flips()
        extra = pw.export_compact() if option == "compact" else (
            pw.export_outliers() if option == "outliers" else None)
        torch.cuda.synchronize()
        g = np.float32(gamma_d.cpu().numpy()[0])
        keep = keep_d.cpu().numpy().astype(bool)
        codes = codes_d.cpu().numpy()
        if option == "outliers":
            ref = oracle.pack_with_outliers(w, n, m, k)
            assert gu.gamma_matches(g, ref["w_rest"]), f"{what}: gamma {g} vs {ref['gamma']}"
            assert np.array_equal(keep, ref["keep"]), f"{what}: keep mask"
            assert np.array_equal(codes, oracle.ternary_codes(ref["w_rest"], ref["keep"], g)), \
                f"{what}: codes"
            pos, val = extra
            assert np.array_equal(pos.cpu().numpy(), ref["opos"]), f"{what}: outlier positions"
            assert np.array_equal(val.cpu().numpy().view(np.uint16), ref["oval"]), \
                f"{what}: outlier values"
        else:
            keep_ref = oracle.nm_keep_mask(w, n, m)
            assert np.array_equal(keep, keep_ref), f"{what}: keep mask"
            if option == "vc":
                ref = oracle.variance_correction(w, n, m)
                assert g == ref["gamma_out"], f"{what}: gamma_out {g} vs {ref['gamma_out']}"
                assert np.array_equal(codes, oracle.ternary_codes(w, keep_ref, ref["gamma"])), \
                    f"{what}: codes"
            else:
                assert gu.gamma_matches(g, w), f"{what}: gamma {g} vs {oracle.absmean_gamma(w)}"
                assert np.array_equal(codes, oracle.ternary_codes(w, keep_ref, g)), f"{what}: codes"
                assert np.array_equal(extra.cpu().numpy(), oracle.compact_pack(codes, n, m)), \
                    f"{what}: compact bytes"
        assert int(flips.cpu().numpy()[0]) == oracle.mask_flips(keep_prev, keep), \
            f"{what}: mask flips"
        keep_prev = keep
    pw.free()


@pytest.mark.parametrize("case", range(8))
def test_extreme_bwd_dx(case):
    """The straight-through data gradient dX = gamma dY codes with huge weights (gamma near 1e30)
    or with dY rows near 1e34 (small enough that no fp32 partial sum overflows), against the
    oracle within the fp32 summation bound."""
    import torch
    n, m = [(2, 4), (8, 16), (6, 8), (4, 8)][case % 4]
    rng = np.random.default_rng(99_500 + case)
    T = int(rng.integers(1, 300))
    N = int(rng.integers(1, 500))
    K = int(rng.integers(1, 2000 // m + 1)) * m
    if case % 2 == 0:
        w = (rng.standard_normal((N, K)) * 1e30).astype(np.float32)
        dy32 = rng.standard_normal((T, N)).astype(np.float32)
    else:
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        dy32 = (rng.standard_normal((T, N)) * 1e34 / max(N, 1)).astype(np.float32)
        dy32[::3] *= np.float32(1e-30)  # and rows near 1e4 / N
    dy = inputs.f32_to_bf16_bits(dy32)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
    dx = binding.bitlinear_bwd_dx(gu.to_dev_bf16(dy), pw)
    codes, _, gamma = pw.export()
    torch.cuda.synchronize()
    codes, gamma, got = codes.cpu().numpy(), np.float32(gamma.cpu().numpy()[0]), dx.cpu().numpy()
    pw.free()
    ref = oracle.ste_dx(dy, codes, gamma).astype(np.float64)
    bound = (N + 2) * 2.0 ** -24 * oracle.ste_dx_abs(dy, codes, gamma) + 2.0 ** -149
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(np.isfinite(got)), "non-finite dX"
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"


@pytest.mark.parametrize("case", range(6))
def test_extreme_group_members(case):
    """A grouped forward whose members' weights differ in scale (1e30, 0.02, mostly subnormal, all
    zero): every member equals its own forward bit for bit, and its accumulators the oracle's."""
    import torch
    n, m = [(2, 4), (8, 16), (6, 8)][case % 3]
    rng = np.random.default_rng(99_700 + case)
    T = [1, 3, 12, 40, 200, 2][case]
    K = int(rng.integers(1, 2000 // m + 1)) * m
    scales = [1e30, 0.02, 4e-39, 0.0]
    ws = [(rng.standard_normal((int(rng.integers(1, 600)), K)) * s).astype(np.float32)
          for s in scales]
    x = inputs.f32_to_bf16_bits(rng.standard_t(4, (T, K)).astype(np.float32))
    xd = gu.to_dev_bf16(x)
    pws = [binding.PackedWeight(gu.to_dev_f32(w), n, m) for w in ws]
    ys_b, q, a = binding.bitlinear_group_bf16(xd, pws, out="f32")
    acc_g = binding.bitlinear_group(q, a, pws, out="i32")
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    for s, w, pw, yb, ag in zip(scales, ws, pws, ys_b, acc_g):
        ys = binding.bitlinear(q, a, pw, out="f32")
        codes, keep, gamma = pw.export()
        torch.cuda.synchronize()
        g = np.float32(gamma.cpu().numpy()[0])
        assert gu.gamma_matches(g, w), (s, g)
        keep_ref = oracle.nm_keep_mask(w, n, m)
        assert np.array_equal(keep.cpu().numpy().astype(bool), keep_ref), s
        assert np.array_equal(codes.cpu().numpy(), oracle.ternary_codes(w, keep_ref, g)), s
        assert np.array_equal(yb.cpu().numpy(), ys.cpu().numpy()), f"grouped y vs single, {s}"
        assert np.array_equal(ag.cpu().numpy(), oracle.int_matmul(qh, codes.cpu().numpy())), s
    for pw in pws:
        pw.free()


@pytest.mark.parametrize("n,m", [(2, 4), (8, 16), (6, 8)])
def test_graph_replayed_repack_scale_jumps(n, m):
    """A re-pack captured once in a graph and replayed across the scale jumps (new weights copied
    into its input between replays, eager forwards in between): whether the fixed-point gamma sum
    is used or the fp64 partials is decided on the device, so every replay gives the oracle's gamma,
    keep mask and codes, and a forward after it matches the oracle."""
    import torch
    rng = np.random.default_rng(99_900 + 10 * n + m)
    N, K = 333, 1536
    w0 = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    steps = [w0 * np.float32(1e6), w0 * np.float32(1e6) * np.float32(1.001),
             w0 * np.float32(1e-6), np.zeros_like(w0), w0, w0 * np.float32(3e-37),
             w0 * np.float32(1.002), w0]
    x = inputs.f32_to_bf16_bits(rng.standard_normal((5, K)).astype(np.float32))
    xd = gu.to_dev_bf16(x)
    xq, a = oracle.quantize_act(x)
    wbuf = gu.to_dev_f32(w0)
    pw = binding.PackedWeight(wbuf, n, m)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pw.pack(wbuf)
    for i, w in enumerate(steps):
        w = np.asarray(w, np.float32)
        wbuf.copy_(gu.to_dev_f32(w))
        torch.cuda.synchronize()
        graph.replay()
        _check(pw, w, n, m, f"replay {i}")
        y, _, _ = binding.bitlinear_bf16(xd, pw)
        acc = oracle.int_matmul(xq, oracle.ternary_codes(w, oracle.nm_keep_mask(w, n, m),
                                                          oracle.absmean_gamma(w)))
        y_ref = oracle.dequantize(acc, oracle.absmean_gamma(w), a)
        gu.assert_y_close(y.cpu().numpy(), y_ref, f"y after replay {i}")
    pw.free()


def test_repack_near_the_fixed_point_threshold():
    """8192 fragments (4096 x 8192 weights, 2:4): re-packs after the weights shrink by 10x (the
    fixed-point sum stays in use, at about 2^45.7 units against the 2^45 floor), 20x (either side
    of the floor) and 50x (the fp64 partials), then grow back. Every gamma matches the oracle's;
    keep mask and codes of sampled rows too."""
    import torch
    n, m, N, K = 2, 4, 4096, 8192
    rng = np.random.default_rng(99_990)
    w0 = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    rows = np.sort(rng.choice(N, size=48, replace=False))
    wbuf = gu.to_dev_f32(w0)
    pw = binding.PackedWeight(wbuf, n, m)
    for f in (0.1, 0.05, 0.02, 1.0, 0.999):
        w = (w0 * np.float32(f)).astype(np.float32)
        wbuf.copy_(torch.from_numpy(w))
        pw.pack(wbuf)
        codes_d, keep_d, gamma_d = pw.export()
        torch.cuda.synchronize()
        g = np.float32(gamma_d.cpu().numpy()[0])
        assert gu.gamma_matches(g, w), f"x{f}: gamma {g} vs {oracle.absmean_gamma(w)}"
        keep_ref = oracle.nm_keep_mask(w[rows], n, m)
        assert np.array_equal(keep_d.cpu().numpy()[rows].astype(bool), keep_ref), f"x{f}: keep"
        assert np.array_equal(codes_d.cpu().numpy()[rows],
                              oracle.ternary_codes(w[rows], keep_ref, g)), f"x{f}: codes"
    pw.free()
