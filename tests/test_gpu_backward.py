"""GPU parity of the straight-through data gradient (sbn_bitlinear_bwd_dx).

dX = fl32(gamma * S) with S = sum_r dY[t][r] * code[r][k] accumulated in fp32. Every product is
exact, so the only error is fp32 summation: for any order, |S - exact| <= (n_out - 1) u sum|terms|
with u = 2^-24, and the final product by gamma adds one rounding. The test bound is
(n_out + 2) * u * gamma * sum_r |dY[t][r] * code[r][k]|, from the oracle's fp64 values.
"""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _case(seed, T, N, K):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    dy = inputs.f32_to_bf16_bits((rng.standard_normal((T, N)) * 0.5).astype(np.float32))
    return dy, w


def _check(dx, dy, codes, gamma, rows=None):
    dy_r = dy if rows is None else dy[rows]
    ref = oracle.ste_dx(dy_r, codes, gamma).astype(np.float64)
    bound = (codes.shape[0] + 2) * U * oracle.ste_dx_abs(dy_r, codes, gamma) + 1e-30
    got = dx.astype(np.float64) if rows is None else dx[rows].astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), "non-finite dX"
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"


def _run(dy, w, n, m, ld_dy=None, ld_dx=None):
    import torch
    T, N = dy.shape
    K = w.shape[1]
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
    dyd = gu.to_dev_bf16(dy, ld_dy)
    ldx = K if ld_dx is None else ld_dx
    dxbuf = torch.full((max(T, 1), ldx), 7.0, dtype=torch.float32, device="cuda")[:T]
    binding.bitlinear_bwd_dx(dyd, pw, dx=dxbuf[:, :K])
    codes, _, gamma = pw.export()
    torch.cuda.synchronize()
    out = dxbuf.cpu().numpy()
    if ldx > K:
        assert np.all(out[:, K:] == 7.0), "dX written past K"
    res = out[:, :K], codes.cpu().numpy(), np.float32(gamma.cpu().numpy()[0])
    pw.free()
    return res


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 16), (3, 8), (8, 8)])
@pytest.mark.parametrize("T,N,K", [(64, 256, 256), (130, 1032, 2048), (130, 300, 520),
                                   (17, 128, 4096)])
def test_bwd_dx_patterns(n, m, T, N, K):
    """Structured-sparse (2:4), positional (6:8, 8:16, dense) and kept (3:8) code forms; n_out a
    multiple of 128, of 8 only, and of neither (buffer and gather paths); ragged T and K."""
    K += (-K) % m
    dy, w = _case(11 * T + N + K + n, T, N, K)
    dx, codes, gamma = _run(dy, w, n, m)
    _check(dx, dy, codes, gamma)


@pytest.mark.parametrize("T,N,K", [(64, 256, 256), (130, 300, 520)])
def test_bwd_dx_24_positional(T, N, K, monkeypatch):
    """2:4 packed in the positional form (SBN_NO_SMFMAC=1 at pack time): the transposed plane is
    built from positional words, as for 6:8 and 8:16, not from the structured-sparse slots."""
    monkeypatch.setenv("SBN_NO_SMFMAC", "1")
    dy, w = _case(7 * T + N + K, T, N, K)
    dx, codes, gamma = _run(dy, w, 2, 4)
    _check(dx, dy, codes, gamma)


def test_bwd_dx_repack_rebuilds_transposed_plane():
    """A re-pack with a different mask is seen by the next data gradient."""
    import torch
    dy, w1 = _case(5, 40, 264, 512)
    _, w2 = _case(6, 40, 264, 512)
    pw = binding.PackedWeight(gu.to_dev_f32(w1), 8, 16)
    dyd = gu.to_dev_bf16(dy)
    dx1 = binding.bitlinear_bwd_dx(dyd, pw).cpu().numpy()
    c1, _, g1 = pw.export()
    dx1b = binding.bitlinear_bwd_dx(dyd, pw).cpu().numpy()
    pw.pack(gu.to_dev_f32(w2))
    dx2 = binding.bitlinear_bwd_dx(dyd, pw).cpu().numpy()
    c2, _, g2 = pw.export()
    torch.cuda.synchronize()
    assert np.array_equal(dx1, dx1b)
    _check(dx1, dy, c1.cpu().numpy(), np.float32(g1.cpu().numpy()[0]))
    _check(dx2, dy, c2.cpu().numpy(), np.float32(g2.cpu().numpy()[0]))
    assert not np.array_equal(dx1, dx2)
    pw.free()


def test_bwd_dx_padded_rows_and_nan_canaries():
    """dY rows wider than n_out whose padding holds NaN (the buffer path must not read it), odd
    leading dimensions (gather path), and dX rows wider than K."""
    dy, w = _case(21, 70, 256, 512)
    for n, m, ld_dy, ld_dx in ((2, 4, 264, 520), (6, 8, 263, 515)):
        dx, codes, gamma = _run(dy, w, n, m, ld_dy=ld_dy, ld_dx=ld_dx)
        _check(dx, dy, codes, gamma)


def test_bwd_dx_edge_cases():
    """n_out == 0 gives dX = 0; T == 0 is a no-op; a zero dY gives zeros; n_out < 16."""
    import torch
    pw = binding.PackedWeight(torch.zeros((0, 256), dtype=torch.float32, device="cuda"), 2, 4)
    dy0 = torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda")
    dx = torch.full((5, 256), 3.0, dtype=torch.float32, device="cuda")
    binding.bitlinear_bwd_dx(dy0, pw, dx=dx)
    assert torch.count_nonzero(dx).item() == 0
    pw.free()
    dy, w = _case(31, 9, 5, 64)
    dx, codes, gamma = _run(dy, w, 2, 4)
    _check(dx, dy, codes, gamma)
    dx, codes, gamma = _run(np.zeros_like(dy), w, 2, 4)
    assert np.all(dx == 0)
    dx, codes, gamma = _run(dy[:0], w, 2, 4)
    assert dx.shape == (0, 64)


def test_bwd_dx_validation():
    import ctypes
    import torch
    pw = binding.PackedWeight(torch.ones((16, 64), dtype=torch.float32, device="cuda"), 2, 4)
    dy = torch.zeros((2, 16), dtype=torch.bfloat16, device="cuda")
    dx = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    f = binding.lib().sbn_bitlinear_bwd_dx
    P = binding._ptr
    s = ctypes.c_void_p(0)
    assert f(None, P(dy), 16, 2, P(dx), 64, s) == -1
    assert f(pw.handle, P(dy), 15, 2, P(dx), 64, s) == -1   # ld_dy < n_out
    assert f(pw.handle, P(dy), 16, 2, P(dx), 63, s) == -1   # ld_dx < K
    assert f(pw.handle, P(dy), 16, -1, P(dx), 64, s) == -1  # T < 0
    assert f(pw.handle, None, 16, 2, P(dx), 64, s) == -1
    assert f(pw.handle, P(dy), 1 << 26, 2, P(dx), 64, s) == -2  # ld_dy too big
    assert f(pw.handle, P(dy), 16, 0, P(dx), 64, s) == 0
    pw.free()


@pytest.mark.parametrize("n,m", [(2, 4), (8, 16), (3, 8)])
def test_bwd_dx_512_column_tiles(n, m):
    """Launches with at least 200 tiles of 512 columns x 128 tokens run 8-wave workgroups: K = 3328
    (13 quads) leaves the last tile's second half past the transposed plane (its waves read zero
    bricks and store nothing), T = 3900 a 60-token tail, n_out = 300 a ragged last row step;
    canaries right of K."""
    T, N, K = 3900, 300, 3328
    assert -(-K // 512) * -(-T // 128) >= 200
    dy, w = _case(500 + 7 * n + m, T, N, K)
    dx, codes, gamma = _run(dy, w, n, m, ld_dx=K + 4)
    _check(dx, dy, codes, gamma)


def test_bwd_dx_7b_shapes_sampled():
    """The 7B FFN shapes at T = 8192 (the launch the benchmark times: 512-column tiles, the last
    one half past the plane for K = 11008), 2:4 and 8:16; the oracle on 24 sampled tokens."""
    import torch
    wl = inputs.W_TRAIN
    rows = np.random.default_rng(0).choice(8192, 24, replace=False)
    for li, (n, m) in ((0, (2, 4)), (1, (8, 16))):
        w = inputs.latent_weights(wl, li)
        N, K = w.shape
        rng = np.random.default_rng(40 + li)
        dy = inputs.f32_to_bf16_bits(rng.standard_normal((8192, N)).astype(np.float32))
        pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
        dx = binding.bitlinear_bwd_dx(gu.to_dev_bf16(dy), pw).cpu().numpy()
        codes, _, gamma = pw.export()
        torch.cuda.synchronize()
        _check(dx, dy, codes.cpu().numpy(), np.float32(gamma.cpu().numpy()[0]), rows=rows)
        pw.free()


@pytest.mark.parametrize("ld_dx", [(1 << 22) - 4, (1 << 22) + 4])
def test_bwd_dx_row_stride_near_2_22(ld_dx):
    """dX vector stores address the tile's rows from its first token row with 32-bit offsets while
    ld_dx < 2^22 (here up to 127 rows x (2^22 - 4) floats, just under 2^31 bytes) and fall back to
    plain stores from 2^22 on; canaries right of K stay untouched."""
    import torch
    T, N, K = 130, 264, 512
    dy, w = _case(ld_dx % 89, T, N, K)
    pw = binding.PackedWeight(gu.to_dev_f32(w), 6, 8)
    dxbuf = torch.full((T, ld_dx), 7.0, dtype=torch.float32, device="cuda")
    binding.bitlinear_bwd_dx(gu.to_dev_bf16(dy), pw, dx=dxbuf[:, :K])
    codes, _, gamma = pw.export()
    torch.cuda.synchronize()
    dx = dxbuf[:, :K].cpu().numpy()
    canary = dxbuf[:, K:K + 64].cpu().numpy()
    codes, gamma = codes.cpu().numpy(), np.float32(gamma.cpu().numpy()[0])
    del dxbuf
    pw.free()
    assert np.all(canary == 7.0)
    _check(dx, dy, codes, gamma)


@pytest.mark.parametrize("n,m", [(2, 4), (8, 16), (3, 8)])
def test_bwd_dx_after_graph_replayed_packs(n, m):
    """Whether the transposed plane matches the last pack is tracked on the device: a re-pack
    replayed from a captured graph (new weights copied into its input between replays) followed
    by an eager data gradient, and a captured data gradient replayed after eager and replayed
    packs, all give the data gradient of the weights the handle holds at that moment. Eager work
    runs between the replays; every result is checked against the oracle."""
    import torch
    rng = np.random.default_rng(500 + 10 * n + m)
    T, N, K = 130, 300, 1040
    K += (-K) % m
    ws = [(rng.standard_normal((N, K)) * 0.02).astype(np.float32) for _ in range(6)]
    dy = inputs.f32_to_bf16_bits((rng.standard_normal((T, N)) * 0.5).astype(np.float32))
    dyd = gu.to_dev_bf16(dy)
    wbuf = gu.to_dev_f32(ws[0])
    pw = binding.PackedWeight(wbuf, n, m)
    dxbuf = torch.empty((T, K), dtype=torch.float32, device="cuda")

    def check(w, what):
        codes, _, gamma = pw.export()
        torch.cuda.synchronize()
        codes_h, g = codes.cpu().numpy(), np.float32(gamma.cpu().numpy()[0])
        assert gu.gamma_matches(g, w), f"{what}: gamma"
        # the oracle's codes at the gamma the kernels used (they differ from the oracle's own
        # gamma only at an fp32 rounding midpoint of the mean)
        ref = oracle.ternary_codes(w, oracle.nm_keep_mask(w, n, m), g)
        assert np.array_equal(codes_h, ref), f"{what}: codes"
        _check(dxbuf.cpu().numpy(), dy, codes_h, g)

    binding.bitlinear_bwd_dx(dyd, pw, dx=dxbuf)
    check(ws[0], "eager")
    g_pack = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_pack):
        pw.pack(wbuf)
    for i in (1, 2):
        wbuf.copy_(gu.to_dev_f32(ws[i]))
        torch.cuda.synchronize()
        g_pack.replay()
        binding.bitlinear_bwd_dx(dyd, pw, dx=dxbuf)
        check(ws[i], f"replayed pack {i}, eager data gradient")
    g_bwd = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_bwd):
        binding.bitlinear_bwd_dx(dyd, pw, dx=dxbuf)
    wbuf.copy_(gu.to_dev_f32(ws[3]))
    torch.cuda.synchronize()
    g_pack.replay()
    dxbuf.zero_()
    g_bwd.replay()
    check(ws[3], "replayed pack, replayed data gradient")
    dxbuf.zero_()
    g_bwd.replay()
    check(ws[3], "replayed data gradient again (plane reused)")
    pw.pack(gu.to_dev_f32(ws[4]))
    dxbuf.zero_()
    g_bwd.replay()
    check(ws[4], "eager pack, replayed data gradient")
    wbuf.copy_(gu.to_dev_f32(ws[5]))
    torch.cuda.synchronize()
    g_pack.replay()
    binding.bitlinear_bwd_dx(dyd, pw, dx=dxbuf)
    check(ws[5], "replayed pack after the eager one, eager data gradient")
    pw.free()
