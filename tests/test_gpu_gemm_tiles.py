"""GPU parity of the GEMM's tile shapes (T > 16). A launch that fits one round of 8-wave
workgroups on 512 rows (200 to 256 tiles of 128, 96 or 64 tokens) takes the widest such
tile. Otherwise launches whose 128-token tiles number more than 256 use them (on 512 rows with 8
waves when those tiles number at least 200); smaller
launches use 64-token tiles (split over K as well while they still number at most 256). Integer
accumulators equal the oracle's exactly; fp32 outputs follow it within the forward's tolerance;
the fp32 scale of each token comes from the tile's LDS copy of a'_t."""

import numpy as np
import pytest

from tests import gpu_util as gu
from sparsity_sbn_quantize_amd import inputs

pytestmark = pytest.mark.gpu


def _case(seed, T, K, N):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(4, (T, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return inputs.f32_to_bf16_bits(x), w


def tiles128(T, N):
    return -(-N // 256) * -(-T // 128)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (3, 8), (8, 16)])
@pytest.mark.parametrize("T", [1930, 1920])
def test_tile_width_boundary(n, m, T):
    """N = 4352 (17 row tiles): T = 1930 gives 272 tiles of 128 tokens, with a 10-token tail;
    T = 1920 gives 255, so the launch takes 64-token tiles (510 of them, no split)."""
    N, K = 4352, 1040 - 1040 % m
    assert (tiles128(T, N) > 256) == (T == 1930)
    x, w = _case(T + 31 * n + m, T, K, N)
    g = gu.gpu_forward(x, w, n, m)
    gu.check_stages(g, x, w, n, m)


def tiles512(T, N):
    return -(-N // 512) * -(-T // 128)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 16), (3, 8)])
def test_512_row_tiles(n, m):
    """Launches with at least 200 tiles of 512 rows x 128 tokens run 8-wave workgroups (the
    positional and 2:4 forms): N = 4352 makes the last row tile half empty (its waves past the
    stored plane read zero bricks and store nothing), T = 2900 a 84-token tail. 3:8 (kept form)
    keeps 256-row tiles at the same size."""
    T, N, K = 2900, 4352, 1040 - 1040 % m
    assert tiles512(T, N) >= 200
    x, w = _case(7 * n + m, T, K, N)
    g = gu.gpu_forward(x, w, n, m)
    gu.check_stages(g, x, w, n, m)


def one_round_cf(T, N):
    """Token-tile width (in 16-token fragments) of the one-round 8-wave launch, or None."""
    for cf in (8, 6, 4):
        tiles = -(-N // 512) * -(-T // (16 * cf))
        if 200 <= tiles <= 256:
            return cf
    return None


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 16)])
@pytest.mark.parametrize("T,K,cf", [(4091, 528, 6), (2600, 1040, 4)])
def test_one_round_512_row_tiles(n, m, T, K, cf):
    """One round of 8-wave workgroups on 512 rows where 128-token tiles would leave CUs idle:
    96-token tiles (T = 4091: 43 token tiles, a 59-token tail) and 64-token tiles (T = 2600: 41,
    a 40-token tail). N = 2304 makes the last row tile half empty."""
    N = 2304
    assert one_round_cf(T, N) == cf
    x, w = _case(T + 13 * n + m, T, K - K % m, N)
    g = gu.gpu_forward(x, w, n, m)
    gu.check_stages(g, x, w, n, m)


def test_wide_tiles_unaligned():
    """128-token tiles with element-wise activation loads (odd leading dimensions of x, w and
    x_q) and a ragged last row tile (4200 rows)."""
    T, K, N = 2100, 528, 4200
    assert tiles128(T, N) > 256
    x, w = _case(5, T, K, N)
    g = gu.gpu_forward(x, w, 6, 8, ld_x=K + 3, ld_w=K + 1, ld_q=K + 5)
    gu.check_stages(g, x, w, 6, 8)


@pytest.mark.parametrize("ld_y", [(1 << 22) - 4, (1 << 22) + 4])
def test_output_row_stride_near_2_22(ld_y):
    """The vector output stores address the tile's rows from its first token row with 32-bit
    offsets while ld_y < 2^22 (here up to 127 rows x (2^22 - 4) floats, just under 2^31 bytes),
    and fall back to plain stores from 2^22 on. 128-token tiles (33024 rows, T = 130: 258 tiles),
    fp32 and int32 outputs, canaries right of n_out."""
    import torch
    from sparsity_sbn_quantize_amd import binding
    import oracle
    T, K, N = 130, 64, 33024
    assert tiles128(T, N) > 256
    x, w = _case(ld_y % 97, T, K, N)
    xd = gu.to_dev_bf16(x)
    q, a = binding.quantize_act(xd)
    pw = binding.PackedWeight(gu.to_dev_f32(w), 6, 8)
    codes, _, g = pw.export()
    acc_ref = oracle.int_matmul(q.cpu().numpy(), codes.cpu().numpy())
    ybuf = torch.full((T, ld_y), -7.0, dtype=torch.float32, device="cuda")
    binding.bitlinear(q, a, pw, out="f32", y=ybuf[:, :N])
    y = ybuf[:, :N].cpu().numpy()
    canary = ybuf[:, N:N + 64].cpu().numpy()
    gu.assert_y_close(y, oracle.dequantize(acc_ref, np.float32(g.cpu().numpy()[0]),
                                           a.cpu().numpy()))
    assert np.all(canary == -7.0)
    yi = ybuf.view(torch.int32)
    yi.fill_(-7)
    binding.bitlinear(q, a, pw, out="i32", y=yi[:, :N])
    assert np.array_equal(yi[:, :N].cpu().numpy(), acc_ref)
    assert np.all(yi[:, N:N + 64].cpu().numpy() == -7)
    del ybuf, yi
    pw.free()
    torch.cuda.synchronize()
