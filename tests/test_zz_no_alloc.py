"""The entry point that allocates nothing (sbn_bitlinear_fwd_latent_static): the pack of the latent
weights and the forward, with the packed planes in the library's fixed device workspace. Its
outputs must equal those of sbn_pack_nm_ternary followed by sbn_bitlinear_fwd bit for bit (int32
accumulators and fp32 outputs), on calls in a row whose later inputs are smaller (the workspace
keeps the earlier call's contents) or whose weights differ in scale by up to 1e69 (each call packs
afresh), through the GEMV, the GEMM and the split-K GEMM, and inside a captured graph replayed
several times. Sizes beyond the workspace are rejected on the host."""

import ctypes

import numpy as np
import pytest

from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu


def _case(seed, T, K, N):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return inputs.f32_to_bf16_bits(x), w


def _handle_path(wd, n, m, q, a, kind):
    pw = binding.PackedWeight(wd, n, m)
    y = binding.bitlinear(q, a, pw, out=kind)
    return pw, y


def test_static_rejects_sizes_beyond_the_workspace():
    """Host-side checks, before any HIP call (no GPU needed)."""
    lib = binding.lib()
    p = ctypes.c_void_p(64)
    # 12288 x 8192 at 2:4 is about 100M weights: its planes do not fit 32 MiB
    assert lib.sbn_bitlinear_fwd_latent_static(p, 12288, 8192, 8192, 2, 4, p, 8192, p, 1, p,
                                               12288, 0, None) == -2
    assert "workspace" in binding.last_error()
    assert lib.sbn_bitlinear_fwd_latent_static(p, 16, 64, 64, 5, 4, p, 64, p, 1, p, 16, 0,
                                               None) == -2
    assert lib.sbn_bitlinear_fwd_latent_static(p, 16, 60, 64, 6, 8, p, 64, p, 1, p, 16, 0,
                                               None) == -1
    assert lib.sbn_bitlinear_fwd_latent_static(p, 16, 64, 64, 2, 4, p, 64, p, 1, p, 8, 0,
                                               None) == -1
    assert lib.sbn_bitlinear_fwd_latent_static(None, 16, 64, 64, 2, 4, p, 64, p, 1, p, 16, 0,
                                               None) == -1
    # the largest 7B-style layer fits: validation passes and T = 0 returns before any HIP call
    assert lib.sbn_bitlinear_fwd_latent_static(p, 11008, 4096, 4096, 2, 4, p, 4096, p, 0, p,
                                               11008, 0, None) == 0


@pytest.mark.gpu
def test_static_equals_handle_path_on_calls_in_a_row():
    import torch
    # (T, K, N, n, m): a GEMM, a smaller split-K GEMM (2 x 3 tiles, 8 K steps), a one-token GEMV,
    # each smaller than the one before
    cases = [(300, 4096, 1100, 2, 4), (150, 2048, 300, 8, 16), (1, 1024, 200, 6, 8),
             (5, 512, 40, 3, 8)]
    for i, (T, K, N, n, m) in enumerate(cases):
        x, w = _case(40 + i, T, K, N)
        xd, wd = gu.to_dev_bf16(x), gu.to_dev_f32(w)
        q, a = binding.quantize_act(xd)
        print(f"[static] call {i}: T={T} K={K} N={N} {n}:{m}", flush=True)
        for kind in ("i32", "f32"):
            ys = binding.bitlinear_latent_static(wd, n, m, q, a, out=kind)
            pw, yh = _handle_path(wd, n, m, q, a, kind)
            torch.cuda.synchronize()
            assert np.array_equal(ys.cpu().numpy(), yh.cpu().numpy()), (i, kind)
            pw.free()


@pytest.mark.gpu
def test_static_calls_across_weight_scales():
    """Calls in a row on weights of very different scales (1e30, 0.02, mostly fp32 subnormals, all
    zero, 0.02 again): each call packs afresh from its own weights, so every call equals the
    handle path bit for bit, and the handle's gamma, keep mask and codes equal the oracle's."""
    import torch
    import oracle
    T, K, N, n, m = 40, 1024, 300, 6, 8
    for i, scale in enumerate([1e30, 0.02, 4e-39, 0.0, 0.02]):
        x, w = _case(60 + i, T, K, N)
        w = (w * np.float32(scale / 0.02)).astype(np.float32)
        xd, wd = gu.to_dev_bf16(x), gu.to_dev_f32(w)
        q, a = binding.quantize_act(xd)
        print(f"[static] scale {scale:g}", flush=True)
        for kind in ("i32", "f32"):
            ys = binding.bitlinear_latent_static(wd, n, m, q, a, out=kind)
            pw, yh = _handle_path(wd, n, m, q, a, kind)
            codes, keep, gamma = pw.export()
            torch.cuda.synchronize()
            assert np.array_equal(ys.cpu().numpy(), yh.cpu().numpy()), (scale, kind)
            g = np.float32(gamma.cpu().numpy()[0])
            assert gu.gamma_matches(g, w), (scale, g, oracle.absmean_gamma(w))
            keep_ref = oracle.nm_keep_mask(w, n, m)
            assert np.array_equal(keep.cpu().numpy().astype(bool), keep_ref), scale
            assert np.array_equal(codes.cpu().numpy(), oracle.ternary_codes(w, keep_ref, g)), scale
            pw.free()


@pytest.mark.gpu
def test_static_in_a_captured_graph():
    """Captured once, replayed with eager work and synchronizations between the replays (and
    another static call of another shape, which rewrites the workspace): every replay equals the
    handle path."""
    import torch
    T, K, N, n, m = 150, 2048, 300, 6, 8
    x, w = _case(7, T, K, N)
    xd, wd = gu.to_dev_bf16(x), gu.to_dev_f32(w)
    q, a = binding.quantize_act(xd)
    pw, ref = _handle_path(wd, n, m, q, a, "f32")
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    binding.bitlinear_latent_static(wd, n, m, q, a, out="f32", y=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.bitlinear_latent_static(wd, n, m, q, a, out="f32", y=y)
    x2, w2 = _case(8, 3, 1024, 64)
    xd2, wd2 = gu.to_dev_bf16(x2), gu.to_dev_f32(w2)
    q2, a2 = binding.quantize_act(xd2)
    for _ in range(3):
        y.zero_()
        binding.bitlinear_latent_static(wd2, 2, 4, q2, a2, out="f32")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
    pw.free()
