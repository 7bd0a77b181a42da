"""GPU parity of the compact inference form (sbn_pack_nm_ternary_ex with SBN_PACK_COMPACT).

The pack writes, next to the 2-bit codes, a plane that keeps only the nonzero positions and their
signs; the GEMV launches (T <= 16) then read it. Integer work, so everything is bit-exact: the
exported compact streams equal the oracle's encoding of the oracle's codes, the int32 accumulators
equal the oracle's, and every forward output equals the one from the same weights packed without
the flag (same accumulators, same scale, same dequantization).
"""

import ctypes

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

PATTERNS = [(2, 4), (6, 8), (8, 16), (3, 8), (1, 4), (8, 8), (12, 16), (4, 8), (16, 16), (5, 16)]


def _w(seed, N, K):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w *= rng.uniform(0.5, 2.0, (N, 1)).astype(np.float32)  # row scales: uneven zero shares
    return w


def _x(seed, T, K):
    rng = np.random.default_rng(seed)
    return inputs.f32_to_bf16_bits(rng.standard_t(4, (T, K)).astype(np.float32))


@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("N,K", [(70, 1040), (16, 256), (300, 2560), (33, 64)])
def test_compact_export(n, m, N, K):
    """The plane's bits: exported streams equal oracle.compact_pack of the oracle's codes (rows
    past a fragment, K ending inside a quad, a single brick)."""
    import torch
    K += (-K) % m
    w = _w(N * 7 + K + 13 * n + m, N, K)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, compact=True)
    data = pw.export_compact()
    codes, _, _ = pw.export()
    d = pw.query()
    torch.cuda.synchronize()
    ref = oracle.pack_nm_ternary(w, n, m)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert d.compact == 1 and d.compact_row_bytes == oracle.compact_row_bytes(n, m, K)
    assert np.array_equal(data.cpu().numpy(), oracle.compact_pack(ref["codes"], n, m))
    pw.free()


def _forward_pair(x, w, n, m, T, ln=False):
    """Every forward output through a compact handle and through a plain one."""
    import torch
    xd = gu.to_dev_bf16(x)
    out = {}
    for tag, cmp in (("c", True), ("p", False)):
        pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, compact=cmp)
        q, a = binding.quantize_act(xd)
        r = dict(y=binding.bitlinear(q, a, pw, out="f32"), acc=binding.bitlinear(q, a, pw, out="i32"))
        if T <= 16:
            r["yb"] = binding.bitlinear_bf16(xd, pw)[0]
            if ln:
                r["yl"] = binding.bitlinear_bf16(xd, pw, ln_eps=1e-5)[0]
        codes, _, g = pw.export()
        torch.cuda.synchronize()
        out[tag] = {k: v.cpu().numpy() for k, v in r.items()}
        out[tag]["codes"] = codes.cpu().numpy()
        out[tag]["gamma"] = np.float32(g.cpu().numpy()[0])
        out[tag]["q"], out[tag]["a"] = q.cpu().numpy(), a.cpu().numpy()
        pw.free()
    return out["c"], out["p"]


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 16), (3, 8), (1, 4), (8, 8), (12, 16)])
@pytest.mark.parametrize("T", [1, 2, 4, 5, 16])
def test_compact_forward(n, m, T):
    """GEMV (int8 and one-kernel bf16 inputs) on the compact plane: accumulators equal the
    oracle's, outputs equal the plain handle's bit for bit."""
    K, N = 2560, 200
    x = _x(T * 3 + n + m, T, K)
    w = _w(T + 11 * n + m, N, K)
    c, p = _forward_pair(x, w, n, m, T, ln=(T <= 4))
    q_ref, a_ref = oracle.quantize_act(x)
    assert np.array_equal(c["q"], q_ref) and np.array_equal(c["a"], a_ref)
    assert np.array_equal(c["acc"], oracle.int_matmul(q_ref, c["codes"]))
    gu.assert_y_close(c["y"], oracle.dequantize(c["acc"], c["gamma"], a_ref))
    for k in ("y", "acc", "yb") + (("yl",) if T <= 4 else ()):
        assert np.array_equal(c[k], p[k]), k


@pytest.mark.parametrize("K", [64, 320, 1040, 4096, 12288, 12544])
def test_compact_forward_k_range(K):
    """One quad up to the GEMV's 48 quads (three per wave), a K tail inside a brick, and K past
    the GEMV limit (the GEMM, which reads the 2-bit codes, serves the call)."""
    n, m = 6, 8
    K += (-K) % m
    x = _x(K, 3, K)
    w = _w(K + 1, 70, K)
    c, p = _forward_pair(x, w, n, m, 3, ln=True)
    q_ref, _ = oracle.quantize_act(x)
    assert np.array_equal(c["acc"], oracle.int_matmul(q_ref, c["codes"]))
    for k in ("y", "acc", "yb", "yl"):
        assert np.array_equal(c[k], p[k]), k


def test_compact_large_t_uses_gemm():
    """T > 16 goes to the GEMM on the 2-bit codes; results equal the plain handle's."""
    x = _x(5, 40, 1024)
    w = _w(6, 300, 1024)
    c, p = _forward_pair(x, w, 8, 16, 40)
    assert np.array_equal(c["acc"], p["acc"]) and np.array_equal(c["y"], p["y"])


def test_compact_repack_toggle():
    """The flag follows each pack: the plane is rewritten from new weights, export is refused
    after a pack without the flag, and the GEMV then reads the 2-bit codes."""
    import torch
    n, m, N, K = 8, 16, 140, 2048
    w1, w2 = _w(1, N, K), _w(2, N, K)
    x = _x(3, 2, K)
    xd = gu.to_dev_bf16(x)
    pw = binding.PackedWeight(gu.to_dev_f32(w1), n, m, compact=True)
    pw.pack(gu.to_dev_f32(w2))  # still compact
    data = pw.export_compact().cpu().numpy()
    ref2 = oracle.pack_nm_ternary(w2, n, m)
    assert np.array_equal(data, oracle.compact_pack(ref2["codes"], n, m))
    y_c = binding.bitlinear_bf16(xd, pw)[0].cpu().numpy()
    pw.pack(gu.to_dev_f32(w2), compact=False)
    assert pw.query().compact == 0
    with pytest.raises(binding.SbnError):
        pw.export_compact()
    y_p = binding.bitlinear_bf16(xd, pw)[0].cpu().numpy()
    pw.pack(gu.to_dev_f32(w1), compact=True)
    data1 = pw.export_compact().cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(y_c, y_p)
    assert np.array_equal(data1, oracle.compact_pack(oracle.pack_nm_ternary(w1, n, m)["codes"], n, m))
    pw.free()


def test_compact_with_variance_correction_and_flips():
    """Both flags together: gamma_out scales the compact GEMV; the flip count is unaffected."""
    import torch
    n, m, N, K = 6, 8, 96, 1024
    w = _w(9, N, K)
    x = _x(10, 4, K)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, variance_correction=True, compact=True)
    y = binding.bitlinear_bf16(gu.to_dev_bf16(x), pw, out="f32")[0].cpu().numpy()
    f = pw.mask_flips()
    torch.cuda.synchronize()
    ref = oracle.variance_correction(w, n, m)
    q_ref, a_ref = oracle.quantize_act(x)
    codes = oracle.pack_nm_ternary(w, n, m)["codes"]
    gu.assert_y_close(y, oracle.dequantize(oracle.int_matmul(q_ref, codes), ref["gamma_out"], a_ref))
    assert int(f.cpu().numpy()[0]) == int(oracle.nm_keep_mask(w, n, m).sum())
    pw.free()


def test_compact_edge_cases():
    """All-zero weights, n_out < 16, n_out == 0."""
    import torch
    for N, K in ((5, 64), (1, 512)):
        w = np.zeros((N, K), np.float32)
        pw = binding.PackedWeight(gu.to_dev_f32(w), 2, 4, compact=True)
        data = pw.export_compact().cpu().numpy()
        y = binding.bitlinear_bf16(gu.to_dev_bf16(_x(1, 2, K)), pw, out="i32")[0].cpu().numpy()
        torch.cuda.synchronize()
        assert not data.any() and not y.any()
        pw.free()
    w = _w(4, 7, 256)
    c, _ = _forward_pair(_x(2, 1, 256), w, 2, 4, 1)
    q_ref, _ = oracle.quantize_act(_x(2, 1, 256))
    assert np.array_equal(c["acc"], oracle.int_matmul(q_ref, c["codes"]))
    pw = binding.PackedWeight(torch.zeros((0, 256), dtype=torch.float32, device="cuda"), 2, 4,
                              compact=True)
    assert pw.export_compact().shape == (0, oracle.compact_row_bytes(2, 4, 256))
    pw.free()


def test_compact_validation():
    import torch
    pw = binding.PackedWeight(torch.ones((16, 64), dtype=torch.float32, device="cuda"), 2, 4)
    out = torch.zeros((16, 8), dtype=torch.uint8, device="cuda")
    f = binding.lib().sbn_packed_export_compact
    assert f(pw.handle, binding._ptr(out), ctypes.c_void_p(0)) == -1  # not packed compact
    pw.pack(torch.ones((16, 64), dtype=torch.float32, device="cuda"), compact=True)
    assert f(pw.handle, None, ctypes.c_void_p(0)) == -1
    assert f(pw.handle, binding._ptr(out), ctypes.c_void_p(0)) == 0
    pw.free()


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 16)])
def test_compact_decode_shape(n, m):
    """The 2560 -> 6912 decode projection at T = 1 and 16 (the launches the benchmark times):
    accumulators equal the oracle's, exported streams equal the oracle's encoding."""
    import torch
    wl = inputs.W_DECODE
    w = inputs.latent_weights(wl, 0)
    K = w.shape[1]
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, compact=True)
    data = pw.export_compact()
    codes, _, _ = pw.export()
    torch.cuda.synchronize()
    codes = codes.cpu().numpy()
    assert np.array_equal(data.cpu().numpy(), oracle.compact_pack(codes, n, m))
    for T in (1, 16):
        x = inputs.activations(wl, 0, T, K)
        xd = gu.to_dev_bf16(x)
        q, a = binding.quantize_act(xd)
        acc = binding.bitlinear(q, a, pw, out="i32").cpu().numpy()
        q_ref, _ = oracle.quantize_act(x)
        assert np.array_equal(acc, oracle.int_matmul(q_ref, codes))
        if T == 1:
            y = binding.bitlinear_bf16(xd, pw, out="i32")[0].cpu().numpy()
            assert np.array_equal(y, acc)
    pw.free()
