"""GPU parity of the quantize-and-multiply entry point (sbn_bitlinear_fwd_bf16).

For T <= 4 and K <= 12288 it is one kernel in which every workgroup quantizes the activations it
needs; otherwise it runs the quantize kernel and the matmul in turn. Either way its int8
activations and a' must equal sbn_quantize_act's byte for byte, its int32 accumulators and fp32
outputs must equal those of the two-call path bit for bit, and all of them must match the oracle
(int8 values exactly, up to counted rounding boundaries; fp32 within 1e-5 relative).
"""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case(seed, T, K, N):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(4, (T, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return inputs.f32_to_bf16_bits(x), w


def _run(x_bits, w, n, m, ld_x=None, ld_q=None):
    import torch
    T, K = x_bits.shape
    xd = gu.to_dev_bf16(x_bits, ld_x)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
    ldq = K if ld_q is None else ld_q
    out = {}
    for kind in ("f32", "i32"):
        qbuf = torch.full((max(T, 1), ldq), 77, dtype=torch.int8, device="cuda")[:T]
        a = torch.full((T,), -1.0, dtype=torch.float32, device="cuda")
        y, _, _ = binding.bitlinear_bf16(xd, pw, out=kind, x_q=qbuf[:, :K], x_absmax=a)
        out[kind] = (y.cpu().numpy(), qbuf.cpu().numpy(), a.cpu().numpy())
    # the two-call path on the same inputs
    q2, a2 = binding.quantize_act(xd)
    y2 = binding.bitlinear(q2, a2, pw, out="f32")
    acc2 = binding.bitlinear(q2, a2, pw, out="i32")
    codes, _, gamma = pw.export()
    torch.cuda.synchronize()
    res = dict(y=out["f32"][0], acc=out["i32"][0], q_pad=out["f32"][1], a=out["f32"][2],
               q_pad_i32=out["i32"][1], a_i32=out["i32"][2], q2=q2.cpu().numpy(),
               a2=a2.cpu().numpy(), y2=y2.cpu().numpy(), acc2=acc2.cpu().numpy(),
               codes=codes.cpu().numpy(), gamma=np.float32(gamma.cpu().numpy()[0]))
    pw.free()
    return res


def _check(r, x_bits, K):
    q = r["q_pad"][:, :K]
    # identical to sbn_quantize_act, and nothing written past column K
    assert np.array_equal(q, r["q2"]), "x_q differs from sbn_quantize_act"
    assert np.array_equal(r["a"], r["a2"]), "a' differs from sbn_quantize_act"
    assert np.array_equal(r["q_pad_i32"][:, :K], r["q2"]) and np.array_equal(r["a_i32"], r["a2"])
    if r["q_pad"].shape[1] > K:
        assert np.all(r["q_pad"][:, K:] == 77), "x_q written past K"
    # identical to the two-call path
    assert np.array_equal(r["acc"], r["acc2"]), "int32 accumulators differ from the two-call path"
    assert np.array_equal(r["y"], r["y2"]), "fp32 output differs from the two-call path"
    # against the oracle
    q_ref, a_ref = oracle.quantize_act(x_bits)
    assert np.array_equal(r["a"], a_ref), "absmax"
    gu.assert_int_exact_except_boundary(q, q_ref, oracle.boundary_elements_act(x_bits, a_ref),
                                        "int8 activations")
    acc_ref = oracle.int_matmul(q, r["codes"])
    assert np.array_equal(r["acc"], acc_ref), "int32 accumulators vs oracle"
    gu.assert_y_close(r["y"], oracle.dequantize(acc_ref, r["gamma"], r["a"]))


@pytest.mark.parametrize("n,m", [(6, 8), (8, 16), (2, 4), (8, 8), (3, 8)])
@pytest.mark.parametrize("T", [1, 3, 4, 9, 16])
@pytest.mark.parametrize("K", [2560, 264, 96])
def test_fused_patterns(n, m, T, K):
    """Several patterns (positional codes and the kept form 3:8); T <= 4 (one kernel) and
    T = 9, 16 (quantize kernel, then GEMV); K a multiple of 256, of 8 but not 16 (264), and
    below one 256-K quad (96)."""
    K += (-K) % m  # 264 -> 272 for m = 16 (K must be a multiple of m)
    x, w = _case(1000 + 7 * T + K + n, T, K, 200)
    _check(_run(x, w, n, m), x, K)


def test_fused_decode_shape():
    """The 2B-style up projection at T = 1 and 16 (6:8, K = 2560 -> N = 6912)."""
    wl = inputs.W_DECODE
    w = inputs.latent_weights(wl, 0)
    for T in (1, 16):
        x = inputs.activations(wl, 0, T, w.shape[1])
        _check(_run(x, w, 6, 8), x, w.shape[1])


def test_fused_unaligned_and_padded():
    """Odd leading dimensions (element loads instead of vector loads) and x_q rows wider than K."""
    x, w = _case(11, 3, 520, 90)
    _check(_run(x, w, 6, 8, ld_x=523, ld_q=531), x, 520)
    x, w = _case(13, 4, 520, 90)
    _check(_run(x, w, 2, 4, ld_x=522, ld_q=530), x, 520)
    x, w = _case(12, 16, 2560, 64)
    _check(_run(x, w, 8, 16, ld_x=2568, ld_q=2576), x, 2560)


def test_fused_fallbacks():
    """T > 16 and K > 12288 run the two kernels; the results are the same. K in (8192, 12288]
    exercises three quads per wave."""
    x, w = _case(21, 40, 1024, 130)
    _check(_run(x, w, 8, 16), x, 1024)
    x, w = _case(22, 2, 12544, 48)
    _check(_run(x, w, 6, 8), x, 12544)
    x, w = _case(23, 3, 11008, 40)
    _check(_run(x, w, 8, 16), x, 11008)


def test_fused_edge_cases():
    """Zero rows (a' floored at 1e-5), n_out < 16, and n_out == 0 (x_q and a' still written)."""
    x, w = _case(31, 4, 512, 5)
    x[1] = 0
    _check(_run(x, w, 2, 4), x, 512)
    import torch
    xd = gu.to_dev_bf16(x)
    pw = binding.PackedWeight(torch.zeros((0, 512), dtype=torch.float32, device="cuda"), 2, 4)
    y, q, a = binding.bitlinear_bf16(xd, pw)
    q_ref, a_ref = oracle.quantize_act(x)
    assert y.shape == (4, 0)
    assert np.array_equal(a.cpu().numpy(), a_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    pw.free()


def test_fused_validation():
    """Leading dimensions and pointers are checked before any launch."""
    import ctypes
    import torch
    x, w = _case(41, 2, 256, 32)
    xd = gu.to_dev_bf16(x)
    pw = binding.PackedWeight(gu.to_dev_f32(w), 6, 8)
    q = torch.empty((2, 256), dtype=torch.int8, device="cuda")
    a = torch.empty((2,), dtype=torch.float32, device="cuda")
    y = torch.empty((2, 32), dtype=torch.float32, device="cuda")
    f = binding.lib().sbn_bitlinear_fwd_bf16
    P = binding._ptr
    s = ctypes.c_void_p(0)
    assert f(pw.handle, P(xd), 255, 2, P(q), 256, P(a), P(y), 32, 0, s) == -1  # ld_x < K
    assert f(pw.handle, P(xd), 256, 2, P(q), 255, P(a), P(y), 32, 0, s) == -1  # ld_q < K
    assert f(pw.handle, P(xd), 256, 2, P(q), 1 << 27, P(a), P(y), 32, 0, s) == -2  # ld_q too big
    assert f(pw.handle, P(xd), 256, 2, P(q), 256, P(a), P(y), 31, 0, s) == -1  # ld_y < n_out
    assert f(pw.handle, P(xd), 256, 2, None, 256, P(a), P(y), 32, 0, s) == -1  # null x_q
    assert f(pw.handle, P(xd), 256, 2, P(q), 256, P(a), P(y), 32, 7, s) == -1  # out_kind
    assert f(pw.handle, P(xd), 256, 0, P(q), 256, P(a), P(y), 32, 0, s) == 0   # T == 0
    pw.free()


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 16)])
@pytest.mark.parametrize("T", [5, 9, 16])
@pytest.mark.parametrize("N,K", [(10480, 1024), (5130, 4096), (6912, 2560)])
def test_fused_wide_5_to_16_tokens(n, m, T, N, K):
    """Five to sixteen tokens on layers of 320 or more row blocks and at most 16 quads: the
    quantize kernel, then the row-block-sharing GEMV (two row blocks per workgroup, three from
    640 on; 10480 rows end past the stored plane's last workgroup, 5130 inside a row block).
    x_q and a' equal sbn_quantize_act's, outputs the two-call path's."""
    x, w = _case(2000 + 3 * T + N + K + n, T, K, N)
    _check(_run(x, w, n, m), x, K)


def test_fused_wide_padded_and_unaligned():
    """The same shapes with x_q rows wider than K (nothing written past K) and x leading
    dimensions wider than K."""
    x, w = _case(51, 16, 2560, 5136)
    _check(_run(x, w, 6, 8, ld_q=2576), x, 2560)
    _check(_run(x, w, 6, 8, ld_x=2568), x, 2560)
    _check(_run(x, w, 6, 8, ld_x=2570), x, 2560)
