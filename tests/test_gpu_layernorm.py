"""GPU parity of the parameter-free LayerNorm + INT8 quantization (sbn_layernorm_quantize_act).

Both sides take the same steps (fp64 statistics, fp32 normalization, bf16 rounding, then the
absmax quantizer), so x_q and a' must equal the oracle's exactly; the GPU's fp64 summation order
differs from the oracle's, which could change a last fp64 bit of the variance and, in rare rows,
one fp32 value of 1/sqrt(var + eps) (not seen in these cases). The call must also equal
sbn_quantize_act applied to the oracle's bf16 LayerNorm output.
"""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _x(seed, T, K, kind):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = rng.standard_normal((T, K)).astype(np.float32) * 3 + 1
    elif kind == "student_t":
        x = rng.standard_t(4, (T, K)).astype(np.float32)
    elif kind == "outliers":
        x = rng.standard_normal((T, K)).astype(np.float32)
        x[:, rng.choice(K, max(1, K // 1000), replace=False)] *= 20
    elif kind == "narrow":  # variance below eps
        x = rng.standard_normal((T, K)).astype(np.float32) * 1e-3
    else:  # constant rows and a zero row
        x = np.tile(rng.standard_normal((T, 1)).astype(np.float32), (1, K))
        x[0] = 0
    return inputs.f32_to_bf16_bits(x)


def _run(x, eps, ld_x=None, ld_q=None):
    import torch
    T, K = x.shape
    xd = gu.to_dev_bf16(x, ld_x)
    ldq = K if ld_q is None else ld_q
    qbuf = torch.full((max(T, 1), ldq), 77, dtype=torch.int8, device="cuda")[:T]
    a = torch.empty((T,), dtype=torch.float32, device="cuda")
    binding.layernorm_quantize_act(xd, eps, out_q=qbuf[:, :K], out_absmax=a)
    torch.cuda.synchronize()
    q = qbuf.cpu().numpy()
    if ldq > K:
        assert np.all(q[:, K:] == 77), "x_q written past K"
    return q[:, :K], a.cpu().numpy()


@pytest.mark.parametrize("kind", ["normal", "student_t", "outliers", "narrow", "constant"])
@pytest.mark.parametrize("T,K", [(8, 256), (17, 2560), (300, 6912), (5, 520), (3, 523),
                                 (2, 20000), (1, 8)])
def test_layernorm_quantize(kind, T, K):
    """Both vector paths (64 and 256 threads per row) and the general path (K % 8 != 0, K >
    16384); heavy tails, outlier channels, variance below eps, constant rows."""
    x = _x(1000 + T + K, T, K, kind)
    q, a = _run(x, 1e-5)
    q_ref, a_ref = oracle.layernorm_quantize_act(x, 1e-5)
    assert np.array_equal(a, a_ref), "a'"
    assert np.array_equal(q, q_ref), f"{int((q != q_ref).sum())} int8 mismatches"


def test_layernorm_equals_quantize_of_oracle_norm():
    """The fused call equals sbn_quantize_act on the oracle's bf16 LayerNorm output."""
    x = _x(5, 64, 2560, "student_t")
    z = oracle.layernorm_bf16(x, 1e-5)
    q, a = _run(x, 1e-5)
    q2, a2 = binding.quantize_act(gu.to_dev_bf16(z))
    assert np.array_equal(q, q2.cpu().numpy()) and np.array_equal(a, a2.cpu().numpy())


def test_layernorm_unaligned_and_eps():
    """Odd leading dimensions (general path), x_q rows wider than K, other eps values."""
    x = _x(7, 9, 1024, "normal")
    for eps in (1e-5, 1e-6, 0.5):
        q, a = _run(x, eps, ld_x=1027, ld_q=1031)
        q_ref, a_ref = oracle.layernorm_quantize_act(x, eps)
        assert np.array_equal(q, q_ref) and np.array_equal(a, a_ref)


def test_layernorm_validation():
    import ctypes
    import torch
    x = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((2, 64), dtype=torch.int8, device="cuda")
    a = torch.zeros((2,), dtype=torch.float32, device="cuda")
    f = binding.lib().sbn_layernorm_quantize_act
    P = binding._ptr
    s = ctypes.c_void_p(0)
    assert f(P(x), 2, 64, 64, 0.0, P(q), 64, P(a), s) == -1        # eps = 0
    assert f(P(x), 2, 64, 64, float("inf"), P(q), 64, P(a), s) == -1
    assert f(P(x), 2, 64, 63, 1e-5, P(q), 64, P(a), s) == -1       # ld_x < K
    assert f(P(x), 2, 64, 64, 1e-5, None, 64, P(a), s) == -1
    assert f(P(x), 0, 64, 64, 1e-5, P(q), 64, P(a), s) == 0        # T == 0


def _fwd_ln(x, w, n, m, eps, ld_x=None, ld_q=None):
    import torch
    T, K = x.shape
    xd = gu.to_dev_bf16(x, ld_x)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
    ldq = K if ld_q is None else ld_q
    out = {}
    for kind in ("f32", "i32"):
        qbuf = torch.full((max(T, 1), ldq), 77, dtype=torch.int8, device="cuda")[:T]
        a = torch.full((T,), -1.0, dtype=torch.float32, device="cuda")
        y, _, _ = binding.bitlinear_bf16(xd, pw, out=kind, x_q=qbuf[:, :K], x_absmax=a,
                                         ln_eps=eps)
        out[kind] = (y.cpu().numpy(), qbuf.cpu().numpy(), a.cpu().numpy())
    q2, a2 = binding.layernorm_quantize_act(xd, eps)
    y2 = binding.bitlinear(q2, a2, pw, out="f32")
    codes, _, gamma = pw.export()
    torch.cuda.synchronize()
    res = dict(y=out["f32"][0], acc=out["i32"][0], q_pad=out["f32"][1], a=out["f32"][2],
               q_i32=out["i32"][1][:, :K], a_i32=out["i32"][2], q2=q2.cpu().numpy(),
               a2=a2.cpu().numpy(), y2=y2.cpu().numpy(), codes=codes.cpu().numpy(),
               gamma=np.float32(gamma.cpu().numpy()[0]))
    pw.free()
    return res


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (3, 8)])
@pytest.mark.parametrize("T", [1, 3, 4, 9])
@pytest.mark.parametrize("K", [2560, 272, 96, 11008])
def test_forward_with_layernorm(n, m, T, K):
    """sbn_bitlinear_fwd_ln_bf16: one kernel for T <= 4 (K = 11008 runs three quads per wave),
    two kernels for T = 9; equal to LayerNorm-quantize + forward and to the oracle."""
    rng = np.random.default_rng(T * 7 + K + n)
    x = inputs.f32_to_bf16_bits(rng.standard_t(4, (T, K)).astype(np.float32) * 2 + 0.5)
    w = (rng.standard_normal((150, K)) * 0.02).astype(np.float32)
    r = _fwd_ln(x, w, n, m, 1e-5)
    q = r["q_pad"][:, :K]
    assert np.array_equal(q, r["q2"]) and np.array_equal(r["a"], r["a2"])
    assert np.array_equal(r["q_i32"], r["q2"]) and np.array_equal(r["a_i32"], r["a2"])
    assert np.array_equal(r["y"], r["y2"])
    q_ref, a_ref = oracle.layernorm_quantize_act(x, 1e-5)
    assert np.array_equal(q, q_ref) and np.array_equal(r["a"], a_ref)
    acc_ref = oracle.int_matmul(q_ref, r["codes"])
    assert np.array_equal(r["acc"], acc_ref)
    gu.assert_y_close(r["y"], oracle.dequantize(acc_ref, r["gamma"], a_ref))


def test_forward_with_layernorm_unaligned_and_fallback():
    """Odd leading dimensions; K > 12288 (two kernels)."""
    rng = np.random.default_rng(99)
    for T, K, ld_x, ld_q in ((3, 520, 523, 531), (2, 12544, None, None), (4, 1040, 1045, None)):
        x = inputs.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
        w = (rng.standard_normal((40, K)) * 0.02).astype(np.float32)
        r = _fwd_ln(x, w, 6, 8, 1e-5, ld_x=ld_x, ld_q=ld_q)
        q_ref, a_ref = oracle.layernorm_quantize_act(x, 1e-5)
        assert np.array_equal(r["q_pad"][:, :K], q_ref) and np.array_equal(r["a"], a_ref)
        if ld_q is not None:
            assert np.all(r["q_pad"][:, K:] == 77)
        assert np.array_equal(r["acc"], oracle.int_matmul(q_ref, r["codes"]))
