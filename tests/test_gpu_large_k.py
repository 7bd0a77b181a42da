"""GPU parity of the GEMV on large K (T <= 16): past 48 quads (K > 12288) the waves take batches
of 48 quads in turn, so decode on e.g. 13B- and 70B-style down projections stays a GEMV. Integer
accumulators are exact; fp32 outputs follow the oracle within the forward's tolerance."""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case(seed, T, N, K):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = inputs.f32_to_bf16_bits(rng.standard_t(4, (T, K)).astype(np.float32))
    return x, w


def _run(x, w, n, m, ld_q=None, **pack_kw):
    import torch
    T, K = x.shape
    xd = gu.to_dev_bf16(x)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, **pack_kw)
    ldq = K if ld_q is None else ld_q
    qbuf = torch.zeros((T, ldq), dtype=torch.int8, device="cuda")
    q, a = binding.quantize_act(xd, out_q=qbuf[:, :K])
    acc = binding.bitlinear(q, a, pw, out="i32")
    y = binding.bitlinear(q, a, pw, out="f32")
    yb = binding.bitlinear_bf16(xd, pw)[0]  # T <= 4: quantize kernel + this GEMV (K > 12288)
    codes, _, g = pw.export()
    torch.cuda.synchronize()
    r = dict(q=q.cpu().numpy(), a=a.cpu().numpy(), acc=acc.cpu().numpy(), y=y.cpu().numpy(),
             yb=yb.cpu().numpy(), codes=codes.cpu().numpy(), gamma=np.float32(g.cpu().numpy()[0]))
    pw.free()
    return r


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 16), (3, 8)])
@pytest.mark.parametrize("T", [1, 3, 16])
@pytest.mark.parametrize("K", [12544, 13824, 28672])
def test_large_k_gemv(n, m, T, K):
    """49, 54 and 112 quads: two and three batches, a ragged last batch; every code form."""
    x, w = _case(K + 7 * T + n, T, 72, K)
    r = _run(x, w, n, m)
    q_ref, a_ref = oracle.quantize_act(x)
    assert np.array_equal(r["q"], q_ref) and np.array_equal(r["a"], a_ref)
    ref = oracle.pack_nm_ternary(w, n, m)
    assert np.array_equal(r["codes"], ref["codes"])
    acc_ref = oracle.int_matmul(q_ref, ref["codes"])
    assert np.array_equal(r["acc"], acc_ref)
    gu.assert_y_close(r["y"], oracle.dequantize(acc_ref, r["gamma"], a_ref))
    assert np.array_equal(r["yb"], r["y"])


def test_large_k_ragged_and_compact():
    """K = 13832 (a K tail inside the last brick, non-vector activation loads), unaligned x_q rows,
    and the compact plane over three batches."""
    for K, n, m, ld_q, kw in ((13832, 6, 8, 13841, {}), (28672, 8, 16, None, {"compact": True}),
                              (20480, 2, 4, None, {"compact": True})):
        x, w = _case(K, 5, 40, K)
        r = _run(x, w, n, m, ld_q=ld_q, **kw)
        q_ref, _ = oracle.quantize_act(x)
        assert np.array_equal(r["acc"], oracle.int_matmul(q_ref, oracle.pack_nm_ternary(w, n, m)["codes"]))


def test_large_k_70b_shape():
    """The 8192 x 28672 down projection of a 70B-style FFN at 8:16, T = 16: all outputs."""
    x, w = _case(70, 16, 8192, 28672)
    r = _run(x, w, 8, 16)
    q_ref, a_ref = oracle.quantize_act(x)
    acc_ref = oracle.int_matmul(q_ref, r["codes"])
    assert np.array_equal(r["acc"], acc_ref)
    gu.assert_y_close(r["y"], oracle.dequantize(acc_ref, r["gamma"], a_ref))
