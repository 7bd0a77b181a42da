"""GPU parity of the GEMV on large K (T <= 16): past 48 quads (K > 12288) each wave loads the bricks
of all its quads at once (up to 128 quads, K <= 32768; positional, 2:4 and compact codes, aligned
int8 rows; for one to four tokens the activation rows are first staged in LDS), otherwise the waves
take batches of 48 quads in turn, so decode on e.g. 13B- and 70B-style down projections stays a
GEMV. Integer accumulators are exact; fp32 outputs follow the oracle within the forward's
tolerance."""

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
@pytest.mark.parametrize("K", [12544, 13824, 28672, 32768, 33024])
def test_large_k_gemv(n, m, T, K):
    """49 to 128 quads: the kernel that loads all of a wave's quads at once (four to eight per wave;
    positional and 2:4 codes) and, for the kept form (3:8), batches of 48 quads in turn; 129 quads:
    batches for every form (three, the last ragged)."""
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


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 16)])
@pytest.mark.parametrize("T", [5, 9, 16])
@pytest.mark.parametrize("N,K,ld_q", [(5200, 1040, None), (5104, 4096, 4112), (6912, 2560, None)])
def test_two_row_blocks_per_workgroup(n, m, T, N, K, ld_q):
    """More than four tokens, at most 16 quads and at least 320 row blocks: one workgroup takes two
    row blocks (5200 rows: 325 blocks, the last workgroup's second block is padding; K = 1040: a
    K tail inside the last quad; a padded x_q row pitch). All outputs against the oracle."""
    x, w = _case(N + K + T + n, T, N, K)
    r = _run(x, w, n, m, ld_q=ld_q)
    q_ref, a_ref = oracle.quantize_act(x)
    assert np.array_equal(r["q"], q_ref) and np.array_equal(r["a"], a_ref)
    acc_ref = oracle.int_matmul(q_ref, r["codes"])
    assert np.array_equal(r["acc"], acc_ref)
    gu.assert_y_close(r["y"], oracle.dequantize(acc_ref, r["gamma"], a_ref))


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 16), (4, 8)])
@pytest.mark.parametrize("T", [1, 3, 16])
@pytest.mark.parametrize("K", [12544, 28672, 32768])
def test_large_k_compact_plane(n, m, T, K):
    """The compact plane past one batch (49 to 128 quads) in the kernel that loads all of a wave's
    quads at once: masks and sign slots per lane, the nibble table in LDS; every output equals the
    oracle and the positional plane's."""
    x, w = _case(K + 5 * T + m, T, 72, K)
    r = _run(x, w, n, m, compact=True)
    q_ref, a_ref = oracle.quantize_act(x)
    acc_ref = oracle.int_matmul(q_ref, oracle.pack_nm_ternary(w, n, m)["codes"])
    assert np.array_equal(r["acc"], acc_ref)
    gu.assert_y_close(r["y"], oracle.dequantize(acc_ref, r["gamma"], a_ref))
    assert np.array_equal(r["yb"], r["y"])
    rp = _run(x, w, n, m)
    assert np.array_equal(rp["y"].view(np.uint32), r["y"].view(np.uint32))


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 16)])
@pytest.mark.parametrize("T", [5, 9, 12])
@pytest.mark.parametrize("K,N", [(12544, 72), (28672, 520), (32768, 264)])
def test_large_k_split_over_k(n, m, T, K, N):
    """Five to sixteen tokens past one batch: workgroups of 16 row blocks and one 8-quad K chunk,
    the chunk's activations shared through LDS, the chunks' int32 partial sums met by the row
    group's last arrival (which resets the group's counter). Three calls in a row on one handle
    give the oracle's integers each time (a counter left over would merge the wrong chunks);
    ragged row groups (72, 520 and 264 rows) and a ragged last K chunk (K = 12544: 49 quads)."""
    import torch
    x, w = _case(K + 11 * T + n, T, N, K)
    xd = gu.to_dev_bf16(x)
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
    q, a = binding.quantize_act(xd)
    q_ref, a_ref = oracle.quantize_act(x)
    acc_ref = oracle.int_matmul(q_ref, oracle.pack_nm_ternary(w, n, m)["codes"])
    g = np.float32(pw.export()[2].cpu().numpy()[0])
    for _ in range(3):
        acc = binding.bitlinear(q, a, pw, out="i32")
        y = binding.bitlinear(q, a, pw, out="f32")
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), acc_ref)
        gu.assert_y_close(y.cpu().numpy(), oracle.dequantize(acc_ref, g, a_ref))
    pw.free()


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 16)])
@pytest.mark.parametrize("T", [5, 16])
@pytest.mark.parametrize("N,K", [(10480, 1024), (10256, 2560)])
def test_many_row_blocks_three_per_workgroup(n, m, T, N, K):
    """Five to sixteen tokens, at most 16 quads and 640 or more row blocks: three row blocks per
    workgroup. 10480 rows are 655 row blocks (656 stored), so the last workgroup's third row block
    lies past the plane and must read zero; 10256 rows end inside a row block."""
    x, w = _case(N + K + 3 * T + n, T, N, K)
    r = _run(x, w, n, m)
    q_ref, a_ref = oracle.quantize_act(x)
    assert np.array_equal(r["q"], q_ref) and np.array_equal(r["a"], a_ref)
    ref = oracle.pack_nm_ternary(w, n, m)
    assert np.array_equal(r["codes"], ref["codes"])
    acc_ref = oracle.int_matmul(q_ref, ref["codes"])
    assert np.array_equal(r["acc"], acc_ref)
    gu.assert_y_close(r["y"], oracle.dequantize(acc_ref, r["gamma"], a_ref))
