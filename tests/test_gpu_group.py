"""GPU parity of the grouped forwards (sbn_bitlinear_fwd_group, sbn_bitlinear_fwd_group_bf16):
several packed weights that read the same activations in one launch.

Every member's output must equal what sbn_bitlinear_fwd (or the bf16 entry) gives for that member
alone, bit for bit, and match the oracle: int32 accumulators exactly (on the GPU's own x_q and
codes), fp32 within 1e-5 relative. The quantized activations must equal sbn_quantize_act's
(sbn_layernorm_quantize_act's with a LayerNorm). Members that cannot share a launch (another
pattern, the compact form, outliers) run one after another with the same results.
"""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _w(seed, N, K):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, K)) * 0.02).astype(np.float32)


def _x(seed, T, K):
    rng = np.random.default_rng(seed)
    return inputs.f32_to_bf16_bits(rng.standard_t(4, (T, K)).astype(np.float32))


def _check_members(pws, ys_group, q, a, kind):
    """Each member: equal to its single forward, and to the oracle on the GPU's own x_q/codes."""
    import torch
    for pw, yg in zip(pws, ys_group):
        ys = binding.bitlinear(q, a, pw, out=kind)
        codes, _, gamma = pw.export()
        torch.cuda.synchronize()
        yg_h, ys_h = yg.cpu().numpy(), ys.cpu().numpy()
        assert np.array_equal(yg_h, ys_h), "grouped output differs from the single forward"
        acc_ref = oracle.int_matmul(q.cpu().numpy(), codes.cpu().numpy())
        if kind == "i32":
            assert np.array_equal(yg_h, acc_ref)
        elif pw.outliers == 0:
            gu.assert_y_close(yg_h, oracle.dequantize(acc_ref, np.float32(gamma.cpu().numpy()[0]),
                                                      a.cpu().numpy()))


@pytest.mark.parametrize("n,m", [(8, 8), (6, 8), (4, 8), (2, 4), (8, 16), (3, 8)])
@pytest.mark.parametrize("T", [1, 3, 4, 9, 16, 40])
@pytest.mark.parametrize("kind", ["f32", "i32"])
def test_group_int8(n, m, T, kind):
    """Three members of different n_out (one not a multiple of 16) on the same int8 input."""
    K = 1024
    shapes = [48, 160, 40]
    ws = [_w(10 * i + n + m, N, K) for i, N in enumerate(shapes)]
    pws = [binding.PackedWeight(gu.to_dev_f32(w), n, m) for w in ws]
    xd = gu.to_dev_bf16(_x(T + n, T, K))
    q, a = binding.quantize_act(xd)
    ys = binding.bitlinear_group(q, a, pws, out=kind)
    _check_members(pws, ys, q, a, kind)
    for p in pws:
        p.free()


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 16), (8, 8), (3, 8)])
@pytest.mark.parametrize("T", [1, 2, 4, 9])
@pytest.mark.parametrize("ln", [0.0, 1e-5])
def test_group_bf16(n, m, T, ln):
    """The grouped quantize-and-multiply: one kernel for T <= 4 (every workgroup quantizes), the
    quantizer and the grouped GEMV for T = 9; x_q and a' equal the quantizer's."""
    import torch
    K = 2560
    shapes = [64, 96, 32]
    ws = [_w(7 * i + n, N, K) for i, N in enumerate(shapes)]
    pws = [binding.PackedWeight(gu.to_dev_f32(w), n, m) for w in ws]
    xb = _x(11 * T + m, T, K)
    xd = gu.to_dev_bf16(xb)
    for kind in ("f32", "i32"):
        ys, q, a = binding.bitlinear_group_bf16(xd, pws, out=kind, ln_eps=ln)
        if ln > 0:
            q2, a2 = binding.layernorm_quantize_act(xd, ln)
        else:
            q2, a2 = binding.quantize_act(xd)
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), q2.cpu().numpy())
        assert np.array_equal(a.cpu().numpy(), a2.cpu().numpy())
        _check_members(pws, ys, q2, a2, kind)
    if ln == 0.0:
        q_ref, a_ref = oracle.quantize_act(xb)
        assert np.array_equal(a.cpu().numpy(), a_ref)
        gu.assert_int_exact_except_boundary(q.cpu().numpy(), q_ref,
                                            oracle.boundary_elements_act(xb, a_ref), "x_q")
    for p in pws:
        p.free()


def test_group_mixed_members_run_in_turn():
    """Members that cannot share a launch (other patterns, a compact pack, outliers) give the
    same results as single calls, through both entries."""
    import torch
    K = 1024
    ws = [_w(100 + i, 64, K) for i in range(4)]
    pws = [binding.PackedWeight(gu.to_dev_f32(ws[0]), 6, 8),
           binding.PackedWeight(gu.to_dev_f32(ws[1]), 2, 4),
           binding.PackedWeight(gu.to_dev_f32(ws[2]), 6, 8, compact=True),
           binding.PackedWeight(gu.to_dev_f32(ws[3]), 6, 8, outliers=8)]
    for T in (1, 5):
        xd = gu.to_dev_bf16(_x(200 + T, T, K))
        q, a = binding.quantize_act(xd)
        ys = binding.bitlinear_group(q, a, pws, out="f32")
        _check_members(pws, ys, q, a, "f32")
        yb, qb, ab = binding.bitlinear_group_bf16(xd, pws, out="f32")
        torch.cuda.synchronize()
        assert np.array_equal(qb.cpu().numpy(), q.cpu().numpy())
        for y1, y2 in zip(yb, ys):
            assert np.array_equal(y1.cpu().numpy(), y2.cpu().numpy())
    for p in pws:
        p.free()


def test_group_validation():
    import torch
    K = 256
    a = binding.PackedWeight(gu.to_dev_f32(_w(1, 32, K)), 2, 4)
    b = binding.PackedWeight(gu.to_dev_f32(_w(2, 32, 2 * K)), 2, 4)
    q = torch.zeros((1, 2 * K), dtype=torch.int8, device="cuda")
    am = torch.ones((1,), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.SbnError) as e:
        binding.bitlinear_group(q[:, :K], am, [a, b])
    assert e.value.status == -3  # members with another K
    with pytest.raises(binding.SbnError) as e:
        binding.bitlinear_group(q[:, :K], am, [a] * 9)
    assert e.value.status == -1  # more than SBN_MAX_GROUP
    ys = binding.bitlinear_group(q[:, :K], am, [a] * 8)  # a handle may repeat
    torch.cuda.synchronize()
    assert len(ys) == 8
    a.free()
    b.free()


@pytest.mark.parametrize("n,m", [(8, 8), (6, 8), (4, 8), (2, 4), (8, 16)])
@pytest.mark.parametrize("T", [1, 16])
def test_group_block_shapes(n, m, T):
    """The 2B-style block's grouped launches at full size: Q, K and V (3 x 2560 -> 2560) on one
    input, gate and up (2 x 2560 -> 6912) on another, every member against the oracle on sampled
    rows; at T = 1 the one-kernel quantize-and-multiply step, at T = 16 the grouped int8 GEMV."""
    import torch
    wl = inputs.W_BLOCK
    for members in ((0, 1, 2), (4, 5)):
        act = wl.layers[members[0]].act_input
        K = wl.layers[members[0]].k
        xb = inputs.activations(wl, act, T, K)
        xd = gu.to_dev_bf16(xb)
        wts = [inputs.latent_weights(wl, li) for li in members]
        pws = [binding.PackedWeight(gu.to_dev_f32(w), n, m) for w in wts]
        print(f"[group] layers={members} T={T} {n}:{m}", flush=True)
        ys, q, a = binding.bitlinear_group_bf16(xd, pws, out="f32")
        acc = binding.bitlinear_group(q, a, pws, out="i32")
        torch.cuda.synchronize()
        qh, ah = q.cpu().numpy(), a.cpu().numpy()
        q_ref, a_ref = oracle.quantize_act(xb)
        assert np.array_equal(ah, a_ref)
        gu.assert_int_exact_except_boundary(qh, q_ref, oracle.boundary_elements_act(xb, a_ref),
                                            "x_q")
        rng = np.random.default_rng(T + n + m)
        for pw, w, y, ac in zip(pws, wts, ys, acc):
            p = oracle.pack_nm_ternary(w, n, m)
            codes, keep, gamma = pw.export()
            torch.cuda.synchronize()
            g = np.float32(gamma.cpu().numpy()[0])
            assert gu.gamma_matches(g, w)
            assert np.array_equal(keep.cpu().numpy().astype(bool), p["keep"])
            ch = codes.cpu().numpy()
            gu.assert_int_exact_except_boundary(ch, p["codes"],
                                                oracle.boundary_elements_weight(w, p["gamma"]),
                                                "codes")
            rows = np.sort(rng.choice(w.shape[0], 64, replace=False))
            acc_ref = oracle.int_matmul(qh, ch[rows])
            assert np.array_equal(ac.cpu().numpy()[:, rows], acc_ref)
            gu.assert_y_close(y.cpu().numpy()[:, rows], oracle.dequantize(acc_ref, g, ah))
        for p_ in pws:
            p_.free()


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 16)])
@pytest.mark.parametrize("T", [5, 16])
@pytest.mark.parametrize("shapes", [[2560, 2570, 1000], [5000, 4000, 1336]])
def test_group_int8_shared_activation_pieces(n, m, T, shapes):
    """Five to sixteen tokens with 320 or more row blocks in all: each workgroup takes two (from
    640 on, three) row blocks of one member and shares its activation pieces among them. Ragged
    members (their last workgroup reaches past the stored plane), outputs equal to the single
    forwards and to the oracle."""
    K = 1024
    ws = [_w(31 * i + n + m + T, N, K) for i, N in enumerate(shapes)]
    pws = [binding.PackedWeight(gu.to_dev_f32(w), n, m) for w in ws]
    xd = gu.to_dev_bf16(_x(5 * T + m, T, K))
    q, a = binding.quantize_act(xd)
    for kind in ("f32", "i32"):
        ys = binding.bitlinear_group(q, a, pws, out=kind)
        _check_members(pws, ys, q, a, kind)
    for p in pws:
        p.free()


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4), (8, 16)])
@pytest.mark.parametrize("T", [5, 16])
@pytest.mark.parametrize("shapes", [[2560, 2570, 1000], [5000, 4000, 1336]])
def test_group_bf16_wide_5_to_16_tokens(n, m, T, shapes):
    """The grouped bf16 entry for five to sixteen tokens on wide members: the quantize kernel,
    then the row-block-sharing grouped GEMV. x_q and a' equal sbn_quantize_act's, every member
    equals its single forward and the oracle."""
    import torch
    K = 1024
    ws = [_w(17 * i + n + m + T, N, K) for i, N in enumerate(shapes)]
    pws = [binding.PackedWeight(gu.to_dev_f32(w), n, m) for w in ws]
    xd = gu.to_dev_bf16(_x(3 * T + n, T, K))
    q2, a2 = binding.quantize_act(xd)
    for kind in ("f32", "i32"):
        ys, q, a = binding.bitlinear_group_bf16(xd, pws, out=kind)
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), q2.cpu().numpy())
        assert np.array_equal(a.cpu().numpy(), a2.cpu().numpy())
        _check_members(pws, ys, q2, a2, kind)
    for p in pws:
        p.free()
