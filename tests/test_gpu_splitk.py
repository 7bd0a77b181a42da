"""GPU parity of the split-K GEMM (launches with at most 256 tiles of 256 rows x 64 tokens and
at least 8 K steps run two workgroups per tile, one per half of K, combined through a handshake
in y). Results must equal the oracle exactly (int32) and to 1e-5 (fp32), every call in a row."""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case(seed, T, K, N):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, K)).astype(np.float32) * 2
    w = (rng.laplace(0.0, 0.015, (N, K))).astype(np.float32)
    return inputs.f32_to_bf16_bits(x), w


@pytest.mark.parametrize("n,m", [(8, 16), (6, 8), (2, 4), (3, 8)])
@pytest.mark.parametrize("T,K,N", [(150, 2048, 300), (17, 2304, 250), (300, 2560, 64),
                                   (129, 4096, 16)])
def test_split_k(n, m, T, K, N):
    """Even (8, 10, 16) and odd (9) step counts, ragged T and n_out, one to six tiles."""
    x, w = _case(7 * T + K + N + n, T, K, N)
    g = gu.gpu_forward(x, w, n, m)
    gu.check_stages(g, x, w, n, m)


def test_split_k_unaligned():
    """Leading dimensions that force the element-wise activation loads and output stores."""
    x, w = _case(3, 40, 2048, 70)
    g = gu.gpu_forward(x, w, 8, 16, ld_x=2048 + 3, ld_w=2048 + 1, ld_q=2048 + 5)
    gu.check_stages(g, x, w, 8, 16)


def test_split_k_repeated_calls_and_prefill_down():
    """The handshake words carry over from call to call: twenty calls in a row on the 6912 -> 2560
    prefill shape give identical outputs, equal to the oracle on sampled tokens and rows."""
    import torch
    wl = inputs.W_PREFILL
    w = inputs.latent_weights(wl, 1)
    T = 256
    x = inputs.activations(wl, 1, T, w.shape[1])
    xd = gu.to_dev_bf16(x)
    q, a = binding.quantize_act(xd)
    pw = binding.PackedWeight(gu.to_dev_f32(w), 8, 16)
    ys = [binding.bitlinear(q, a, pw, out="i32").cpu().numpy() for _ in range(20)]
    for yy in ys[1:]:
        assert np.array_equal(yy, ys[0])
    codes = pw.export()[0].cpu().numpy()
    rows = np.random.default_rng(0).choice(w.shape[0], 64, replace=False)
    acc_ref = oracle.int_matmul(q.cpu().numpy(), codes[rows])
    assert np.array_equal(ys[0][:, rows], acc_ref)
    pw.free()
    torch.cuda.synchronize()


def test_split_k_giveup_is_counted_and_does_not_leak(monkeypatch):
    """A waiting half that never sees its partner's partial sums (the first halves withhold them
    in a test mode set at pack time) gives up after a bounded spin, counts it in the handle and
    exits normally. A re-pack of the same handle in the normal mode then gives correct results:
    the words left by the launch that gave up never match a later launch. A handle packed
    normally counts no give-ups."""
    import torch
    x, w = _case(11, 150, 2048, 300)  # 2 x 3 tiles of 256 rows x 64 tokens, 8 K steps: split
    xd = gu.to_dev_bf16(x)
    q, a = binding.quantize_act(xd)
    monkeypatch.setenv("SBN_SPLITK_SPIN_LIMIT", "64")
    monkeypatch.setenv("SBN_SPLITK_WITHHOLD", "1")
    pw = binding.PackedWeight(gu.to_dev_f32(w), 8, 16)
    binding.bitlinear(q, a, pw, out="i32")
    torch.cuda.synchronize()
    assert pw.query().splitk_giveups == 6 * 4  # every (tile, wave) pair
    monkeypatch.delenv("SBN_SPLITK_WITHHOLD")
    monkeypatch.delenv("SBN_SPLITK_SPIN_LIMIT")
    pw.pack(gu.to_dev_f32(w))
    codes = pw.export()[0].cpu().numpy()
    acc_ref = oracle.int_matmul(q.cpu().numpy(), codes)
    for _ in range(3):
        acc = binding.bitlinear(q, a, pw, out="i32")
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert pw.query().splitk_giveups == 6 * 4
    pw.free()
    pw2 = binding.PackedWeight(gu.to_dev_f32(w), 8, 16)
    acc = binding.bitlinear(q, a, pw2, out="i32")
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert pw2.query().splitk_giveups == 0
    pw2.free()


def test_split_k_graph_replays():
    """The handshake keeps no host-side state: a captured split-K forward replayed several times,
    with eager work and synchronizations between the replays, gives the eager result every time."""
    import torch
    x, w = _case(12, 150, 2048, 300)
    xd = gu.to_dev_bf16(x)
    q, a = binding.quantize_act(xd)
    pw = binding.PackedWeight(gu.to_dev_f32(w), 6, 8)
    y = torch.empty((150, 300), dtype=torch.int32, device="cuda")
    binding.bitlinear(q, a, pw, out="i32", y=y)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.bitlinear(q, a, pw, out="i32", y=y)
    for _ in range(4):
        y.zero_()
        binding.bitlinear(q, a, pw, out="i32")  # eager work on the same handle between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
    assert pw.query().splitk_giveups == 0
    pw.free()


@pytest.mark.parametrize("T", [1, 3, 16, 150, 300])
def test_sparse_mfma_2of4_matches_dense_path(T, monkeypatch):
    """2:4 handles use the structured-sparse MFMA (kept weights + position indices); with
    SBN_NO_SMFMAC=1 they use positional codes and the dense MFMA. Both must give the same int32
    accumulators, fp32 outputs and exports, equal to the oracle."""
    import torch
    x, w = _case(100 + T, T, 2560, 300)
    res = {}
    for flag in ("0", "1"):
        monkeypatch.setenv("SBN_NO_SMFMAC", flag)
        g = gu.gpu_forward(x, w, 2, 4)
        gu.check_stages(g, x, w, 2, 4)
        res[flag] = g
        xd = gu.to_dev_bf16(x)
        pw = binding.PackedWeight(gu.to_dev_f32(w), 2, 4)
        y, _, _ = binding.bitlinear_bf16(xd, pw)
        res[flag + "_bf16"] = y.cpu().numpy()
        pw.free()
    for key in ("acc", "y", "codes", "keep", "code_bytes", "mask_bytes"):
        assert np.array_equal(res["0"][key], res["1"][key]), key
    assert np.array_equal(res["0_bf16"], res["1_bf16"])
    torch.cuda.synchronize()
