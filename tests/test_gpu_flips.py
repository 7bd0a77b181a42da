"""GPU parity of the keep-mask flip count (sbn_packed_mask_flips; Sparse-BitNet, Figure 3 (b),
mask flip rate r_t). A pack counts the keep bits it changes while it overwrites the mask; the
count must equal the oracle's Hamming distance between the two oracle masks exactly."""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _flips(pw):
    import torch
    f = pw.mask_flips()
    torch.cuda.synchronize()
    return int(f.cpu().numpy()[0])


def _keep(pw):
    return pw.export()[1].cpu().numpy().astype(bool)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 16), (3, 8), (1, 4), (12, 16), (8, 8)])
@pytest.mark.parametrize("N,K", [(70, 1040), (16, 256), (300, 2560)])
def test_flips_repack_sequence(n, m, N, K):
    """First pack (against an empty mask), a perturbed re-pack, an identical re-pack and a large
    perturbation; ragged n_out, K ending inside a quad, several row blocks."""
    K += (-K) % m
    rng = np.random.default_rng(17 * N + K + 3 * n + m)
    w1 = rng.standard_normal((N, K)).astype(np.float32)
    seq = [w1,
           (w1 + 0.05 * rng.standard_normal((N, K))).astype(np.float32),
           None,  # the same weights again
           rng.standard_normal((N, K)).astype(np.float32)]
    pw = binding.PackedWeight(gu.to_dev_f32(w1), n, m)
    prev_ref = None
    cur = w1
    for i, w in enumerate(seq):
        if i > 0:
            cur = cur if w is None else w
            pw.pack(gu.to_dev_f32(cur))
        keep_ref = oracle.nm_keep_mask(cur, n, m)
        assert np.array_equal(_keep(pw), keep_ref), f"step {i}: keep mask"
        expect = 0 if n == m else oracle.mask_flips(prev_ref, keep_ref)
        assert _flips(pw) == expect, f"step {i}"
        prev_ref = keep_ref
    # reading the count does not change it; a forward does not either
    x = inputs.f32_to_bf16_bits(rng.standard_normal((3, K)).astype(np.float32))
    binding.bitlinear_bf16(gu.to_dev_bf16(x), pw)
    assert _flips(pw) == expect
    pw.free()


def test_flips_training_drift_ffn_up():
    """A small latent update on the 6912 x 2560 up projection at 6:8 and 2:4: the count equals
    the oracle's, and r_t = flips / (n_out * K) is small but non-zero."""
    wl = inputs.W_DECODE
    w = inputs.latent_weights(wl, 0)
    rng = np.random.default_rng(3)
    w2 = (w + 1e-3 * rng.standard_normal(w.shape)).astype(np.float32)
    for n, m in ((6, 8), (2, 4)):
        pw = binding.PackedWeight(gu.to_dev_f32(w), n, m)
        k1 = oracle.nm_keep_mask(w, n, m)
        assert _flips(pw) == int(k1.sum())
        pw.pack(gu.to_dev_f32(w2))
        k2 = oracle.nm_keep_mask(w2, n, m)
        f = _flips(pw)
        assert f == oracle.mask_flips(k1, k2)
        assert 0 < f / w.size < 0.5
        pw.free()


def test_flips_validation():
    import ctypes
    import torch
    pw = binding.PackedWeight(torch.ones((16, 64), dtype=torch.float32, device="cuda"), 2, 4)
    out = torch.zeros((1,), dtype=torch.int64, device="cuda")
    f = binding.lib().sbn_packed_mask_flips
    assert f(None, binding._ptr(out), ctypes.c_void_p(0)) == -1
    assert f(pw.handle, None, ctypes.c_void_p(0)) == -1
    # all-equal magnitudes: ties go to the lower positions, so the first pack keeps 2 of 4
    assert _flips(pw) == 16 * 64 // 2
    pw.free()
