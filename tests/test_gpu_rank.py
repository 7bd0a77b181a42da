"""GPU parity of the rank export (sbn_packed_export_rank): each group's n-of-m keep mask as its rank
in the combinatorial number system (colex order), then its kept codes, the metadata width the
pages print for 2:4 and 8:16 ("From 2:4 to 8:16 sparsity patterns in LLMs for Outliers and
Weights with Variance Correction", abstract). Integer work: the exported bytes equal
oracle.rank_pack of the oracle's codes and keep mask exactly, for every code form of the pack."""

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import binding
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

PATTERNS = [(2, 4), (1, 4), (3, 4), (4, 4), (6, 8), (3, 8), (4, 8), (8, 8), (8, 16), (5, 16),
            (12, 16), (16, 16)]


def _export(w, n, m, **kw):
    import torch
    pw = binding.PackedWeight(gu.to_dev_f32(w), n, m, **kw)
    data = pw.export_rank()
    codes, keep, _ = pw.export()
    d = pw.query()
    torch.cuda.synchronize()
    out = data.cpu().numpy(), codes.cpu().numpy(), keep.cpu().numpy().astype(bool), d
    pw.free()
    return out


@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("N,K", [(37, 1040), (16, 128), (5, 4096), (300, 2560), (3, 48)])
def test_rank_export(n, m, N, K):
    """Rows of one to many chunks of 128 positions, K ending inside a chunk and inside a brick,
    every code form (positional, kept, structured 2:4, dense)."""
    K -= K % m
    rng = np.random.default_rng(N * 31 + K + 7 * n + m)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    data, codes, keep, d = _export(w, n, m)
    ref = oracle.pack_nm_ternary(w, n, m)
    assert np.array_equal(codes, ref["codes"]) and np.array_equal(keep, ref["keep"])
    assert d.rank_row_bytes == oracle.rank_row_bytes(n, m, K)
    assert np.array_equal(data, oracle.rank_pack(ref["codes"], ref["keep"], n, m))
    c2, k2 = oracle.rank_unpack(data, n, m, K)
    assert np.array_equal(c2, ref["codes"]) and np.array_equal(k2, ref["keep"])


def test_rank_export_with_outliers_and_compact():
    """The export follows the ternary part of a pack with k:256 outliers (outlier positions read
    as 0) and is independent of the compact option."""
    n, m, N, K = 8, 16, 40, 1024
    w = (np.random.default_rng(3).standard_normal((N, K)) * 0.02).astype(np.float32)
    data, codes, keep, _ = _export(w, n, m, outliers=8, compact=True)
    ref = oracle.pack_with_outliers(w, n, m, 8)
    assert np.array_equal(codes, ref["codes"])
    assert np.array_equal(data, oracle.rank_pack(ref["codes"], ref["keep"], n, m))


def test_rank_export_edge_cases():
    """All-zero weights (ranks of the lowest positions, zero codes) and n_out == 0."""
    import torch
    w = np.zeros((5, 64), np.float32)
    data, codes, keep, _ = _export(w, 2, 4)
    assert np.array_equal(data, oracle.rank_pack(codes, keep, 2, 4))
    pw = binding.PackedWeight(torch.zeros((0, 256), dtype=torch.float32, device="cuda"), 2, 4)
    assert pw.export_rank().shape == (0, oracle.rank_row_bytes(2, 4, 256))
    pw.free()
