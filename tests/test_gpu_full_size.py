"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Quantization, keep masks, codes and packed bytes are compared in full; int32 accumulators and fp32
outputs on sampled tokens (all rows) and sampled rows (all tokens), which the oracle computes in
seconds. Every (layer shape, pattern, token count) that the benchmark times is covered:

- the decode layer 2560 -> 6912 at 6:8, T = 1 and 16;
- both prefill layers at 8:16, T = 2048;
- the three distinct shapes of the 2B-style block (Q/K/V/O 2560 -> 2560, gate/up 2560 -> 6912,
  down 6912 -> 2560) at all five patterns, T = 1, 16 and 4096;
- both 7B FFN layers at 2:4 and 8:16, T = 8192.

At T <= 4 the quantize-and-multiply entry (one kernel, the decode step the benchmark times) runs on
the same packed weights as the two-call path and must equal it bit for bit.
"""

import functools

import numpy as np
import pytest

import oracle
from sparsity_sbn_quantize_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

BLOCK_PATTERNS = [(8, 8), (6, 8), (4, 8), (2, 4), (8, 16)]
BLOCK_SHAPES = [0, 4, 6]  # Q (2560 -> 2560), gate (2560 -> 6912), down (6912 -> 2560)


def _samples(count, size, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(size, size=min(count, size), replace=False))


@functools.lru_cache(maxsize=16)
def _weights_and_pack(wl_index, layer_index, n, m):
    wl = inputs.WORKLOADS[wl_index]
    w = inputs.latent_weights(wl, layer_index)
    return w, oracle.pack_nm_ternary(w, n, m)


def _run(wl, layer_index, T, n, m, seed):
    layer = wl.layers[layer_index]
    x = inputs.activations(wl, layer.act_input, T, layer.k)
    w, p = _weights_and_pack(wl.index, layer_index, n, m)
    print(f"[full-size] {wl.name} layer={layer.name} T={T} {n}:{m}", flush=True)
    g = gu.gpu_forward(x, w, n, m, bf16_step=T <= 4)
    toks = _samples(24, T, seed)
    rows = _samples(48, layer.n_out, seed + 1)
    gu.check_stages(g, x, w, n, m, acc_tokens=toks, acc_rows=rows, p=p)


@pytest.mark.parametrize("T", [1, 16])
def test_decode_6of8(T):
    _run(inputs.W_DECODE, 0, T, 6, 8, 100 + T)


@pytest.mark.parametrize("layer", [0, 1])
def test_prefill_8of16(layer):
    _run(inputs.W_PREFILL, layer, 2048, 8, 16, 200 + layer)


@pytest.mark.parametrize("n,m", BLOCK_PATTERNS)
@pytest.mark.parametrize("li", BLOCK_SHAPES)
@pytest.mark.parametrize("T", [1, 16, 4096])
def test_block(T, li, n, m):
    _run(inputs.W_BLOCK, li, T, n, m, 300 + 10 * li + T % 97)


@pytest.mark.parametrize("layer,n,m", [(0, 2, 4), (0, 8, 16), (1, 2, 4), (1, 8, 16)])
def test_train_step_T8192(layer, n, m):
    _run(inputs.W_TRAIN, layer, 8192, n, m, 500 + layer)
