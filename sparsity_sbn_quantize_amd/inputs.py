"""Seeded synthetic inputs for the Sparse-BitNet BitLinear forward.

This module holds random-number generation and storage-format conversion only (fp32 values to
bf16 bit patterns by round-to-nearest-even); none of the method's arithmetic lives here. The CPU
oracle's tests and the HIP path's tests and benchmark both draw their inputs from it, so that the
two sides see identical bytes.

Every tensor comes from NumPy's PCG64 generator seeded with
``SeedSequence(entropy=0, spawn_key=(workload index, tensor kind, tensor index, extra))``.

The workloads are synthetic stand-ins with the layer shapes of a 2B-parameter BitNet-style block
(2560 hidden, 6912 FFN) and of a 7B-style FFN (4096 hidden, 11008 FFN); the pages give no layer
shapes of their own and no trained weights are available.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# Tensor-kind tags in the spawn key.
_ACT = 0
_WEIGHT = 1
_GRAD = 2


@dataclass(frozen=True)
class Layer:
    """One BitLinear: ``K`` input features -> ``n_out`` output features."""

    name: str
    n_out: int
    k: int
    act_input: int  # index of the activation tensor this layer consumes


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    layers: tuple
    patterns: tuple  # ((n, m), ...)
    tokens: tuple  # token counts T
    weight_dist: str  # "normal" | "normal_rowscaled" | "laplace"
    weight_scale: float
    act_dist: str  # "normal" | "student_t4" | "normal_outliers"
    repack_every_step: bool = False


# Small single layer, 2:4 along K, seed 0.
W_SMALL = Workload(
    0, "bitlinear_2of4_T8_K256_N256",
    (Layer("proj", 256, 256, 0),),
    ((2, 4),), (8,), "normal", 0.02, "normal")

# Decode GEMV: 2560 -> 6912 (FFN up of a 2B-style block), 6:8, packed once.
W_DECODE = Workload(
    1, "decode_gemv_6of8_K2560_N6912",
    (Layer("ffn_up", 6912, 2560, 0),),
    ((6, 8),), (1, 16), "normal_rowscaled", 0.02, "student_t4")

# Prefill GEMM: 2048 tokens, 8:16, both FFN directions.
W_PREFILL = Workload(
    2, "prefill_gemm_8of16_T2048",
    (Layer("ffn_up", 6912, 2560, 0), Layer("ffn_down", 2560, 6912, 1)),
    ((8, 16),), (2048,), "laplace", 0.015, "normal_outliers")

# Whole 2B-style block: Q/K/V/O 2560x2560, gate/up 2560->6912, down 6912->2560.
W_BLOCK = Workload(
    3, "block_2b_sweep",
    (Layer("q", 2560, 2560, 0), Layer("k", 2560, 2560, 0), Layer("v", 2560, 2560, 0),
     Layer("o", 2560, 2560, 1), Layer("gate", 6912, 2560, 2), Layer("up", 6912, 2560, 2),
     Layer("down", 2560, 6912, 3)),
    ((8, 8), (6, 8), (4, 8), (2, 4), (8, 16)), (1, 16, 4096), "normal", 0.02, "normal")

# 7B-style dynamic sparse training step: re-pack every step, then the forward GEMM.
W_TRAIN = Workload(
    4, "train_step_7b_ffn_T8192",
    (Layer("ffn_up", 11008, 4096, 0), Layer("ffn_down", 4096, 11008, 1)),
    ((2, 4), (8, 16)), (8192,), "normal", 0.02, "normal", repack_every_step=True)

WORKLOADS = (W_SMALL, W_DECODE, W_PREFILL, W_BLOCK, W_TRAIN)


def _rng(*spawn_key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(0, spawn_key=spawn_key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    Finite inputs only (the generators never produce NaN or Inf).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + rounding) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values (storage conversion only)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_channels(k: int, workload_index: int, act_index: int) -> np.ndarray:
    """Input channels scaled x20 for the outlier activation recipe: round(0.001*K) of them,
    drawn without replacement."""
    count = int(round(0.001 * k))
    rng = _rng(workload_index, _ACT, act_index, 1_000_000)
    return np.sort(rng.choice(k, size=count, replace=False))


def activations(wl: Workload, act_index: int, tokens: int, k: int) -> np.ndarray:
    """bf16 bit patterns [tokens][k] for activation input ``act_index`` of workload ``wl``."""
    rng = _rng(wl.index, _ACT, act_index, tokens)
    if wl.act_dist == "normal":
        x = rng.standard_normal((tokens, k), dtype=np.float32)
    elif wl.act_dist == "student_t4":
        x = rng.standard_t(4.0, size=(tokens, k)).astype(np.float32)
    elif wl.act_dist == "normal_outliers":
        x = rng.standard_normal((tokens, k), dtype=np.float32)
        x[:, outlier_channels(k, wl.index, act_index)] *= np.float32(20.0)
    else:
        raise ValueError(wl.act_dist)
    return f32_to_bf16_bits(x)


def latent_weights(wl: Workload, layer_index: int, n_out: int | None = None,
                   k: int | None = None) -> np.ndarray:
    """fp32 latent weights [n_out][k] (nn.Linear layout) for layer ``layer_index``.

    ``n_out``/``k`` default to the layer's shape; smaller values give a seeded sample of the same
    distribution (used for bounded CPU timing samples and quick tests).
    """
    layer = wl.layers[layer_index]
    n_out = layer.n_out if n_out is None else n_out
    k = layer.k if k is None else k
    rng = _rng(wl.index, _WEIGHT, layer_index, n_out * 1_000_003 + k)
    if wl.weight_dist == "normal":
        w = rng.standard_normal((n_out, k), dtype=np.float32) * np.float32(wl.weight_scale)
    elif wl.weight_dist == "normal_rowscaled":
        w = rng.standard_normal((n_out, k), dtype=np.float32) * np.float32(wl.weight_scale)
        row_scale = rng.uniform(0.5, 2.0, size=(n_out, 1)).astype(np.float32)
        w *= row_scale
    elif wl.weight_dist == "laplace":
        w = rng.laplace(0.0, wl.weight_scale, size=(n_out, k)).astype(np.float32)
    else:
        raise ValueError(wl.weight_dist)
    return np.ascontiguousarray(w, dtype=np.float32)


def grad_output(wl: Workload, layer_index: int, tokens: int) -> np.ndarray:
    """bf16 bit patterns [tokens][n_out]: a standard-normal stand-in for the gradient of layer
    ``layer_index``'s output (the pages give no gradient distribution)."""
    layer = wl.layers[layer_index]
    rng = _rng(wl.index, _GRAD, layer_index, tokens)
    return f32_to_bf16_bits(rng.standard_normal((tokens, layer.n_out), dtype=np.float32))


def layer_inputs(wl: Workload, layer_index: int, tokens: int):
    """(x_bf16_bits [tokens][K], w_latent [n_out][K]) for one layer of a workload."""
    layer = wl.layers[layer_index]
    return activations(wl, layer.act_input, tokens, layer.k), latent_weights(wl, layer_index)
