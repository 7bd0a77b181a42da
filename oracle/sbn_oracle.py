"""CPU oracle for the Sparse-BitNet BitLinear forward.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, obviously-correct statement of what the
hot path computes. Only the test suite, the smoke check of the entry module and the benchmark's
CPU-baseline leg may import it; the product path (the HIP library and its Python binding) never
does, and it shares no code, table or helper with that path.

Sources (page titles, with the section each step follows):
  [BitNet-blog]   "Microsoft BitNet 1.58: The Era of 1-Bit Large Language Models",
                  section "The BitLinear Layer" (five operations; the latent-weight paragraph
                  after it), "Training with the Straight-Through Estimator" (the backward pass
                  treats the quantizers as the identity) and "bitnet.cpp: Matrix-Free Inference"
                  (four ternary values per byte).
  [BitNet-index]  "BitNet b1.58: How Ternary Weights Cut LLM Memory by 82% Without Losing
                  Accuracy", section "How ternary quantization works during training".
  [Sparse-BitNet] "Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to Semi-Structured
                  Sparsity", Abstract (dynamic N:M sparsification jointly with 1.58-bit
                  quantization), Figure 6 (per-block threshold = the (N+1)-th largest normalized
                  magnitude, i.e. the N largest of each M-block are kept), Table 6 (N:8 sweep),
                  Figure 3 (b) (mask flip rate r_t between consecutive masks).
  [8:16]          "From 2:4 to 8:16 sparsity patterns in LLMs for Outliers and Weights with
                  Variance Correction", abstract / Core claim (8:16 pattern; 0.875 vs 0.75
                  metadata bits per element).

Readings taken where the pages are silent or disagree (each is also listed in the design notes):
  * weights are divided by their mean absolute value (the index page says "divided"; the blog's
    "multiply" would send every code to zero), then rounded to nearest and clamped to [-1, 1];
  * rounding is round-half-to-even;
  * the weight scale is one per tensor and is taken over the dense latent weights, before
    selection (Figure 6 places the thresholds on normalized magnitudes);
  * the activation scale is per token: absmax with a floor of 1e-5, symmetric 127 levels;
  * the parameter-free LayerNorm (operation 1) is the standard one without affine terms: fp64
    mean and biased variance, r = 1/sqrt(var + eps), z = bf16(fl32(fl32(x - mu) * r)) with mu and
    r rounded to fp32; the quantizer then takes z (the page says BF16 is quantized to INT8);
  * the int8 code sequence is s = fl32(127 / a'), v = fl32(x * s), q = clamp(rne(v), -127, 127);
  * the N:M groups are M consecutive weights along the reduction axis K of each output row;
    selection keys on |w|; ties go to the lower index; kept weights that ternarize to 0 still
    count as kept;
  * the packed layout ("RPF") puts, per output row, a code bitstream (2n bits per group: the kept
    codes in ascending position, 2-bit two's complement 00=0, 01=+1, 11=-1, LSB first) and, when
    n < m, a mask bitstream (m bits per group, bit i <-> position i of the group, LSB first); each
    stream is padded with zero bits to a whole byte per row;
  * the output is fp32 y = fl32(fl32(fl32(acc) * gamma) * fl32(a' / 127)).
  * variance correction (optional) rescales the ternary weights gamma * codes to the mean square of
    the dense ternary weights: gamma_out = fl32(gamma * sqrt(nd / ns)) per tensor;
  * the straight-through data gradient is dX = gamma * dY @ codes: both quantizers pass the
    gradient unchanged, so only the ternary weights of the forward remain; dY is bf16, dX fp32;
  * the mask flip rate r_t counts positions whose keep bit differs between consecutive masks,
    divided by the number of weights; a first mask is compared with one that keeps nothing;
  * the compact inference encoding keeps, per group, a nonzero mask (m bits) and n sign slots
    for the nonzero codes in ascending position (1 = -1), m + n bits per group, LSB first;
  * structured outliers (optional): the k largest |w| of each 256-group along K are kept apart
    as bf16 values; scale, selection and codes use the other weights (outlier positions as 0).

Floating point follows the precision the path decides integers in (fp32 scale and product); the
weight-scale sum is accumulated in fp64.
"""

from __future__ import annotations

import math

import numpy as np

ABSMAX_FLOOR = np.float32(1e-5)
QMAX = 127
SUPPORTED_M = (4, 8, 16)


# ----------------------------------------------------------------------------------------------
# Activations: [BitNet-blog] "The BitLinear Layer", operation 2; [BitNet-index] per-token INT8.
# ----------------------------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact: the bf16 pattern is the top half of the fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def act_absmax(x: np.ndarray) -> np.ndarray:
    """a'_t = max(max_k |x[t, k]|, 1e-5) per token row (fp32; max is exact)."""
    x = np.asarray(x, dtype=np.float32)
    assert np.all(np.isfinite(x)), "activations must be finite"
    if x.shape[1] == 0:
        return np.full(x.shape[0], ABSMAX_FLOOR, dtype=np.float32)
    return np.maximum(np.max(np.abs(x), axis=1), ABSMAX_FLOOR).astype(np.float32)


def act_scale(a_prime: np.ndarray) -> np.ndarray:
    """s_t = fl32(127 / a'_t), the correctly rounded fp32 quotient.

    Computed as an fp64 quotient rounded once to fp32; for division that double rounding equals
    the correctly rounded fp32 result because 53 >= 2*24 + 2.
    """
    return (np.float64(QMAX) / np.asarray(a_prime, dtype=np.float64)).astype(np.float32)


def f32_to_bf16_rne(z: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, rounded to nearest even (finite inputs)."""
    u = np.asarray(z, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def layernorm_bf16(x_bf16: np.ndarray, eps: float) -> np.ndarray:
    """Parameter-free LayerNorm ([BitNet-blog] "The BitLinear Layer", operation 1), output bf16.

    Statistics in fp64 (biased variance), normalization in fp32, one rounding to bf16:
    z = bf16(fl32(fl32(x - fl32(mu)) * fl32(1 / sqrt(var + eps)))).
    """
    x = bf16_to_f32(x_bf16).astype(np.float64)
    k = x.shape[1]
    mu = x.sum(axis=1) / np.float64(k)
    d = x - mu[:, None]
    var = (d * d).sum(axis=1) / np.float64(k)
    r = 1.0 / np.sqrt(var + np.float64(np.float32(eps)))
    x32 = x.astype(np.float32)
    z = (x32 - mu.astype(np.float32)[:, None]).astype(np.float32) * r.astype(np.float32)[:, None]
    return f32_to_bf16_rne(z.astype(np.float32))


def layernorm_quantize_act(x_bf16: np.ndarray, eps: float):
    """LayerNorm, then the absmax INT8 quantization of its bf16 output: (q, a')."""
    return quantize_act(layernorm_bf16(x_bf16, eps))


def quantize_act(x_bf16: np.ndarray):
    """Per-token absmax INT8 quantization.

    Returns (q int8 [T][K], a_prime fp32 [T]).  v = fl32(x * s) is exact in fp64 before its single
    rounding (an 8-bit by 24-bit significand product), so it is the fp32 product.
    """
    x = bf16_to_f32(x_bf16)
    a_prime = act_absmax(x)
    s = act_scale(a_prime)
    v = (x.astype(np.float64) * s.astype(np.float64)[:, None]).astype(np.float32)
    q = np.clip(np.rint(v), -QMAX, QMAX).astype(np.int8)
    return q, a_prime


# ----------------------------------------------------------------------------------------------
# Weights: [BitNet-blog] operation 3 + [BitNet-index] absmean; [Sparse-BitNet] Abstract, Fig. 6.
# ----------------------------------------------------------------------------------------------

def absmean_gamma(w: np.ndarray) -> np.float32:
    """gamma = fl32( (sum |w| in fp64) / (n_out * K) ), one scale per tensor over dense weights.

    NumPy's fp64 sum (pairwise) is within ~1e-15 relative of the exact sum.
    """
    w = np.asarray(w, dtype=np.float32)
    assert np.all(np.isfinite(w)), "latent weights must be finite"
    if w.size == 0:
        return np.float32(0.0)
    total = np.sum(np.abs(w.astype(np.float64)), dtype=np.float64)
    return np.float32(total / np.float64(w.size))


def check_pattern(n: int, m: int, k: int) -> None:
    if m not in SUPPORTED_M:
        raise ValueError(f"m must be one of {SUPPORTED_M}, got {m}")
    if not 1 <= n <= m:
        raise ValueError(f"need 1 <= n <= m, got n={n}, m={m}")
    if k % m:
        raise ValueError(f"K={k} is not a multiple of m={m}")


def nm_keep_mask(w: np.ndarray, n: int, m: int) -> np.ndarray:
    """Keep mask (bool [n_out][K]): in each group of m consecutive weights along K, the n with the
    largest |w|; equal magnitudes are ordered by position (lower index first)."""
    w = np.asarray(w, dtype=np.float32)
    n_out, k = w.shape
    check_pattern(n, m, k)
    mag = np.abs(w).reshape(n_out, k // m, m)
    # A stable sort of -|w| lists equal magnitudes in ascending position.
    order = np.argsort(-mag, axis=2, kind="stable")
    keep = np.zeros(mag.shape, dtype=bool)
    np.put_along_axis(keep, order[:, :, :n], True, axis=2)
    return keep.reshape(n_out, k)


def ternary_codes(w: np.ndarray, keep: np.ndarray, gamma: np.float32) -> np.ndarray:
    """code = keep ? RoundClip(w / gamma, -1, 1) : 0, as int8 in {-1, 0, +1}.

    With round-half-to-even, RoundClip(w / gamma) is nonzero exactly when |w| > gamma / 2, so the
    code is taken by that exact comparison (gamma / 2 is exact in fp32) instead of a rounded
    quotient.
    """
    w = np.asarray(w, dtype=np.float32)
    half = np.float32(0.5) * np.float32(gamma)
    nonzero = np.abs(w) > half
    return np.where(keep & nonzero, np.sign(w), 0).astype(np.int8)


def rpf_row_bytes(n: int, m: int, k: int):
    """(code bytes per row, mask bytes per row) of the packed layout."""
    groups = k // m
    code_bytes = (groups * 2 * n + 7) // 8
    mask_bytes = (k + 7) // 8 if n < m else 0
    return code_bytes, mask_bytes


def rpf_pack(codes: np.ndarray, keep: np.ndarray, n: int, m: int):
    """Packed layout: per row a code bitstream and (n < m) a mask bitstream, LSB first.

    [BitNet-blog] "bitnet.cpp" packs four ternary values per byte (2 bits each); the per-group mask
    is the index metadata.  Returns (code_bytes uint8 [n_out][cb], mask_bytes uint8 [n_out][mb]).
    """
    n_out, k = codes.shape
    check_pattern(n, m, k)
    groups = k // m
    kept = codes.reshape(n_out, groups, m)[keep.reshape(n_out, groups, m)]
    kept = kept.reshape(n_out, groups * n)
    two_bit = kept.astype(np.int16) & 3  # two's complement: 0 -> 00, +1 -> 01, -1 -> 11
    bits = np.empty((n_out, groups * n * 2), dtype=np.uint8)
    bits[:, 0::2] = two_bit & 1
    bits[:, 1::2] = two_bit >> 1
    code_bytes = np.packbits(bits, axis=1, bitorder="little")
    if n < m:
        mask_bytes = np.packbits(keep.astype(np.uint8), axis=1, bitorder="little")
    else:
        mask_bytes = np.zeros((n_out, 0), dtype=np.uint8)
    cb, mb = rpf_row_bytes(n, m, k)
    assert code_bytes.shape == (n_out, cb) and mask_bytes.shape == (n_out, mb)
    return code_bytes, mask_bytes


def rpf_unpack(code_bytes: np.ndarray, mask_bytes: np.ndarray, n: int, m: int, k: int):
    """Inverse of rpf_pack: (codes int8 [n_out][K], keep bool [n_out][K])."""
    n_out = code_bytes.shape[0]
    groups = k // m
    bits = np.unpackbits(code_bytes, axis=1, bitorder="little")[:, : groups * n * 2]
    two_bit = bits[:, 0::2].astype(np.int8) | (bits[:, 1::2].astype(np.int8) << 1)
    values = np.where(two_bit == 3, -1, two_bit).astype(np.int8)  # 10 is never written
    if n < m:
        keep = np.unpackbits(mask_bytes, axis=1, bitorder="little")[:, :k].astype(bool)
    else:
        keep = np.ones((n_out, k), dtype=bool)
    codes = np.zeros((n_out, k), dtype=np.int8)
    codes[keep] = values.reshape(-1)
    return codes, keep


def pack_nm_ternary(w: np.ndarray, n: int, m: int) -> dict:
    """absmean -> keep mask -> codes -> packed bytes, for one latent weight tensor."""
    gamma = absmean_gamma(w)
    keep = nm_keep_mask(w, n, m)
    codes = ternary_codes(w, keep, gamma)
    code_bytes, mask_bytes = rpf_pack(codes, keep, n, m)
    return {"gamma": gamma, "keep": keep, "codes": codes,
            "code_bytes": code_bytes, "mask_bytes": mask_bytes}


# ----------------------------------------------------------------------------------------------
# Matmul and dequantization: [BitNet-blog] operations 4 and 5.
# ----------------------------------------------------------------------------------------------

def int_matmul(q: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """acc[t, r] = sum_k q[t, k] * code[r, k], exact.

    Every partial sum is an integer of magnitude <= 127 * K < 2^53, so the fp64 matrix product is
    exact regardless of its blocking order.
    """
    acc = np.asarray(q, dtype=np.float64) @ np.asarray(codes, dtype=np.float64).T
    assert np.all(np.abs(acc) < 2.0**31)
    return acc.astype(np.int32)


def dequantize(acc: np.ndarray, gamma: np.float32, a_prime: np.ndarray) -> np.ndarray:
    """y[t, r] = fl32( fl32( fl32(acc) * gamma ) * fl32(a'_t / 127) )."""
    acc_f = np.asarray(acc).astype(np.float32)  # exact: |acc| < 2^24
    act_step = (np.asarray(a_prime, dtype=np.float32) / np.float32(QMAX)).astype(np.float32)
    return ((acc_f * np.float32(gamma)).astype(np.float32) * act_step[:, None]).astype(np.float32)


def bitlinear_forward(x_bf16: np.ndarray, w: np.ndarray, n: int, m: int) -> dict:
    """Whole forward: quantize activations, pack weights, integer matmul, dequantize."""
    q, a_prime = quantize_act(x_bf16)
    packed = pack_nm_ternary(w, n, m)
    acc = int_matmul(q, packed["codes"])
    y = dequantize(acc, packed["gamma"], a_prime)
    return dict(packed, q=q, a_prime=a_prime, acc=acc, y=y)


# ----------------------------------------------------------------------------------------------
# Variance correction: [8:16] method summary (after pruning, the remaining weights are rescaled
# back to the dense variance). The page gives no formula; the reading applies it to the weights
# the matmul uses, gamma * codes, per tensor like gamma: their mean square is gamma^2 times the
# share of nonzero codes, so the factor is sqrt(nonzero dense codes / nonzero n:m codes).
# ----------------------------------------------------------------------------------------------

def variance_correction(w: np.ndarray, n: int, m: int) -> dict:
    """gamma, the nonzero counts nd (dense ternary, n = m) and ns (n:m ternary), and the output
    scale gamma_out = fl32(gamma * sqrt(nd / ns)) (gamma when ns == 0)."""
    w = np.asarray(w, dtype=np.float32)
    gamma = absmean_gamma(w)
    dense = ternary_codes(w, np.ones(w.shape, dtype=bool), gamma)
    sparse = ternary_codes(w, nm_keep_mask(w, n, m), gamma)
    nd = int(np.count_nonzero(dense))
    ns = int(np.count_nonzero(sparse))
    if ns == 0:
        gamma_out = np.float32(gamma)
    else:
        gamma_out = np.float32(np.float64(gamma) * np.sqrt(np.float64(nd) / np.float64(ns)))
    return {"gamma": gamma, "nd": nd, "ns": ns, "gamma_out": gamma_out}


# ----------------------------------------------------------------------------------------------
# Structured outliers: [8:16] summary ("Summary", "Key points": salient weights kept in structured
# 4:256, 8:256 or 16:256 patterns, about 1.5%, 3.1% and 6.25% of the weights). Reading: in each
# group of 256 consecutive weights along K, the k of largest |w| (equal magnitudes: lower position
# first) are kept apart as bf16 values; the ternary n:m path then sees the other weights only
# (outlier positions read as 0 for the scale, the selection and the codes).
# ----------------------------------------------------------------------------------------------

OUTLIER_GROUP = 256


def outlier_select(w: np.ndarray, k: int):
    """(pos uint8 [n_out][K/256][k] ascending, val uint16 bf16 bits [n_out][K/256][k],
    mask bool [n_out][K]) of the k largest |w| in each group of 256 along K."""
    w = np.asarray(w, dtype=np.float32)
    n_out, K = w.shape
    if K % OUTLIER_GROUP != 0 or k not in (4, 8, 16):
        raise ValueError("outliers need K % 256 == 0 and k in {4, 8, 16}")
    groups = K // OUTLIER_GROUP
    mag = np.abs(w).reshape(n_out, groups, OUTLIER_GROUP)
    order = np.argsort(-mag, axis=2, kind="stable")  # equal magnitudes: ascending position
    pos = np.sort(order[:, :, :k], axis=2)
    vals = np.take_along_axis(w.reshape(n_out, groups, OUTLIER_GROUP), pos, axis=2)
    mask = np.zeros((n_out, groups, OUTLIER_GROUP), dtype=bool)
    np.put_along_axis(mask, pos, True, axis=2)
    return (pos.astype(np.uint8), f32_to_bf16_rne(vals).astype(np.uint16),
            mask.reshape(n_out, K))


def pack_with_outliers(w: np.ndarray, n: int, m: int, k: int) -> dict:
    """Outliers apart, then absmean / keep mask / codes of the remaining weights w' (w with the
    outlier positions set to 0)."""
    w = np.asarray(w, dtype=np.float32)
    pos, val, omask = outlier_select(w, k)
    w_rest = np.where(omask, np.float32(0.0), w).astype(np.float32)
    gamma = absmean_gamma(w_rest)
    keep = nm_keep_mask(w_rest, n, m)
    codes = ternary_codes(w_rest, keep, gamma)
    return {"gamma": gamma, "keep": keep, "codes": codes, "w_rest": w_rest,
            "opos": pos, "oval": val, "omask": omask}


def outlier_matrix(pos: np.ndarray, val: np.ndarray, K: int) -> np.ndarray:
    """The outliers as a dense fp64 matrix [n_out][K] (zero elsewhere)."""
    n_out, groups, k = pos.shape
    dense = np.zeros((n_out, K), dtype=np.float64)
    cols = pos.astype(np.int64) + OUTLIER_GROUP * np.arange(groups)[None, :, None]
    rows = np.broadcast_to(np.arange(n_out)[:, None, None], cols.shape)
    dense[rows, cols] = bf16_to_f32(val).astype(np.float64)
    return dense


def forward_with_outliers(q: np.ndarray, a_prime: np.ndarray, codes: np.ndarray,
                          gamma: np.float32, pos: np.ndarray, val: np.ndarray) -> dict:
    """y = (gamma * acc + o) * a'/127 in fp64, with acc the ternary accumulators and o = x_q @ O^T
    the outlier term (exact: products of int8 and bf16 values summed in fp64). Also returns the
    magnitude sum |gamma acc| + |x_q| @ |O|^T that bounds the fp32 evaluation's rounding."""
    K = codes.shape[1]
    acc = int_matmul(q, codes)
    O = outlier_matrix(pos, val, K)
    qf = np.asarray(q, dtype=np.float64)
    o = qf @ O.T
    step = np.asarray(a_prime, dtype=np.float64)[:, None] / 127.0
    y = (np.float64(gamma) * acc.astype(np.float64) + o) * step
    mag = (np.abs(np.float64(gamma) * acc.astype(np.float64)) + np.abs(qf) @ np.abs(O).T) * step
    return {"acc": acc, "o": o, "y": y, "mag": mag}


# ----------------------------------------------------------------------------------------------
# Data gradient under the straight-through estimator: [BitNet-blog] "Training with the
# Straight-Through Estimator" (the backward pass treats the quantizers as the identity) with the
# forward of "The BitLinear Layer" (y from the ternary weights gamma * codes).
# ----------------------------------------------------------------------------------------------

def ste_dx(dy_bf16: np.ndarray, codes: np.ndarray, gamma: np.float32) -> np.ndarray:
    """dX = gamma * dY @ codes (fp64, one rounding to fp32 at the end).

    dy_bf16: bf16 bit patterns [T][n_out]; codes: ternary int8 [n_out][K]. Every product is a bf16
    value or zero, and the fp64 sum of up to 2^20 of them is exact for gradients of ordinary range.
    """
    dy = bf16_to_f32(dy_bf16).astype(np.float64)
    c = np.asarray(codes, dtype=np.float64)
    return (np.float64(gamma) * (dy @ c)).astype(np.float32)


def ste_dx_abs(dy_bf16: np.ndarray, codes: np.ndarray, gamma: np.float32) -> np.ndarray:
    """gamma * |dY| @ |codes| (fp64): the magnitude that bounds the rounding error of any fp32
    summation order of dX (recursive-summation bound)."""
    dy = np.abs(bf16_to_f32(dy_bf16).astype(np.float64))
    c = np.abs(np.asarray(codes, dtype=np.float64))
    return np.float64(gamma) * (dy @ c)


# ----------------------------------------------------------------------------------------------
# Mask flips between consecutive re-packs: [Sparse-BitNet] Figure 3 (b), the mask flip rate r_t.
# The page plots r_t but does not print its formula; the plainest reading is the share of weight
# positions whose keep decision differs between two consecutive masks.
# ----------------------------------------------------------------------------------------------

def mask_flips(keep_prev, keep_new) -> int:
    """Number of positions whose keep bit differs between two masks of the same shape.

    ``keep_prev`` may be None, which stands for a mask that keeps nothing (no earlier pack).
    r_t = mask_flips(prev, new) / new.size.
    """
    new = np.asarray(keep_new, dtype=bool)
    prev = np.zeros_like(new) if keep_prev is None else np.asarray(keep_prev, dtype=bool)
    if prev.shape != new.shape:
        raise ValueError(f"mask shapes differ: {prev.shape} vs {new.shape}")
    return int(np.count_nonzero(prev != new))


# ----------------------------------------------------------------------------------------------
# Compact inference encoding: [BitNet-blog] "Why 1.58 Bits?" (a ternary weight holds log2 3 bits)
# and "bitnet.cpp: Matrix-Free Inference" (packed ternary weights are unpacked on chip);
# [8:16] abstract (the per-group metadata cost of an n:m pattern). Once packed, the product needs
# only which positions are nonzero and their signs: a pruned position and a kept zero both give 0.
# ----------------------------------------------------------------------------------------------

def compact_row_bytes(n: int, m: int, k: int) -> int:
    """Bytes per row of the compact encoding: m + n bits per group, padded to a byte."""
    return ((k // m) * (m + n) + 7) // 8


def compact_pack(codes: np.ndarray, n: int, m: int) -> np.ndarray:
    """Compact encoding of n:m ternary codes, per row, LSB first.

    Group g (positions g*m .. g*m+m-1) owns bits [g*(m+n), (g+1)*(m+n)) of the row stream:
      bit i      (0 <= i < m): 1 when position g*m + i holds a nonzero code;
      bit m + j  (0 <= j < n): 1 when the group's j-th nonzero code, counting by ascending
                               position, is -1; slots past the group's nonzero count are 0.
    Requires at most n nonzero codes per group (true of every n:m pack).  Returns uint8
    [n_out][compact_row_bytes].
    """
    codes = np.asarray(codes, dtype=np.int8)
    n_out, k = codes.shape
    check_pattern(n, m, k)
    groups = k // m
    c = codes.reshape(n_out, groups, m)
    nz = c != 0
    if np.any(nz.sum(axis=2) > n):
        raise ValueError("a group has more than n nonzero codes")
    rank = np.cumsum(nz, axis=2) - 1  # index of each nonzero among its group's nonzeros
    slots = np.zeros((n_out, groups, n), dtype=bool)
    for j in range(n):
        slots[:, :, j] = np.any(nz & (rank == j) & (c < 0), axis=2)
    bits = np.concatenate([nz, slots], axis=2).reshape(n_out, groups * (m + n))
    out = np.packbits(bits.astype(np.uint8), axis=1, bitorder="little")
    assert out.shape == (n_out, compact_row_bytes(n, m, k))
    return out


def compact_unpack(data: np.ndarray, n: int, m: int, k: int) -> np.ndarray:
    """Inverse of compact_pack: ternary codes int8 [n_out][K]. Rejects streams whose unused sign
    slots or padding bits are not zero."""
    data = np.asarray(data, dtype=np.uint8)
    n_out = data.shape[0]
    groups = k // m
    allbits = np.unpackbits(data, axis=1, bitorder="little")
    if np.any(allbits[:, groups * (m + n):]):
        raise ValueError("nonzero padding bits")
    bits = allbits[:, : groups * (m + n)].reshape(n_out, groups, m + n).astype(bool)
    nz, slots = bits[:, :, :m], bits[:, :, m:]
    count = nz.sum(axis=2)
    if np.any(count > n):
        raise ValueError("a group has more than n nonzero positions")
    if np.any(slots & (np.arange(n) >= count[:, :, None])):
        raise ValueError("a sign slot past the group's nonzero count is set")
    rank = np.cumsum(nz, axis=2) - 1
    neg = np.take_along_axis(slots, np.clip(rank, 0, n - 1), axis=2) & nz
    codes = np.where(nz, np.where(neg, -1, 1), 0).astype(np.int8)
    return codes.reshape(n_out, k)


# ----------------------------------------------------------------------------------------------
# Combinatorial mask rank: the metadata sizes the pages print (0.75 bits/element for 2:4, 0.875 for
# 8:16; [8:16] abstract, Sparse-BitNet "Sparse-BitNet" section) are ceil(log2 C(m, n)) / m, the
# width of a fixed-size index of the n-of-m choice. Each group's choice is written as its rank in
# the combinatorial number system (colexicographic order of the kept positions, the textbook
# bijection between n-subsets of {0..m-1} and 0 .. C(m, n) - 1), then its n kept codes.
# ----------------------------------------------------------------------------------------------

def rank_bits(n: int, m: int) -> int:
    """Bits of a group's rank: ceil(log2 C(m, n)) (0 when n == m: one choice)."""
    c = math.comb(m, n)
    return (c - 1).bit_length()


def rank_row_bytes(n: int, m: int, k: int) -> int:
    """Bytes per row of the rank encoding: rank_bits + 2n bits per group, padded to a byte."""
    return ((k // m) * (rank_bits(n, m) + 2 * n) + 7) // 8


def mask_rank(positions) -> int:
    """Rank of an n-subset (ascending positions c_0 < ... < c_{n-1}) in the combinatorial number
    system: sum over i of C(c_i, i + 1)."""
    return sum(math.comb(c, i + 1) for i, c in enumerate(positions))


def mask_unrank(r: int, n: int, m: int) -> list:
    """Inverse of mask_rank: the ascending positions of rank r (0 <= r < C(m, n)). Greedy from the
    largest element: c_{i-1} is the largest c with C(c, i) <= the remaining rank."""
    if not 0 <= r < math.comb(m, n):
        raise ValueError("rank out of range")
    out = []
    for i in range(n, 0, -1):
        c = i - 1
        while c + 1 < m and math.comb(c + 1, i) <= r:
            c += 1
        r -= math.comb(c, i)
        out.append(c)
    return out[::-1]


def rank_pack(codes: np.ndarray, keep: np.ndarray, n: int, m: int) -> np.ndarray:
    """Rank encoding of an n:m pack, per row, LSB first. Group g owns bits
    [g (R + 2n), (g + 1)(R + 2n)), R = rank_bits(n, m): first the rank of its keep mask, then the
    two's-complement low two bits of its n kept codes by ascending position (0 -> 00, +1 -> 01,
    -1 -> 11, as in the 2-bit code stream of rpf_pack). Returns uint8 [n_out][rank_row_bytes]."""
    codes = np.asarray(codes, dtype=np.int8)
    keep = np.asarray(keep, dtype=bool)
    n_out, k = codes.shape
    check_pattern(n, m, k)
    groups = k // m
    R = rank_bits(n, m)
    per = R + 2 * n
    bits = np.zeros((n_out, groups * per), dtype=np.uint8)
    for row in range(n_out):
        for g in range(groups):
            sel = np.flatnonzero(keep[row, g * m:(g + 1) * m])
            if sel.size != n:
                raise ValueError("a group does not keep exactly n positions")
            r = mask_rank(sel.tolist())
            base = g * per
            for b in range(R):
                bits[row, base + b] = (r >> b) & 1
            for j, p in enumerate(sel):
                two = int(codes[row, g * m + p]) & 3
                bits[row, base + R + 2 * j] = two & 1
                bits[row, base + R + 2 * j + 1] = two >> 1
    out = np.packbits(bits, axis=1, bitorder="little")
    if out.shape[1] < rank_row_bytes(n, m, k):  # k == 0
        out = np.zeros((n_out, rank_row_bytes(n, m, k)), dtype=np.uint8)
    return out


def rank_unpack(data: np.ndarray, n: int, m: int, k: int):
    """Inverse of rank_pack: (codes int8 [n_out][K], keep bool [n_out][K]). Rejects ranks out of
    range, the code 10 and nonzero padding bits."""
    data = np.asarray(data, dtype=np.uint8)
    n_out = data.shape[0]
    groups = k // m
    R = rank_bits(n, m)
    per = R + 2 * n
    allbits = np.unpackbits(data, axis=1, bitorder="little")
    if np.any(allbits[:, groups * per:]):
        raise ValueError("nonzero padding bits")
    codes = np.zeros((n_out, k), dtype=np.int8)
    keep = np.zeros((n_out, k), dtype=bool)
    for row in range(n_out):
        for g in range(groups):
            b = allbits[row, g * per:(g + 1) * per].astype(np.int64)
            r = int(sum(int(b[i]) << i for i in range(R)))
            pos = mask_unrank(r, n, m)
            for j, p in enumerate(pos):
                two = int(b[R + 2 * j]) | (int(b[R + 2 * j + 1]) << 1)
                if two == 2:
                    raise ValueError("code 10 is never written")
                codes[row, g * m + p] = -1 if two == 3 else two
                keep[row, g * m + p] = True
    return codes, keep


# ----------------------------------------------------------------------------------------------
# Metadata size: [8:16] abstract (0.875 vs 0.75 bits/element).
# ----------------------------------------------------------------------------------------------

def combinatorial_metadata_bits(n: int, m: int) -> float:
    """Bits per element of the smallest fixed-width index of an n-of-m choice:
    ceil(log2 C(m, n)) / m."""
    return math.ceil(math.log2(math.comb(m, n))) / m


def boundary_elements_act(x_bf16: np.ndarray, a_prime: np.ndarray, rel: float = 1e-6):
    """Elements whose exact 127*x/a' lies within ``rel`` (relative) of a k + 0.5 rounding boundary.

    Computed in fp64; used to count (not excuse silently) int8 mismatches near a boundary.
    """
    x = bf16_to_f32(x_bf16).astype(np.float64)
    v = np.abs(x * (QMAX / np.asarray(a_prime, dtype=np.float64))[:, None])
    frac = v - np.floor(v)
    return (np.abs(frac - 0.5) <= rel * np.maximum(v, 1e-300)) & (v > 0)


def boundary_elements_weight(w: np.ndarray, gamma: np.float32, rel: float = 1e-6):
    """Weights with ||w| - gamma/2| <= rel * gamma/2 (codes there may legitimately flip)."""
    half = np.float64(gamma) / 2.0
    return np.abs(np.abs(np.asarray(w, dtype=np.float64)) - half) <= rel * half
