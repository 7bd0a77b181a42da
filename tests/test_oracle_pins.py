"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU needed).

Each test checks the oracle against something other than itself: the hand-derived worked example,
the metadata sizes the pages print, a pure-Python brute force, closed-form zero fractions,
invariants, special cases that reduce to textbook definitions, and symmetries.
"""

import itertools
import json
import math
import os
import struct

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy import integrate, special

import oracle
from sparsity_sbn_quantize_amd import inputs
from tests.conftest import GOLDEN

PATTERNS = [(2, 4), (1, 4), (3, 4), (4, 4), (8, 8), (7, 8), (6, 8), (5, 8), (4, 8), (3, 8),
            (2, 8), (1, 8), (8, 16), (4, 16), (12, 16), (16, 16), (1, 16)]


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------------------------
# Worked example (hand-derived from the definitions; fixture carries the citation).
# ---------------------------------------------------------------------------------------------

def test_worked_example_2of4():
    g = load("worked_example_2of4.json")
    exp = g["expected"]
    w = np.array([g["w"]], dtype=np.float32)
    x = inputs.f32_to_bf16_bits(np.array([g["x"]], dtype=np.float32))
    assert np.array_equal(inputs.bf16_bits_to_f32(x)[0], np.array(g["x"], np.float32)), \
        "example activations must be exact in bf16"
    r = oracle.bitlinear_forward(x, w, 2, 4)
    assert r["gamma"] == np.float32(exp["gamma"])
    assert r["a_prime"][0] == np.float32(exp["a_prime"])
    assert r["q"][0].tolist() == exp["q"]
    assert r["keep"][0].astype(int).tolist() == exp["keep_2of4"]
    assert r["codes"][0].tolist() == exp["codes_2of4"]
    assert r["code_bytes"][0].tolist() == exp["code_bytes_2of4"]
    assert r["mask_bytes"][0].tolist() == exp["mask_bytes_2of4"]
    assert int(r["acc"][0, 0]) == exp["acc_2of4"]
    assert r["y"][0, 0] == np.float32(exp["y_2of4"])

    d = oracle.bitlinear_forward(x, w, 4, 4)
    assert d["codes"][0].tolist() == exp["codes_dense"]
    assert d["code_bytes"][0].tolist() == exp["code_bytes_dense_4of4"]
    assert d["mask_bytes"].shape == (1, 0)
    assert int(d["acc"][0, 0]) == exp["acc_dense"]
    assert d["y"][0, 0] == np.float32(exp["y_dense"])


def test_metadata_bits_match_pages():
    g = load("metadata_bits.json")["bits_per_element"]
    assert oracle.combinatorial_metadata_bits(2, 4) == g["2:4"]
    assert oracle.combinatorial_metadata_bits(8, 16) == g["8:16"]


# ---------------------------------------------------------------------------------------------
# Brute force: a pure-Python, loop-by-loop restatement on tiny shapes.
# ---------------------------------------------------------------------------------------------

def f32(v: float) -> float:
    """Round a Python float (binary64) to the nearest binary32, ties to even."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def brute_forward(x_vals, w_vals, n, m):
    """Plain loops over Python floats and ints; no NumPy arithmetic."""
    T, K, N = len(x_vals), len(x_vals[0]), len(w_vals)
    floor = f32(1e-5)
    q, a_primes = [], []
    for t in range(T):
        a = 0.0
        for k in range(K):
            a = max(a, abs(x_vals[t][k]))
        a = max(a, floor)
        s = f32(127.0 / a)
        row = []
        for k in range(K):
            v = f32(x_vals[t][k] * s)
            r = round(v)  # Python rounds half to even
            row.append(max(-127, min(127, r)))
        q.append(row)
        a_primes.append(a)
    total = math.fsum(abs(w_vals[r][k]) for r in range(N) for k in range(K))
    gamma = f32(total / (N * K)) if N * K else 0.0
    half = f32(0.5 * gamma)
    codes = [[0] * K for _ in range(N)]
    keep = [[0] * K for _ in range(N)]
    for r in range(N):
        for g0 in range(0, K, m):
            order = sorted(range(m), key=lambda i: (-abs(w_vals[r][g0 + i]), i))
            for i in order[:n]:
                keep[r][g0 + i] = 1
                wv = w_vals[r][g0 + i]
                if abs(wv) > half:
                    codes[r][g0 + i] = 1 if wv > 0 else -1
    acc = [[0] * N for _ in range(T)]
    for t in range(T):
        for r in range(N):
            s = 0
            for k in range(K):
                s += q[t][k] * codes[r][k]
            acc[t][r] = s
    y = [[f32(f32(float(acc[t][r]) * gamma) * f32(a_primes[t] / 127.0)) for r in range(N)]
         for t in range(T)]
    # packed bytes, bit by bit
    code_rows, mask_rows = [], []
    for r in range(N):
        bits = []
        for g0 in range(0, K, m):
            for i in range(m):
                if keep[r][g0 + i]:
                    c = codes[r][g0 + i] & 3
                    bits += [c & 1, c >> 1]
        code_rows.append(_bits_to_bytes(bits))
        mask_rows.append(_bits_to_bytes(keep[r]) if n < m else [])
    return dict(q=q, a_prime=a_primes, gamma=gamma, keep=keep, codes=codes, acc=acc, y=y,
                code_bytes=code_rows, mask_bytes=mask_rows)


def _bits_to_bytes(bits):
    out = []
    for b0 in range(0, len(bits), 8):
        v = 0
        for i, b in enumerate(bits[b0:b0 + 8]):
            v |= b << i
        out.append(v)
    return out


# Values with many exact ties, signed zeros and bf16 half-boundaries.
_w_atoms = [0.0, -0.0, 0.125, -0.125, 0.25, -0.25, 0.375, 0.5, -0.5, 1.0, -1.0, 0.0625,
            -0.03125, 2.0, 0.75]
_x_atoms = [0.0, -0.0, 1.0, -1.0, 0.5, 0.25, -2.0, 1.984375, 0.9765625, 0.0078125, -1.0390625,
            3.0, -0.75, 127.0, 1e-6]


@st.composite
def tiny_case(draw):
    n, m = draw(st.sampled_from(PATTERNS))
    groups = draw(st.integers(1, 4 if m < 16 else 2))
    K = groups * m
    T = draw(st.integers(1, 4))
    N = draw(st.integers(1, 6))
    wv = st.one_of(st.sampled_from(_w_atoms),
                   st.floats(-0.125, 0.125, width=32, allow_subnormal=False))
    xv = st.one_of(st.sampled_from(_x_atoms), st.floats(-8, 8, width=32, allow_subnormal=False))
    w = np.array(draw(st.lists(st.lists(wv, min_size=K, max_size=K), min_size=N, max_size=N)),
                 dtype=np.float32)
    x = np.array(draw(st.lists(st.lists(xv, min_size=K, max_size=K), min_size=T, max_size=T)),
                 dtype=np.float32)
    return n, m, w, inputs.f32_to_bf16_bits(x)


@settings(max_examples=300, deadline=None)
@given(tiny_case())
def test_oracle_matches_brute_force(case):
    n, m, w, xb = case
    r = oracle.bitlinear_forward(xb, w, n, m)
    x_vals = inputs.bf16_bits_to_f32(xb).astype(np.float64).tolist()
    b = brute_forward(x_vals, w.astype(np.float64).tolist(), n, m)
    assert r["q"].tolist() == b["q"]
    assert r["a_prime"].tolist() == b["a_prime"]
    assert float(r["gamma"]) == b["gamma"]
    assert r["keep"].astype(int).tolist() == b["keep"]
    assert r["codes"].tolist() == b["codes"]
    assert r["code_bytes"].tolist() == b["code_bytes"]
    assert r["mask_bytes"].tolist() == b["mask_bytes"]
    assert r["acc"].tolist() == b["acc"]
    assert r["y"].tolist() == b["y"]


def test_brute_force_random_shapes():
    """Non-square shapes so a transposed operand cannot pass."""
    rng = np.random.default_rng(7)
    for (n, m) in [(2, 4), (6, 8), (8, 16), (3, 8)]:
        T, K, N = 3, 3 * m, 5
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        xb = inputs.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
        r = oracle.bitlinear_forward(xb, w, n, m)
        b = brute_forward(inputs.bf16_bits_to_f32(xb).astype(np.float64).tolist(),
                          w.astype(np.float64).tolist(), n, m)
        assert r["acc"].tolist() == b["acc"]
        assert r["y"].tolist() == b["y"]
        assert r["code_bytes"].tolist() == b["code_bytes"]


# ---------------------------------------------------------------------------------------------
# Closed forms: zero fraction of ternarized weights (dense and after n:m selection).
# ---------------------------------------------------------------------------------------------

def _gauss_abs(sigma):
    F = lambda u: special.erf(u / (sigma * math.sqrt(2.0)))
    f = lambda u: 2.0 * math.exp(-0.5 * (u / sigma) ** 2) / (sigma * math.sqrt(2.0 * math.pi))
    return F, f


def _laplace_abs(b):
    return (lambda u: 1.0 - math.exp(-u / b)), (lambda u: math.exp(-u / b) / b)


def masked_zero_fraction(F, f, half, n, m):
    """1 - P(kept and |w| > half): an element of magnitude u is kept when fewer than n of the
    other m-1 group members exceed it (continuous law, so no ties)."""
    def integrand(u):
        Fu = F(u)
        return f(u) * sum(math.comb(m - 1, j) * (1 - Fu) ** j * Fu ** (m - 1 - j)
                          for j in range(n))
    val, _ = integrate.quad(integrand, half, np.inf, limit=200)
    return 1.0 - val


def test_closed_form_population_values():
    """The closed forms at the population scale (gamma = E|w|) give the textbook constants."""
    s = 1.0
    F, f = _gauss_abs(s)
    half = s * math.sqrt(2 / math.pi) / 2
    assert abs(F(half) - special.erf(1 / (2 * math.sqrt(math.pi)))) < 1e-15
    assert abs(F(half) - 0.310064) < 5e-7
    Fl, fl = _laplace_abs(1.0)
    assert abs(Fl(0.5) - (1 - math.exp(-0.5))) < 1e-15
    assert abs(masked_zero_fraction(F, f, half, 2, 4) - 0.525188) < 5e-6
    assert abs(masked_zero_fraction(F, f, half, 6, 8) - 0.345973) < 5e-6
    assert abs(masked_zero_fraction(F, f, half, 8, 16) - 0.502719) < 5e-6
    assert abs(masked_zero_fraction(Fl, fl, 0.5, 8, 16) - 0.512764) < 5e-6
    # n = m keeps everything: the masked form reduces to the dense one.
    assert abs(masked_zero_fraction(F, f, half, 8, 8) - F(half)) < 1e-9


@pytest.mark.parametrize("dist,n,m", [("normal", 2, 4), ("normal", 6, 8), ("normal", 8, 16),
                                      ("normal", 8, 8), ("laplace", 8, 16), ("laplace", 4, 4)])
def test_zero_fraction_matches_closed_form(dist, n, m):
    rng = np.random.default_rng(11)
    N, K = 512, 2048
    if dist == "normal":
        sigma = 0.02
        w = (rng.standard_normal((N, K)) * sigma).astype(np.float32)
        F, f = _gauss_abs(sigma)
    else:
        b = 0.015
        w = rng.laplace(0, b, (N, K)).astype(np.float32)
        F, f = _laplace_abs(b)
    p = oracle.pack_nm_ternary(w, n, m)
    half = float(p["gamma"]) / 2.0  # realized scale
    expected = masked_zero_fraction(F, f, half, n, m)
    per_group = (p["codes"] == 0).reshape(-1, m).mean(axis=1)
    se = per_group.std(ddof=1) / math.sqrt(per_group.size)
    assert abs(per_group.mean() - expected) < 5 * se, (per_group.mean(), expected, se)


def test_zero_fraction_rowscaled_gaussian():
    """Per-row scale U(0.5, 2) on N(0, 0.02) with one per-tensor gamma (decode workload)."""
    w = inputs.latent_weights(inputs.W_DECODE, 0, n_out=1024, k=2560)
    p = oracle.pack_nm_ternary(w, 8, 8)
    half = float(p["gamma"]) / 2.0
    sig = 0.02
    expected, _ = integrate.quad(
        lambda s: special.erf(half / (sig * s * math.sqrt(2.0))) / 1.5, 0.5, 2.0)
    per_row = (p["codes"] == 0).mean(axis=1)
    se = per_row.std(ddof=1) / math.sqrt(per_row.size)
    assert abs(per_row.mean() - expected) < 5 * se + 1e-4, (per_row.mean(), expected, se)


# ---------------------------------------------------------------------------------------------
# Invariants.
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n,m", PATTERNS)
def test_invariants(n, m):
    rng = np.random.default_rng(n * 100 + m)
    N, K = 37, 8 * m
    # quantized magnitudes force many ties
    w = (rng.integers(-6, 7, (N, K)) * 0.01).astype(np.float32)
    xb = inputs.f32_to_bf16_bits(rng.standard_normal((5, K)).astype(np.float32) * 3)
    r = oracle.bitlinear_forward(xb, w, n, m)
    codes, keep = r["codes"], r["keep"]
    assert set(np.unique(codes)).issubset({-1, 0, 1})
    g_keep = keep.reshape(N, -1, m)
    g_codes = codes.reshape(N, -1, m)
    assert np.all(g_keep.sum(axis=2) == n)
    assert np.all((g_codes != 0).sum(axis=2) <= n)
    assert np.all(codes[~keep] == 0)
    mag = np.abs(w).reshape(N, -1, m)
    kept_min = np.where(g_keep, mag, np.inf).min(axis=2)
    pruned_max = np.where(~g_keep, mag, -np.inf).max(axis=2)
    assert np.all(kept_min >= pruned_max)
    # ties resolved toward the lower index: no pruned element of equal magnitude precedes a kept one
    for r_ in range(N):
        for g in range(K // m):
            for i in range(m):
                for j in range(i):
                    if mag[r_, g, i] == mag[r_, g, j] and g_keep[r_, g, i]:
                        assert g_keep[r_, g, j]
    q = r["q"].astype(int)
    assert q.min() >= -127 and q.max() <= 127
    assert np.all(np.abs(q).max(axis=1) == 127)
    back_codes, back_keep = oracle.rpf_unpack(r["code_bytes"], r["mask_bytes"], n, m, K)
    assert np.array_equal(back_codes, codes) and np.array_equal(back_keep, keep)
    cb, mb = oracle.rpf_row_bytes(n, m, K)
    assert r["code_bytes"].shape == (N, cb) and r["mask_bytes"].shape == (N, mb)
    assert cb == K * 2 * n // (8 * m) and mb == (K // 8 if n < m else 0)


def test_packed_bits_per_weight():
    """Code + mask bits per weight: (2n + m)/m, or 2 when n = m (no mask)."""
    for (n, m), bpw in {(2, 4): 2.0, (6, 8): 2.5, (8, 16): 2.0, (8, 8): 2.0, (4, 8): 2.0}.items():
        cb, mb = oracle.rpf_row_bytes(n, m, 2560)
        assert (cb + mb) * 8 / 2560 == bpw


# ---------------------------------------------------------------------------------------------
# Special cases that reduce to textbook definitions.
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("m", [4, 8, 16])
def test_dense_reduces_to_roundclip(m):
    """n = m keeps every weight, so codes = RoundClip(W / gamma, -1, 1) with the quotient taken in
    fp64 and rounded half-to-even (the BitNet b1.58 definition written directly)."""
    rng = np.random.default_rng(m)
    w = (rng.standard_normal((64, 16 * m)) * 0.02).astype(np.float32)
    w[0, :4] = [0.0, -0.0, 1e-9, -1e-9]
    p = oracle.pack_nm_ternary(w, m, m)
    mean_abs = math.fsum(abs(float(v)) for v in w.ravel()) / w.size
    assert p["gamma"] == np.float32(mean_abs)
    ref = np.clip(np.rint(w.astype(np.float64) / np.float64(p["gamma"])), -1, 1).astype(np.int8)
    assert np.array_equal(p["codes"], ref)
    assert np.all(p["keep"])


def test_exact_half_ties_round_to_zero():
    """|w| == gamma/2 exactly rounds to 0 (half to even), |w| just above rounds to +-1."""
    w = np.array([[0.5, 0.5, 0.5, 0.5, 1.5, 1.5, 1.5, 1.5]], np.float32)  # gamma = 1, half = 0.5
    p = oracle.pack_nm_ternary(w, 8, 8)
    assert p["gamma"] == 1.0
    assert p["codes"][0].tolist() == [0, 0, 0, 0, 1, 1, 1, 1]
    w2 = w.copy()
    w2[0, 0] = np.nextafter(np.float32(0.5), np.float32(1))
    w2[0, 4] = np.nextafter(np.float32(1.5), np.float32(0))  # keeps sum close; gamma now != 1
    p2 = oracle.pack_nm_ternary(w2, 8, 8)
    assert p2["codes"][0, 0] == (1 if w2[0, 0] > p2["gamma"] / 2 else 0)


def test_identity_weights():
    """W = I: dense codes are I, acc = q; 2:4 keeps the diagonal plus the lowest-index zero."""
    K = 64
    w = np.eye(K, dtype=np.float32)
    rng = np.random.default_rng(3)
    xb = inputs.f32_to_bf16_bits(rng.standard_normal((4, K)).astype(np.float32))
    r = oracle.bitlinear_forward(xb, w, 4, 4)
    assert np.array_equal(r["codes"], np.eye(K, dtype=np.int8))
    assert np.array_equal(r["acc"], r["q"].astype(np.int32))
    assert r["gamma"] == np.float32(1.0 / K)
    s = oracle.pack_nm_ternary(w, 2, 4)
    for row in range(K):
        g0 = row - row % 4
        kept = np.nonzero(s["keep"][row, g0:g0 + 4])[0].tolist()
        lowest_zero = min(i for i in range(4) if g0 + i != row)
        assert kept == sorted({row - g0, lowest_zero})


def test_all_equal_weights_sum_rows():
    """All-equal positive W (dense) gives acc = row sums of q."""
    w = np.full((8, 32), 0.01, np.float32)
    rng = np.random.default_rng(4)
    xb = inputs.f32_to_bf16_bits(rng.standard_normal((3, 32)).astype(np.float32))
    r = oracle.bitlinear_forward(xb, w, 8, 8)
    assert np.all(r["codes"] == 1)
    assert np.array_equal(r["acc"], np.repeat(r["q"].astype(np.int64).sum(1, keepdims=True),
                                                8, axis=1))
    # 2:4 on equal weights keeps positions 0, 1 of every group
    s = oracle.pack_nm_ternary(w, 2, 4)
    assert np.all(s["keep"].reshape(8, -1, 4)[:, :, :2]) and not s["keep"].reshape(8, -1, 4)[:, :, 2:].any()


def test_zero_and_tiny_rows():
    """An all-zero activation row gives a' = 1e-5 and q = 0; an all-zero W gives gamma = 0 and
    all codes 0."""
    x = np.zeros((2, 16), np.float32)
    x[1, 3] = 1e-30
    q, a = oracle.quantize_act(inputs.f32_to_bf16_bits(x))
    assert a[0] == np.float32(1e-5) and np.all(q[0] == 0)
    assert a[1] == np.float32(1e-5)
    p = oracle.pack_nm_ternary(np.zeros((4, 16), np.float32), 2, 4)
    assert p["gamma"] == 0 and np.all(p["codes"] == 0)
    assert np.all(p["keep"].reshape(4, -1, 4)[:, :, :2])


def test_empty_inputs():
    q, a = oracle.quantize_act(np.zeros((0, 16), np.uint16))
    assert q.shape == (0, 16) and a.shape == (0,)
    p = oracle.pack_nm_ternary(np.zeros((0, 16), np.float32), 2, 4)
    assert p["code_bytes"].shape == (0, 2) and p["mask_bytes"].shape == (0, 2)
    acc = oracle.int_matmul(np.zeros((0, 16), np.int8), p["codes"])
    assert acc.shape == (0, 0)


def test_pattern_validation():
    w = np.zeros((2, 12), np.float32)
    with pytest.raises(ValueError):
        oracle.nm_keep_mask(w, 2, 8)  # 12 % 8
    with pytest.raises(ValueError):
        oracle.nm_keep_mask(w, 0, 4)
    with pytest.raises(ValueError):
        oracle.nm_keep_mask(w, 5, 4)
    with pytest.raises(ValueError):
        oracle.nm_keep_mask(np.zeros((2, 12), np.float32), 2, 6)


# ---------------------------------------------------------------------------------------------
# Symmetries.
# ---------------------------------------------------------------------------------------------

def test_symmetries():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((16, 64)) * 0.02).astype(np.float32)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    xb = inputs.f32_to_bf16_bits(x)
    for n, m in [(2, 4), (6, 8), (8, 16)]:
        p = oracle.pack_nm_ternary(w, n, m)
        pn = oracle.pack_nm_ternary(-w, n, m)
        assert np.array_equal(pn["keep"], p["keep"]) and np.array_equal(pn["codes"], -p["codes"])
        p4 = oracle.pack_nm_ternary(w * np.float32(4.0), n, m)
        assert np.array_equal(p4["codes"], p["codes"]) and p4["gamma"] == p["gamma"] * 4
        # permuting whole groups along K (same permutation for x and w) leaves acc unchanged
        perm_groups = rng.permutation(64 // m)
        perm = (perm_groups[:, None] * m + np.arange(m)[None, :]).ravel()
        r = oracle.bitlinear_forward(xb, w, n, m)
        rp = oracle.bitlinear_forward(xb[:, perm], w[:, perm], n, m)
        assert np.array_equal(rp["acc"], r["acc"])
    q, a = oracle.quantize_act(xb)
    qn, an = oracle.quantize_act(inputs.f32_to_bf16_bits(-x))
    assert np.array_equal(qn, -q) and np.array_equal(an, a)
    q2, a2 = oracle.quantize_act(inputs.f32_to_bf16_bits(x * 8))
    assert np.array_equal(q2, q) and np.array_equal(a2, a * 8)


def test_boundary_counters():
    x = np.array([[1.984375, 0.9765625, 0.0078125, 0.25]], np.float32)  # s = 64: 62.5, 0.5 ties
    xb = inputs.f32_to_bf16_bits(x)
    q, a = oracle.quantize_act(xb)
    b = oracle.boundary_elements_act(xb, a)
    assert b[0].tolist() == [False, True, True, False]
    w = np.array([[0.5, 0.5, 0.5, 0.5, 1.5, 1.5, 1.5, 1.5]], np.float32)
    assert oracle.boundary_elements_weight(w, np.float32(1.0))[0].tolist() == [True] * 4 + [False] * 4


# ---------------------------------------------------------------------------------------------
# Mask flips between consecutive masks (Sparse-BitNet, Figure 3 (b), mask flip rate r_t).
# ---------------------------------------------------------------------------------------------

def test_mask_flips_hand_example():
    """2:4 on one row of two groups. Group 0 reverses its magnitude order, so the kept pair
    {0, 1} becomes {2, 3} (four positions change); group 1 keeps {2, 3} both times."""
    w1 = np.array([[4, 3, 2, 1, 1, 2, 3, 4]], dtype=np.float32)
    w2 = np.array([[1, 2, 3, 4, 1, 2, 3, 4]], dtype=np.float32)
    k1, k2 = oracle.nm_keep_mask(w1, 2, 4), oracle.nm_keep_mask(w2, 2, 4)
    assert k1.astype(int).tolist() == [[1, 1, 0, 0, 0, 0, 1, 1]]
    assert k2.astype(int).tolist() == [[0, 0, 1, 1, 0, 0, 1, 1]]
    assert oracle.mask_flips(k1, k2) == 4
    assert oracle.mask_flips(None, k1) == 4  # first mask: every kept position counts


def test_mask_flips_brute_force_and_metric():
    """Against a pure-Python bit count; symmetric; zero only for equal masks; triangle
    inequality; complement gives every position."""
    rng = np.random.default_rng(5)
    a, b, c = (rng.random((7, 24)) < 0.4 for _ in range(3))
    brute = sum(1 for i in range(7) for j in range(24) if bool(a[i, j]) != bool(b[i, j]))
    assert oracle.mask_flips(a, b) == brute
    assert oracle.mask_flips(b, a) == brute
    assert oracle.mask_flips(a, a) == 0
    assert oracle.mask_flips(a, c) <= oracle.mask_flips(a, b) + oracle.mask_flips(b, c)
    assert oracle.mask_flips(a, ~a) == a.size
    with pytest.raises(ValueError):
        oracle.mask_flips(a, b[:, :8])


@pytest.mark.parametrize("n,m", PATTERNS)
def test_mask_flips_nm_structure(n, m):
    """Two n:m masks keep n per group each, so a group changes an even number of positions, at
    most 2*min(n, m - n); a first mask counts n per group; positive scaling keeps the mask and
    n == m never flips."""
    rng = np.random.default_rng(31 * n + m)
    N, K = 9, 4 * m
    w1 = rng.standard_normal((N, K)).astype(np.float32)
    w2 = (w1 + 0.7 * rng.standard_normal((N, K))).astype(np.float32)
    k1, k2 = oracle.nm_keep_mask(w1, n, m), oracle.nm_keep_mask(w2, n, m)
    per_group = (k1 != k2).reshape(N, -1, m).sum(axis=2)
    assert np.all(per_group % 2 == 0)
    assert np.all(per_group <= 2 * min(n, m - n))
    assert oracle.mask_flips(k1, k2) == int(per_group.sum())
    assert oracle.mask_flips(None, k1) == N * K * n // m
    assert oracle.mask_flips(k1, oracle.nm_keep_mask(w1 * np.float32(3), n, m)) == 0
    if n == m:
        assert oracle.mask_flips(k1, k2) == 0


# ---------------------------------------------------------------------------------------------
# Straight-through data gradient (BitNet blog, "Training with the Straight-Through Estimator").
# ---------------------------------------------------------------------------------------------

def brute_ste_dx(dy_bits, codes, gamma):
    """Pure-Python dX = fl32(gamma * fsum_r dy[t][r] * code[r][k])."""
    dy = inputs.bf16_bits_to_f32(np.asarray(dy_bits)).astype(np.float64).tolist()
    cl = np.asarray(codes).astype(int).tolist()
    T, N, K = len(dy), len(cl), len(cl[0]) if cl else 0
    out = []
    for t in range(T):
        row = []
        for k in range(K):
            s = math.fsum(dy[t][r] * cl[r][k] for r in range(N))
            row.append(struct.unpack("f", struct.pack("f", float(gamma) * s))[0])
        out.append(row)
    return np.array(out, dtype=np.float32).reshape(T, K)


def _ste_case(seed, T, N, K, n, m):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    p = oracle.pack_nm_ternary(w, n, m)
    dy = inputs.f32_to_bf16_bits(rng.standard_normal((T, N)).astype(np.float32))
    return dy, p["codes"], p["gamma"], w


def _ste_pins_fail(fn) -> bool:
    """True when an implementation of dX disagrees with the brute force, the autograd adjoint or
    the one-hot rows (used on the oracle and on planted mistakes)."""
    import torch
    cases = [(3, 8, 12, 2, 4), (2, 16, 8, 6, 8), (4, 5, 16, 8, 16), (3, 16, 16, 8, 16)]
    for seed, (T, N, K, n, m) in enumerate(cases):
        dy, codes, gamma, _ = _ste_case(seed, T, N, K, n, m)
        got = fn(dy, codes, gamma)
        if got.shape != (T, K) or not np.array_equal(got, brute_ste_dx(dy, codes, gamma)):
            return True
        # autograd of the forward definition y = x (gamma C)^T, in fp64
        x = torch.zeros((T, K), dtype=torch.float64, requires_grad=True)
        wt = torch.from_numpy(np.float64(gamma) * codes.astype(np.float64))
        y = x @ wt.T
        y.backward(torch.from_numpy(inputs.bf16_bits_to_f32(dy).astype(np.float64)))
        if not np.allclose(got, x.grad.numpy(), rtol=2 ** -22, atol=0):
            return True
        # one-hot rows of dY select gamma times one code row
        onehot = np.zeros((N, N), np.float32)
        np.fill_diagonal(onehot, 1.0)
        sel = fn(inputs.f32_to_bf16_bits(onehot), codes, gamma)
        if not np.array_equal(sel, (np.float32(gamma) * codes.astype(np.float32))):
            return True
    return False


def test_ste_dx_pins():
    assert not _ste_pins_fail(oracle.ste_dx)


@pytest.mark.parametrize("mutant", ["no_gamma", "transposed", "negated", "dy_truncated",
                                    "codes_as_keep"])
def test_ste_dx_mutants_caught(mutant):
    """Plausible mistakes in the data gradient fail the pins."""
    def f(dy, codes, gamma):
        if mutant == "no_gamma":
            return oracle.ste_dx(dy, codes, np.float32(1.0))
        if mutant == "transposed":  # the codes' transpose (shape-compatible only when square)
            d = inputs.bf16_bits_to_f32(dy).astype(np.float64)
            c = codes.astype(np.float64)
            if c.shape[0] != c.shape[1]:
                return np.zeros((d.shape[0], c.shape[1]), np.float32)
            return (np.float64(gamma) * (d @ c.T)).astype(np.float32)
        if mutant == "negated":
            return -oracle.ste_dx(dy, codes, gamma)
        if mutant == "dy_truncated":  # dy taken as its integer part
            d = np.trunc(inputs.bf16_bits_to_f32(dy)).astype(np.float32)
            return oracle.ste_dx(inputs.f32_to_bf16_bits(d), codes, gamma)
        return oracle.ste_dx(dy, (codes != 0).astype(np.int8), gamma)
    assert _ste_pins_fail(f)


def test_ste_dx_abs_bounds_value():
    """|dX| <= gamma |dY| |C| elementwise, with equality where all terms share a sign."""
    dy, codes, gamma, _ = _ste_case(9, 5, 24, 32, 6, 8)
    dx = oracle.ste_dx(dy, codes, gamma).astype(np.float64)
    ab = oracle.ste_dx_abs(dy, codes, gamma)
    assert np.all(np.abs(dx) <= ab * (1 + 2 ** -23) + 1e-30)
    pos = np.abs(inputs.f32_to_bf16_bits(np.ones((2, 24), np.float32)))
    same = oracle.ste_dx(pos, np.abs(codes).astype(np.int8), gamma).astype(np.float64)
    assert np.allclose(same, oracle.ste_dx_abs(pos, codes, gamma), rtol=2 ** -23)


# ---------------------------------------------------------------------------------------------
# Parameter-free LayerNorm before the quantizer (BitNet blog, "The BitLinear Layer", op 1).
# ---------------------------------------------------------------------------------------------

def _fl32(v: float) -> float:
    return struct.unpack("f", struct.pack("f", v))[0]


def _bf16_bits_py(v: float) -> int:
    u = struct.unpack("I", struct.pack("f", v))[0]
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF


def brute_layernorm(x_bits, eps):
    """Pure Python: fsum statistics, fp32 normalization, bf16 rounding (bit patterns)."""
    xs = inputs.bf16_bits_to_f32(np.asarray(x_bits)).astype(np.float64).tolist()
    out = []
    for row in xs:
        k = len(row)
        mu = math.fsum(row) / k
        var = math.fsum((v - mu) ** 2 for v in row) / k
        r = 1.0 / math.sqrt(var + float(np.float32(eps)))
        mu32, r32 = _fl32(mu), _fl32(r)
        out.append([_bf16_bits_py(_fl32(_fl32(_fl32(v) - mu32) * r32)) for v in row])
    return np.array(out, dtype=np.uint16)


def _ln_pins_fail(fn) -> bool:
    import torch
    rng = np.random.default_rng(77)
    eps = 1e-5
    for T, K, scale in ((3, 8, 3.0), (2, 16, 3.0), (4, 12, 3.0), (3, 16, 1e-3)):
        # scale 1e-3 gives a variance below eps, where eps matters
        x = inputs.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32) * scale)
        with np.errstate(invalid="ignore", divide="ignore"):
            z = fn(x, eps)
        if z.shape != (T, K) or not np.array_equal(z, brute_layernorm(x, eps)):
            return True
    # the library LayerNorm (no affine) in fp64, to bf16 precision
    x = inputs.f32_to_bf16_bits(rng.standard_normal((6, 64)).astype(np.float32) * 2 - 0.5)
    ref = torch.nn.functional.layer_norm(
        torch.from_numpy(inputs.bf16_bits_to_f32(x).astype(np.float64)), (64,), eps=eps).numpy()
    z = inputs.bf16_bits_to_f32(fn(x, eps)).astype(np.float64)
    if not np.all(np.abs(z - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6):
        return True
    # scaling x by 2^k and eps by 4^k leaves every bit of z unchanged
    x2 = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x) * np.float32(8.0))
    if not np.array_equal(fn(x2, eps * 64.0), fn(x, eps)):
        return True
    # a constant row normalizes to zero
    c = inputs.f32_to_bf16_bits(np.full((2, 32), 1.75, np.float32))
    with np.errstate(invalid="ignore", divide="ignore"):
        zc = fn(c, eps)
    if not np.all(inputs.bf16_bits_to_f32(zc) == 0):
        return True
    return False


def test_layernorm_pins():
    assert not _ln_pins_fail(oracle.layernorm_bf16)


def test_layernorm_quantize_zero_rows():
    c = inputs.f32_to_bf16_bits(np.full((2, 32), -3.0, np.float32))
    q, a = oracle.layernorm_quantize_act(c, 1e-5)
    assert np.all(q == 0) and np.all(a == np.float32(1e-5))


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(3)
    z = np.concatenate([rng.standard_normal(5000).astype(np.float32),
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.0e38, 1e-40])])
    ours = oracle.f32_to_bf16_rne(z)
    ref = torch.from_numpy(z).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("mutant", ["unbiased", "no_eps", "var_not_std", "no_mean"])
def test_layernorm_mutants_caught(mutant):
    def f(x, eps):
        xv = inputs.bf16_bits_to_f32(x).astype(np.float64)
        k = xv.shape[1]
        mu = xv.mean(axis=1)
        d = xv - mu[:, None]
        if mutant == "unbiased":
            var = (d * d).sum(axis=1) / (k - 1)
        else:
            var = (d * d).sum(axis=1) / k
        if mutant == "no_eps":
            r = 1.0 / np.sqrt(var)
        elif mutant == "var_not_std":
            r = 1.0 / (var + eps)
        else:
            r = 1.0 / np.sqrt(var + eps)
        m32 = np.zeros_like(mu, dtype=np.float32) if mutant == "no_mean" else mu.astype(np.float32)
        z = (xv.astype(np.float32) - m32[:, None]).astype(np.float32) * r.astype(np.float32)[:, None]
        return oracle.f32_to_bf16_rne(z.astype(np.float32))
    assert _ln_pins_fail(f)


# ---------------------------------------------------------------------------------------------
# Variance correction (8:16 paper, method summary): gamma_out = gamma * sqrt(nd / ns).
# ---------------------------------------------------------------------------------------------

def _vc_pins_fail(fn) -> bool:
    """fn(w, n, m) -> dict with gamma_out, nd, ns."""
    g = load("worked_example_2of4.json")
    w = np.array([g["w"]], np.float32)
    r = fn(w, 2, 4)
    # hand count: dense codes [+1,-1,+1,+1,0,0,+1,+1] (6 nonzero), 2:4 codes [+1,-1,0,0,0,0,+1,+1]
    if r["nd"] != 6 or r["ns"] != 4:
        return True
    if r["gamma_out"] != np.float32(_fl32(0.48046875 * math.sqrt(6 / 4))):
        return True
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    # n = m: nothing is pruned, the scale is unchanged
    r = fn(w, 8, 8)
    if r["gamma_out"] != oracle.absmean_gamma(w):
        return True
    # population closed form for Gaussian weights: nonzero shares 1 - F(gamma/2) (dense) and
    # 1 - masked zero fraction (n:m) at the realized gamma
    w = (np.random.default_rng(22).standard_normal((512, 2048)) * 0.02).astype(np.float32)
    F, f = _gauss_abs(0.02)
    for n, m in ((2, 4), (8, 16)):
        r = fn(w, n, m)
        half = float(oracle.absmean_gamma(w)) / 2
        k2 = (1 - F(half)) / (1 - masked_zero_fraction(F, f, half, n, m))
        if abs(r["gamma_out"] / oracle.absmean_gamma(w) - math.sqrt(k2)) > 2e-3:
            return True
    # a power-of-two scale of the weights scales gamma_out exactly
    if fn(w * np.float32(4), 2, 4)["gamma_out"] != np.float32(4) * fn(w, 2, 4)["gamma_out"]:
        return True
    return False


def test_variance_correction_pins():
    assert not _vc_pins_fail(oracle.variance_correction)


@pytest.mark.parametrize("mutant", ["inverted", "squared", "keep_count"])
def test_variance_correction_mutants_caught(mutant):
    def f(w, n, m):
        r = dict(oracle.variance_correction(w, n, m))
        g64 = np.float64(r["gamma"])
        if mutant == "inverted":
            r["gamma_out"] = np.float32(g64 * np.sqrt(r["ns"] / r["nd"])) if r["nd"] else r["gamma"]
        elif mutant == "squared":
            r["gamma_out"] = np.float32(g64 * (r["nd"] / r["ns"])) if r["ns"] else r["gamma"]
        else:  # kept positions instead of nonzero codes
            ns = int(oracle.nm_keep_mask(w, n, m).sum())
            r["ns"] = ns
            r["gamma_out"] = np.float32(g64 * np.sqrt(r["nd"] / ns))
        return r
    assert _vc_pins_fail(f)


# ---------------------------------------------------------------------------------------------
# Compact inference encoding: per group, m nonzero-mask bits then n sign slots (1 = -1) for the
# nonzero codes in ascending position; m + n bits per group, LSB first.
# ---------------------------------------------------------------------------------------------

# Hand-encoded rows (codes, n, m, bytes). 2:4 [+1,-1,0,0 | 0,0,+1,+1] (the worked example's
# sparse codes): group 0 mask 1100, slots (0, 1); group 1 mask 0011, slots (0, 0): bits
# 110001 001100 -> 0x23 0x03. 6:8 [+1,0,-1,0,0,+1,-1,0]: mask 10100110, slots 0,1,0,1,0,0 ->
# 0x65 0x0A. 2:4 [0,0,0,-1 | -1,0,+1,0]: group 0 has one nonzero (slots 1, 0), group 1 mask 1010,
# slots (1, 0) -> bits 000110 101010 -> 0x58 0x05.
COMPACT_HAND = [
    ([1, -1, 0, 0, 0, 0, 1, 1], 2, 4, [0x23, 0x03]),
    ([1, 0, -1, 0, 0, 1, -1, 0], 6, 8, [0x65, 0x0A]),
    ([0, 0, 0, -1, -1, 0, 1, 0], 2, 4, [0x58, 0x05]),
]


def _compact_brute(codes, n, m):
    """Bit-by-bit encoder in plain Python."""
    out = []
    for row in codes:
        bits = []
        for g in range(len(row) // m):
            grp = [int(v) for v in row[g * m:(g + 1) * m]]
            bits += [1 if v != 0 else 0 for v in grp]
            signs = [1 if v < 0 else 0 for v in grp if v != 0]
            bits += signs + [0] * (n - len(signs))
        bits += [0] * (-len(bits) % 8)
        out.append([sum(b << i for i, b in enumerate(bits[o:o + 8]))
                    for o in range(0, len(bits), 8)])
    return np.array(out, np.uint8)


def _random_nm_codes(rng, n_out, k, n, m):
    """Ternary codes with at most n nonzeros per group (some groups with fewer)."""
    c = rng.integers(-1, 2, (n_out, k // m, m)).astype(np.int8)
    for r in range(n_out):
        for g in range(k // m):
            nz = np.flatnonzero(c[r, g])
            limit = rng.integers(0, n + 1)
            if len(nz) > limit:
                c[r, g, rng.choice(nz, len(nz) - limit, replace=False)] = 0
    return c.reshape(n_out, k)


def _compact_pins_fail(pack) -> bool:
    for codes, n, m, expect in COMPACT_HAND:
        if not np.array_equal(pack(np.array([codes], np.int8), n, m)[0], np.array(expect, np.uint8)):
            return True
    rng = np.random.default_rng(31)
    for n, m in ((2, 4), (6, 8), (8, 16), (3, 8), (1, 4), (8, 8), (12, 16)):
        c = _random_nm_codes(rng, 3, 4 * m, n, m)
        if not np.array_equal(pack(c, n, m), _compact_brute(c, n, m)):
            return True
    return False


def test_compact_pins():
    assert not _compact_pins_fail(oracle.compact_pack)


def test_compact_size():
    """m + n bits per group: 1.5 bits per weight at 2:4 and 8:16, 1.75 at 6:8, 2 when dense."""
    for (n, m), bpw in (((2, 4), 1.5), ((8, 16), 1.5), ((6, 8), 1.75), ((8, 8), 2.0),
                        ((4, 8), 1.5), ((3, 8), 1.375)):
        assert oracle.compact_row_bytes(n, m, 2560) * 8 == bpw * 2560
    assert oracle.compact_row_bytes(6, 8, 8) == 2  # 14 bits -> 2 bytes


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 16), (3, 8), (1, 4), (8, 8), (16, 16)])
def test_compact_roundtrip(n, m):
    """unpack(pack(c)) == c for random codes and for the oracle's own n:m packs."""
    rng = np.random.default_rng(n * 17 + m)
    c = _random_nm_codes(rng, 5, 20 * m, n, m)
    assert np.array_equal(oracle.compact_unpack(oracle.compact_pack(c, n, m), n, m, 20 * m), c)
    w = (rng.standard_normal((7, 40 * m)) * 0.02).astype(np.float32)
    p = oracle.pack_nm_ternary(w, n, m)
    data = oracle.compact_pack(p["codes"], n, m)
    assert np.array_equal(oracle.compact_unpack(data, n, m, 40 * m), p["codes"])
    # the nonzero mask bits count the nonzero codes
    bits = np.unpackbits(data, axis=1, bitorder="little")[:, : 40 * (m + n)].reshape(7, 40, m + n)
    assert np.array_equal(bits[:, :, :m].sum(axis=2),
                          (p["codes"].reshape(7, 40, m) != 0).sum(axis=2))


def test_compact_rejects_bad_streams():
    with pytest.raises(ValueError):
        oracle.compact_pack(np.array([[1, 1, 1, 0]], np.int8), 2, 4)  # 3 nonzeros in a 2:4 group
    with pytest.raises(ValueError):
        oracle.compact_unpack(np.array([[0x21]], np.uint8), 2, 4, 4)  # slot 1 set, 1 nonzero
    with pytest.raises(ValueError):
        oracle.compact_unpack(np.array([[0x00, 0x10]], np.uint8), 2, 4, 8)  # padding bit set


@pytest.mark.parametrize("mutant", ["polarity", "descending", "running_slots", "msb_mask"])
def test_compact_mutants_caught(mutant):
    def pack(codes, n, m):
        c = np.asarray(codes, np.int8)
        n_out, k = c.shape
        rows = []
        for row in c:
            bits = []
            run = []
            for g in range(k // m):
                grp = [int(v) for v in row[g * m:(g + 1) * m]]
                mask = [1 if v != 0 else 0 for v in grp]
                signs = [1 if v < 0 else 0 for v in grp if v != 0]
                if mutant == "polarity":
                    signs = [1 - s for s in signs]
                elif mutant == "descending":
                    signs = signs[::-1]
                elif mutant == "msb_mask":
                    mask = mask[::-1]
                if mutant == "running_slots":  # sign slots shared by the whole row, not per group
                    run += signs
                    bits += mask + [0] * n
                else:
                    bits += mask + signs + [0] * (n - len(signs))
            if mutant == "running_slots":
                for g in range(k // m):
                    for j in range(n):
                        idx = g * n + j
                        bits[g * (m + n) + m + j] = run[idx] if idx < len(run) else 0
            bits += [0] * (-len(bits) % 8)
            rows.append([sum(b << i for i, b in enumerate(bits[o:o + 8]))
                         for o in range(0, len(bits), 8)])
        return np.array(rows, np.uint8)

    assert _compact_pins_fail(pack)


# ---------------------------------------------------------------------------------------------
# Structured k:256 outliers (8:16 paper, "Key points"): the k largest |w| of each 256-group along
# K are kept apart as bf16; the ternary path sees the rest.
# ---------------------------------------------------------------------------------------------

def _outlier_hand_row():
    """One 256-wide row: magnitude 2 at 200, a four-way tie of magnitude 1 at 10, 20, 30, 40, a
    value 3 + 2^-7 (rounds to bf16 3.0) at 100 and small values elsewhere."""
    w = np.full((1, 256), 0.01, np.float32)
    w[0, 1::2] = -0.01
    w[0, 200] = -2.0
    w[0, [10, 20, 30, 40]] = [1.0, -1.0, 1.0, -1.0]
    w[0, 100] = 3.0 + 2.0 ** -7
    return w


def _outlier_pins_fail(select, pack) -> bool:
    w = _outlier_hand_row()
    pos, val, mask = select(w, 4)
    # k = 4: 100 (3.0078), 200 (2.0), then the tie of 1.0 broken toward the lower positions 10, 20
    if pos.tolist() != [[[10, 20, 100, 200]]]:
        return True
    if oracle.bf16_to_f32(val).tolist() != [[[1.0, -1.0, 3.0, -2.0]]]:
        return True
    if int(mask.sum()) != 4 or not mask[0, 100] or mask[0, 30]:
        return True
    r = pack(w, 2, 4, 4)
    rest = w.copy()
    rest[0, [10, 20, 100, 200]] = 0
    if r["gamma"] != np.float32(np.abs(rest.astype(np.float64)).sum() / 256):
        return True
    if np.any(r["codes"][0, [10, 20, 100, 200]] != 0):
        return True
    # the page's shares: k of every 256 weights (4:256 ~1.5%, 8:256 ~3.1%, 16:256 = 6.25%)
    rng = np.random.default_rng(5)
    w = rng.laplace(0, 0.02, (16, 1024)).astype(np.float32)
    for k, share in ((4, 0.015625), (8, 0.03125), (16, 0.0625)):
        pos, val, mask = select(w, k)
        if mask.mean() != share:
            return True
        g = np.abs(w).reshape(16, 4, 256)
        mk = mask.reshape(16, 4, 256)
        if np.any(np.where(mk, g, np.inf).min(axis=2) < np.where(mk, -np.inf, g).max(axis=2)):
            return True  # an outlier smaller than a weight left in the group
        if not np.array_equal(val, oracle.f32_to_bf16_rne(np.take_along_axis(
                w.reshape(16, 4, 256), pos.astype(np.int64), axis=2))):
            return True
    return False


def test_outlier_pins():
    assert not _outlier_pins_fail(oracle.outlier_select, oracle.pack_with_outliers)


@pytest.mark.parametrize("mutant", ["ties_high", "magnitude_order", "smallest", "fp32_values",
                                    "not_removed"])
def test_outlier_mutants_caught(mutant):
    def select(w, k):
        pos, val, mask = oracle.outlier_select(w, k)
        n_out, K = w.shape
        g = K // 256
        if mutant == "ties_high":
            mag = np.abs(w).reshape(n_out, g, 256)[:, :, ::-1]
            order = 255 - np.argsort(-mag, axis=2, kind="stable")[:, :, :k]
            pos = np.sort(order, axis=2).astype(np.uint8)
        elif mutant == "magnitude_order":
            mag = np.abs(w).reshape(n_out, g, 256)
            pos = np.argsort(-mag, axis=2, kind="stable")[:, :, :k].astype(np.uint8)
        elif mutant == "smallest":
            mag = np.abs(w).reshape(n_out, g, 256)
            pos = np.sort(np.argsort(mag, axis=2, kind="stable")[:, :, :k], axis=2).astype(np.uint8)
        vals = np.take_along_axis(w.reshape(n_out, g, 256), pos.astype(np.int64), axis=2)
        val = oracle.f32_to_bf16_rne(vals).astype(np.uint16)
        if mutant == "fp32_values":  # truncated instead of rounded
            val = (vals.view(np.uint32) >> 16).astype(np.uint16)
        mask = np.zeros((n_out, g, 256), bool)
        np.put_along_axis(mask, pos.astype(np.int64), True, axis=2)
        return pos, val, mask.reshape(n_out, K)

    def pack(w, n, m, k):
        if mutant == "not_removed":
            r = dict(oracle.pack_with_outliers(w, n, m, k))
            r["gamma"] = oracle.absmean_gamma(w)
            r["codes"] = oracle.ternary_codes(w, oracle.nm_keep_mask(w, n, m), r["gamma"])
            return r
        return oracle.pack_with_outliers(w, n, m, k)

    assert _outlier_pins_fail(select, pack)


def test_outlier_forward_against_dense_product():
    """The two-term forward equals x_q (gamma C + O)^T a'/127 formed as one dense fp64 matrix, and
    a pure-Python loop on a tiny case."""
    rng = np.random.default_rng(8)
    w = rng.laplace(0, 0.02, (9, 512)).astype(np.float32)
    x = oracle.f32_to_bf16_rne(rng.standard_normal((3, 512)).astype(np.float32))
    q, a = oracle.quantize_act(x)
    r = oracle.pack_with_outliers(w, 6, 8, 8)
    f = oracle.forward_with_outliers(q, a, r["codes"], r["gamma"], r["opos"], r["oval"])
    W_eff = np.float64(r["gamma"]) * r["codes"].astype(np.float64) + oracle.outlier_matrix(
        r["opos"], r["oval"], 512)
    y_dense = (q.astype(np.float64) @ W_eff.T) * (a.astype(np.float64)[:, None] / 127.0)
    assert np.allclose(f["y"], y_dense, rtol=1e-12, atol=0)
    # brute force, row 0 / token 0
    t, rr = 0, 0
    s = 0.0
    for kk in range(512):
        s += float(q[t, kk]) * float(r["gamma"]) * float(r["codes"][rr, kk])
    for gi in range(2):
        for j in range(8):
            p = gi * 256 + int(r["opos"][rr, gi, j])
            s += float(q[t, p]) * float(oracle.bf16_to_f32(r["oval"][rr, gi, j]))
    assert math.isclose(f["y"][t, rr], s * float(a[t]) / 127.0, rel_tol=1e-12)


# ------------------------------------------------------------------------------------------------
# Combinatorial mask rank (the pages' metadata sizes: 0.75 bits/element for 2:4, 0.875 for 8:16)
# ------------------------------------------------------------------------------------------------

# The six 2-of-4 choices in colexicographic order (by largest position, then the next), written out
# by hand: their ranks are 0 .. 5.
RANK_2OF4 = [((0, 1), 0), ((0, 2), 1), ((1, 2), 2), ((0, 3), 3), ((1, 3), 4), ((2, 3), 5)]
RANK_PATTERNS = [(2, 4), (1, 4), (3, 4), (4, 4), (6, 8), (3, 8), (4, 8), (8, 8), (8, 16), (5, 16),
                 (12, 16), (16, 16)]


def test_rank_bits_match_the_printed_metadata_sizes():
    """ceil(log2 C(m, n)) / m reproduces the printed 0.75 (2:4) and 0.875 (8:16) bits per element;
    with the 2-bit kept codes a group costs 1.75 and 1.875 bits per weight; a dense group needs no
    rank."""
    assert oracle.rank_bits(2, 4) / 4 == 0.75 and oracle.rank_bits(8, 16) / 16 == 0.875
    assert oracle.rank_bits(2, 4) / 4 == oracle.combinatorial_metadata_bits(2, 4)
    assert (oracle.rank_bits(2, 4) + 4) / 4 == 1.75 and (oracle.rank_bits(8, 16) + 16) / 16 == 1.875
    for m in (4, 8, 16):
        assert oracle.rank_bits(m, m) == 0
    assert oracle.rank_row_bytes(8, 16, 32) == 8 and oracle.rank_row_bytes(2, 4, 8) == 2


def _rank_pins_fail(rank, unrank) -> bool:
    try:
        for subset, r in RANK_2OF4:
            if rank(list(subset)) != r or list(unrank(r, 2, 4)) != list(subset):
                return True
        for n, m in RANK_PATTERNS:
            subsets = sorted(itertools.combinations(range(m), n), key=lambda c: c[::-1])  # colex
            for r, c in enumerate(subsets):
                if rank(list(c)) != r or list(unrank(r, n, m)) != list(c):
                    return True
    except (ValueError, IndexError):
        return True
    return False


def test_rank_is_the_colex_bijection():
    """Every n-of-m subset (up to 12870 for 8:16) gets its index in the colex-sorted list of all
    subsets, and unrank inverts it."""
    assert not _rank_pins_fail(oracle.mask_rank, oracle.mask_unrank)


def _rank_brute(codes, keep, n, m):
    """The rank stream built another way: each group's index in the colex-sorted subset list, then
    its kept codes' low two bits, accumulated into one integer per row."""
    n_out, k = codes.shape
    R = (math.comb(m, n) - 1).bit_length()
    subsets = {c: i for i, c in enumerate(sorted(itertools.combinations(range(m), n),
                                                 key=lambda c: c[::-1]))}
    nbytes = ((k // m) * (R + 2 * n) + 7) // 8
    out = np.zeros((n_out, nbytes), dtype=np.uint8)
    for row in range(n_out):
        acc, shift = 0, 0
        for g in range(k // m):
            sel = tuple(int(i) for i in np.flatnonzero(keep[row, g * m:(g + 1) * m]))
            acc |= subsets[sel] << shift
            shift += R
            for p in sel:
                acc |= (int(codes[row, g * m + p]) & 3) << shift
                shift += 2
        out[row] = np.frombuffer(acc.to_bytes(nbytes, "little"), dtype=np.uint8)
    return out


def _rank_pack_pins_fail(pack) -> bool:
    rng = np.random.default_rng(5)
    for n, m in RANK_PATTERNS:
        for k in (m, 3 * m, 64 + m):
            w = rng.standard_normal((5, k)).astype(np.float32)
            ref = oracle.pack_nm_ternary(w, n, m)
            got = pack(ref["codes"], ref["keep"], n, m)
            if got.shape != (5, oracle.rank_row_bytes(n, m, k)):
                return True
            if not np.array_equal(got, _rank_brute(ref["codes"], ref["keep"], n, m)):
                return True
    return False


def test_rank_pack_against_brute_force_and_roundtrip():
    assert not _rank_pack_pins_fail(oracle.rank_pack)
    rng = np.random.default_rng(6)
    for n, m in RANK_PATTERNS:
        w = rng.standard_normal((7, 4 * m + 64)).astype(np.float32)
        ref = oracle.pack_nm_ternary(w, n, m)
        data = oracle.rank_pack(ref["codes"], ref["keep"], n, m)
        codes, keep = oracle.rank_unpack(data, n, m, w.shape[1])
        assert np.array_equal(codes, ref["codes"]) and np.array_equal(keep, ref["keep"])


def test_rank_pins_catch_mutants():
    """Lexicographic ranks, MSB-first rank bits and codes written before the rank all fail."""
    def lex_rank(pos):
        m = 16 if max(pos) >= 8 else (8 if max(pos) >= 4 else 4)
        return list(itertools.combinations(range(m), len(pos))).index(tuple(pos))

    assert _rank_pins_fail(lex_rank, oracle.mask_unrank)

    def msb_first(codes, keep, n, m):
        R = oracle.rank_bits(n, m)
        data = oracle.rank_pack(codes, keep, n, m)
        bits = np.unpackbits(data, axis=1, bitorder="little")
        per = R + 2 * n
        for g in range(codes.shape[1] // m):
            bits[:, g * per:g * per + R] = bits[:, g * per:g * per + R][:, ::-1]
        return np.packbits(bits, axis=1, bitorder="little")

    def codes_first(codes, keep, n, m):
        R = oracle.rank_bits(n, m)
        data = oracle.rank_pack(codes, keep, n, m)
        bits = np.unpackbits(data, axis=1, bitorder="little")
        per = R + 2 * n
        for g in range(codes.shape[1] // m):
            seg = bits[:, g * per:(g + 1) * per].copy()
            bits[:, g * per:(g + 1) * per] = np.concatenate([seg[:, R:], seg[:, :R]], axis=1)
        return np.packbits(bits, axis=1, bitorder="little")

    assert _rank_pack_pins_fail(msb_first)
    assert _rank_pack_pins_fail(codes_first)
