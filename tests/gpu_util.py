"""Helpers of the GPU parity tests: run the HIP path through the binding and compare it with the
oracle stage by stage."""

from __future__ import annotations

import numpy as np

import oracle
from sparsity_sbn_quantize_amd import binding

REL_TOL_Y = 1e-5          # fp32 output tolerance (relative)
BOUNDARY_FRACTION = 1e-6  # allowed share of boundary mismatches in integer codes


def to_dev_bf16(x_bits: np.ndarray, ld: int | None = None):
    import torch
    T, K = x_bits.shape
    ld = K if ld is None else ld
    buf = np.full((T, ld), 0x7FC0, np.uint16)  # NaN canaries beyond K
    buf[:, :K] = x_bits
    t = torch.from_numpy(buf.view(np.int16)).cuda()
    return t[:, :K].view(torch.bfloat16)


def to_dev_f32(w: np.ndarray, ld: int | None = None):
    import torch
    n, K = w.shape
    ld = K if ld is None else ld
    buf = np.full((n, ld), np.nan if ld > K else 0, np.float32)
    buf[:, :K] = w
    return torch.from_numpy(buf).cuda()[:, :K]


def gpu_forward(x_bits, w, n, m, ld_x=None, ld_w=None, ld_q=None, outs=("f32", "i32"),
                bf16_step=False):
    """Runs quantize -> pack -> forward on the GPU; returns host arrays of every stage. With
    bf16_step, the quantize-and-multiply entry (sbn_bitlinear_fwd_bf16) also runs on the same
    packed weights, and its outputs are returned under "bf16_*"."""
    import torch
    T, K = x_bits.shape
    xd = to_dev_bf16(x_bits, ld_x)
    wd = to_dev_f32(w, ld_w)
    ldq = K if ld_q is None else ld_q
    qbuf = torch.full((max(T, 1), ldq), 77, dtype=torch.int8, device="cuda")[:T]
    q = qbuf[:, :K]
    a = torch.empty((T,), dtype=torch.float32, device="cuda")
    binding.quantize_act(xd, out_q=q, out_absmax=a)
    pw = binding.PackedWeight(wd, n, m)
    res = {}
    for kind in outs:
        res[kind] = binding.bitlinear(q, a, pw, out=kind)
    if bf16_step:
        for kind in outs:
            yb, qb, ab = binding.bitlinear_bf16(xd, pw, out=kind)
            res["bf16_" + kind] = yb
        res["bf16_q"], res["bf16_a"] = qb, ab
    codes, keep, gamma = pw.export()
    cb, mb = pw.export_rpf()
    torch.cuda.synchronize()
    out = dict(q=q.cpu().numpy(), q_pad=qbuf.cpu().numpy(), a_prime=a.cpu().numpy(),
               codes=codes.cpu().numpy(), keep=keep.cpu().numpy().astype(bool),
               gamma=np.float32(gamma.cpu().numpy()[0]), code_bytes=cb.cpu().numpy(),
               mask_bytes=mb.cpu().numpy(), desc=pw.query())
    if "f32" in res:
        out["y"] = res["f32"].cpu().numpy()
    if "i32" in res:
        out["acc"] = res["i32"].cpu().numpy()
    for k, v in res.items():
        if k.startswith("bf16_"):
            out[k] = v.cpu().numpy()
    pw.free()
    return out


def assert_int_exact_except_boundary(got, ref, boundary, what):
    bad = got != ref
    nbad = int(bad.sum())
    if nbad == 0:
        return 0
    assert np.all(boundary[bad]), f"{what}: {nbad} mismatches, some not at a rounding boundary"
    assert nbad <= BOUNDARY_FRACTION * got.size, f"{what}: {nbad} boundary mismatches"
    return nbad


def assert_y_close(y, y_ref, what="y"):
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    err = np.abs(y - y_ref)
    ok = err <= REL_TOL_Y * np.abs(y_ref)
    assert np.all(ok), (f"{what}: {int((~ok).sum())} elements beyond {REL_TOL_Y} relative; "
                        f"max err {err.max()}")


def gamma_matches(got, w) -> bool:
    """gamma must be bit-equal, except that one ulp is allowed when the fp64 mean lies within
    1e-9 (relative) of an fp32 rounding midpoint (summation order can then decide the rounding)."""
    ref = oracle.absmean_gamma(w)
    if got == ref:
        return True
    mean = float(np.sum(np.abs(np.asarray(w, np.float64)))) / max(w.size, 1)
    lo, hi = sorted([float(ref), float(got)])
    if np.nextafter(np.float32(lo), np.float32(np.inf)) != np.float32(hi):
        return False
    mid = (lo + hi) / 2.0
    return abs(mean - mid) <= 1e-9 * abs(mean)


def check_stages(g, x_bits, w, n, m, acc_tokens=None, acc_rows=None, p=None):
    """Compares every stage of a GPU run `g` with the oracle. The int32 accumulators and fp32
    outputs are compared in full, or, when samples are given, on the sampled tokens (all rows)
    and the sampled rows (all tokens). `p` may carry the oracle's pack of (w, n, m) computed
    before. Outputs of the quantize-and-multiply entry (gpu_forward's bf16_step) must equal the
    two-call path's bit for bit."""
    if "bf16_q" in g:
        assert np.array_equal(g["bf16_q"], g["q"]), "bf16 entry: x_q differs from the quantizer"
        assert np.array_equal(g["bf16_a"], g["a_prime"]), "bf16 entry: a' differs"
        if "acc" in g:
            assert np.array_equal(g["bf16_i32"], g["acc"]), "bf16 entry: int32 accumulators differ"
        if "y" in g:
            assert np.array_equal(g["bf16_f32"], g["y"]), "bf16 entry: fp32 output differs"
    q_ref, a_ref = oracle.quantize_act(x_bits)
    assert np.array_equal(g["a_prime"], a_ref), "absmax"
    assert_int_exact_except_boundary(g["q"], q_ref, oracle.boundary_elements_act(x_bits, a_ref),
                                     "int8 activations")
    if p is None:
        p = oracle.pack_nm_ternary(w, n, m)
    assert gamma_matches(g["gamma"], w), (g["gamma"], p["gamma"])
    assert np.array_equal(g["keep"], p["keep"]), "keep mask"
    assert_int_exact_except_boundary(g["codes"], p["codes"],
                                     oracle.boundary_elements_weight(w, p["gamma"]), "codes")
    if np.array_equal(g["codes"], p["codes"]):
        assert np.array_equal(g["code_bytes"], p["code_bytes"]), "packed code bytes"
        assert np.array_equal(g["mask_bytes"], p["mask_bytes"]), "packed mask bytes"
    d = g["desc"]
    assert d.code_row_bytes == p["code_bytes"].shape[1]
    assert d.mask_row_bytes == p["mask_bytes"].shape[1]
    # Matmul on identical inputs (the GPU's own q and codes): exact, no exceptions.
    if acc_tokens is None and acc_rows is None:
        views = [(slice(None), slice(None))]
    else:
        views = []
        if acc_tokens is not None:
            views.append((acc_tokens, slice(None)))
        if acc_rows is not None:
            views.append((slice(None), acc_rows))
    for toks, rows in views:
        acc_ref = oracle.int_matmul(g["q"][toks], g["codes"][rows])
        if "acc" in g:
            assert np.array_equal(g["acc"][toks][:, rows], acc_ref), "int32 accumulators"
        if "y" in g:
            y_ref = oracle.dequantize(acc_ref, g["gamma"], g["a_prime"][toks])
            assert_y_close(g["y"][toks][:, rows], y_ref)
    return p
