"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments on the host
before any HIP call (no GPU needed: validation never reaches the runtime)."""

import ctypes
import subprocess

import pytest

from sparsity_sbn_quantize_amd import binding as b

ERR_INVALID, ERR_UNSUPPORTED, ERR_SHAPE = -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    return b.lib()


def test_exports_match_header(lib):
    declared = b.header_symbols()
    assert set(declared) == {"sbn_quantize_act", "sbn_layernorm_quantize_act",
                             "sbn_pack_nm_ternary", "sbn_pack_nm_ternary_ex", "sbn_bitlinear_fwd",
                             "sbn_bitlinear_fwd_bf16", "sbn_bitlinear_fwd_ln_bf16",
                             "sbn_bitlinear_bwd_dx", "sbn_free",
                             "sbn_packed_export", "sbn_packed_export_rpf", "sbn_packed_export_compact",
                             "sbn_packed_export_rank",
                             "sbn_packed_export_outliers",
                             "sbn_packed_query",
                             "sbn_packed_mask_flips", "sbn_last_error",
                             "sbn_bitlinear_fwd_group", "sbn_bitlinear_fwd_group_bf16",
                             "sbn_bitlinear_fwd_latent_static",
                             "sbn_ceiling_stream_read", "sbn_ceiling_mfma_i8", "sbn_ceiling_smfmac_i8",
                             "sbn_ceiling_empty"}
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, name
        assert getattr(lib, name) is not None


def _h():
    return ctypes.c_void_p(0)


@pytest.mark.parametrize("args,code", [
    ((None, -1, 8, 8, None, 8, None, None), ERR_INVALID),        # T < 0
    ((None, 4, 0, 8, None, 8, None, None), ERR_INVALID),         # K = 0
    ((None, 4, 1 << 18, 1 << 18, None, 1 << 18, None, None), ERR_INVALID),  # K > max
    ((None, 4, 16, 8, None, 16, None, None), ERR_INVALID),       # ld_x < K
    ((None, 4, 16, 16, None, 15, None, None), ERR_INVALID),      # ld_q < K
    ((None, 4, 16, 16, None, 16, None, None), ERR_INVALID),      # null pointers
])
def test_quantize_validation(lib, args, code):
    assert lib.sbn_quantize_act(*args) == code
    assert b.last_error()


def test_quantize_T0_is_noop(lib):
    assert lib.sbn_quantize_act(None, 0, 16, 16, None, 16, None, None) == 0


@pytest.mark.parametrize("n_out,K,ld,n,m,code", [
    (16, 64, 64, 2, 6, ERR_UNSUPPORTED),    # m not in {4, 8, 16}
    (16, 64, 64, 0, 4, ERR_UNSUPPORTED),    # n < 1
    (16, 64, 64, 5, 4, ERR_UNSUPPORTED),    # n > m
    (16, 60, 60, 6, 8, ERR_INVALID),        # K % m
    (16, 8, 8, 8, 16, ERR_INVALID),         # K < m
    (-1, 64, 64, 2, 4, ERR_INVALID),        # n_out < 0
    (16, 64, 32, 2, 4, ERR_INVALID),        # ld_w < K
    (16, 64, 64, 2, 4, ERR_INVALID),        # w null
])
def test_pack_validation(lib, n_out, K, ld, n, m, code):
    h = _h()
    assert lib.sbn_pack_nm_ternary(None, n_out, K, ld, n, m, ctypes.byref(h), None) == code
    assert not h.value
    assert b.last_error()


def test_pack_null_handle_pointer(lib):
    assert lib.sbn_pack_nm_ternary(None, 16, 64, 64, 2, 4, None, None) == ERR_INVALID


def test_forward_and_misc_validation(lib):
    assert lib.sbn_bitlinear_fwd(None, None, 0, None, 1, None, 0, 0, None) == ERR_INVALID
    assert lib.sbn_bitlinear_fwd_bf16(None, None, 0, 1, None, 0, None, None, 0, 0,
                                      None) == ERR_INVALID
    assert lib.sbn_packed_export(None, None, None, None, None) == ERR_INVALID
    assert lib.sbn_packed_export_rpf(None, None, None, None) == ERR_INVALID
    assert lib.sbn_packed_query(None, None) == ERR_INVALID
    assert lib.sbn_packed_mask_flips(None, None, None) == ERR_INVALID
    assert lib.sbn_packed_export_compact(None, None, None) == ERR_INVALID
    assert lib.sbn_packed_export_rank(None, None, None) == ERR_INVALID
    assert lib.sbn_packed_export_outliers(None, None, None, None) == ERR_INVALID
    h = ctypes.c_void_p(0)
    for k in (1, 3, 5, 32):  # outliers per 256 must be 4, 8 or 16
        assert lib.sbn_pack_nm_ternary_ex(None, 16, 512, 512, 2, 4, k << 8, ctypes.byref(h),
                                          None) == ERR_INVALID
    assert lib.sbn_pack_nm_ternary_ex(None, 16, 320, 320, 2, 4, 4 << 8, ctypes.byref(h),
                                      None) == -2  # K % 256 != 0
    for flags in (4, -1, 1 << 30):  # unknown flag bits are rejected before any device work
        assert lib.sbn_pack_nm_ternary_ex(None, 16, 64, 64, 2, 4, flags, ctypes.byref(h),
                                          None) == ERR_INVALID
    assert lib.sbn_pack_nm_ternary_ex(None, 16, 64, 64, 2, 4, 1, None, None) == ERR_INVALID
    assert lib.sbn_bitlinear_bwd_dx(None, None, 0, 1, None, 0, None) == ERR_INVALID
    assert lib.sbn_layernorm_quantize_act(None, 1, 8, 8, 1e-5, None, 8, None, None) == ERR_INVALID
    assert lib.sbn_layernorm_quantize_act(None, 1, 8, 8, 0.0, None, 8, None, None) == ERR_INVALID
    assert lib.sbn_layernorm_quantize_act(None, 0, 8, 8, 1e-5, None, 8, None, None) == 0
    assert lib.sbn_bitlinear_fwd_ln_bf16(None, None, 0, 1, 1e-5, None, 0, None, None, 0, 0,
                                         None) == ERR_INVALID
    assert lib.sbn_bitlinear_fwd_ln_bf16(None, None, 0, 1, 0.0, None, 0, None, None, 0, 0,
                                         None) == ERR_INVALID
    lib.sbn_free(None)  # no-op
    one = (ctypes.c_void_p * 1)(None)
    ld1 = (ctypes.c_int64 * 1)(16)
    assert lib.sbn_bitlinear_fwd_group(None, 1, None, 16, None, 1, one, ld1, 0, None) == ERR_INVALID
    assert lib.sbn_bitlinear_fwd_group(one, 1, None, 16, None, 1, one, ld1, 0, None) == ERR_INVALID
    assert lib.sbn_bitlinear_fwd_group(one, 0, None, 16, None, 1, one, ld1, 0, None) == ERR_INVALID
    assert lib.sbn_bitlinear_fwd_group(one, 9, None, 16, None, 1, one, ld1, 0, None) == ERR_INVALID
    assert lib.sbn_bitlinear_fwd_group_bf16(one, 1, None, 16, 1, 0.0, None, 16, None, one, ld1, 0,
                                            None) == ERR_INVALID
    assert lib.sbn_bitlinear_fwd_group_bf16(None, 1, None, 16, 1, 0.0, None, 16, None, one, ld1,
                                            0, None) == ERR_INVALID
    sink = ctypes.c_void_p(16)
    ops = ctypes.c_double(0)
    assert lib.sbn_ceiling_stream_read(None, 1024, 1, sink, None) == ERR_INVALID
    assert lib.sbn_ceiling_stream_read(ctypes.c_void_p(64), 1000, 1, sink, None) == ERR_INVALID
    assert lib.sbn_ceiling_stream_read(ctypes.c_void_p(8), 1024, 1, sink, None) == ERR_INVALID
    assert lib.sbn_ceiling_mfma_i8(0, 1024, sink, ctypes.byref(ops), None) == ERR_INVALID
    assert lib.sbn_ceiling_mfma_i8(100, 6, sink, ctypes.byref(ops), None) == ERR_INVALID
    assert lib.sbn_ceiling_mfma_i8(100, 1024, sink, None, None) == ERR_INVALID
    assert lib.sbn_ceiling_smfmac_i8(0, 1024, sink, ctypes.byref(ops), None) == ERR_INVALID
    assert lib.sbn_ceiling_smfmac_i8(100, 6, sink, ctypes.byref(ops), None) == ERR_INVALID
    assert lib.sbn_ceiling_smfmac_i8(100, 1024, None, ctypes.byref(ops), None) == ERR_INVALID


def test_error_message_is_per_call(lib):
    lib.sbn_quantize_act(None, 4, 0, 8, None, 8, None, None)
    assert "K=0" in b.last_error()
    lib.sbn_bitlinear_fwd(None, None, 0, None, 1, None, 0, 0, None)
    assert "handle" in b.last_error()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        b.lib()
