"""Thin Python binding of libsbn (ctypes): argument marshalling only.

Every step of the forward runs in the HIP kernels behind the C ABI declared in include/sbn.h;
PyTorch supplies device memory and the current stream. There is no CPU fallback: if the built
library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
# SBN_LIB names another build of the library to load (the host-sanitizer build, for instance)
LIB_PATH = os.environ.get("SBN_LIB") or os.path.join(HERE, "libsbn.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HEADERS = [os.path.join(INCLUDE, h) for h in ("sbn.h", "sbn_ceilings.h")]

SBN_OUT_F32 = 0
SBN_OUT_I32_ACC = 1
SBN_PACK_VARIANCE_CORRECTION = 1
SBN_PACK_COMPACT = 2
STATUS = {0: "SBN_OK", -1: "SBN_ERR_INVALID_ARG", -2: "SBN_ERR_UNSUPPORTED", -3: "SBN_ERR_SHAPE",
          -4: "SBN_ERR_HIP", -5: "SBN_ERR_OOM"}


class SbnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class PackedDesc(ctypes.Structure):
    _fields_ = [("n_out", ctypes.c_int64), ("K", ctypes.c_int64), ("n", ctypes.c_int),
                ("m", ctypes.c_int), ("code_row_bytes", ctypes.c_size_t),
                ("mask_row_bytes", ctypes.c_size_t), ("rpf_bytes", ctypes.c_size_t),
                ("packed_bytes", ctypes.c_size_t), ("device_bytes", ctypes.c_size_t),
                ("compact_row_bytes", ctypes.c_size_t), ("compact_bytes", ctypes.c_size_t),
                ("compact", ctypes.c_int), ("outlier_k", ctypes.c_int),
                ("rank_row_bytes", ctypes.c_size_t), ("splitk_giveups", ctypes.c_uint32),
                ("single_pass", ctypes.c_int)]


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGNATURES = {
    "sbn_quantize_act": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P, _P]),
    "sbn_layernorm_quantize_act": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.c_float, _P,
                                                  _I64, _P, _P]),
    "sbn_pack_nm_ternary": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.c_int, ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_void_p), _P]),
    "sbn_pack_nm_ternary_ex": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), _P]),
    "sbn_bitlinear_fwd": (ctypes.c_int, [_P, _P, _I64, _P, _I64, _P, _I64, ctypes.c_int, _P]),
    "sbn_bitlinear_fwd_bf16": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, _P, _P, _I64,
                                              ctypes.c_int, _P]),
    "sbn_free": (None, [_P]),
    "sbn_packed_export": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "sbn_packed_export_rpf": (ctypes.c_int, [_P, _P, _P, _P]),
    "sbn_packed_export_compact": (ctypes.c_int, [_P, _P, _P]),
    "sbn_packed_export_rank": (ctypes.c_int, [_P, _P, _P]),
    "sbn_packed_export_outliers": (ctypes.c_int, [_P, _P, _P, _P]),
    "sbn_packed_query": (ctypes.c_int, [_P, ctypes.POINTER(PackedDesc)]),
    "sbn_packed_mask_flips": (ctypes.c_int, [_P, _P, _P]),
    "sbn_bitlinear_bwd_dx": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, _P]),
    "sbn_bitlinear_fwd_ln_bf16": (ctypes.c_int, [_P, _P, _I64, _I64, ctypes.c_float, _P, _I64,
                                                 _P, _P, _I64, ctypes.c_int, _P]),
    "sbn_last_error": (ctypes.c_char_p, []),
    "sbn_bitlinear_fwd_group": (ctypes.c_int, [_P, ctypes.c_int, _P, _I64, _P, _I64, _P, _P,
                                               ctypes.c_int, _P]),
    "sbn_bitlinear_fwd_group_bf16": (ctypes.c_int, [_P, ctypes.c_int, _P, _I64, _I64,
                                                    ctypes.c_float, _P, _I64, _P, _P, _P,
                                                    ctypes.c_int, _P]),
    "sbn_bitlinear_fwd_latent_static": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.c_int,
                                                       ctypes.c_int, _P, _I64, _P, _I64, _P, _I64,
                                                       ctypes.c_int, _P]),
    "sbn_ceiling_stream_read": (ctypes.c_int, [_P, ctypes.c_size_t, ctypes.c_uint32, _P, _P]),
    "sbn_ceiling_mfma_i8": (ctypes.c_int, [_I64, _I64, _P, ctypes.POINTER(ctypes.c_double), _P]),
    "sbn_ceiling_smfmac_i8": (ctypes.c_int, [_I64, _I64, _P, ctypes.POINTER(ctypes.c_double),
                                             _P]),
    "sbn_ceiling_empty": (ctypes.c_int, [_P]),
}


def header_symbols() -> list:
    """Function names declared in the headers under include/."""
    names = set()
    for path in HEADERS:
        with open(path) as f:
            text = f.read()
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(sbn_\w+)\s*\(", text, re.M))
    return sorted(names)


def lib() -> ctypes.CDLL:
    """Loads libsbn.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is None:
        # torch first: the process then holds torch's HIP runtime, which libsbn.so binds to (a
        # library loaded before torch would bring in another copy of the runtime)
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def last_error() -> str:
    return (lib().sbn_last_error() or b"").decode()


def check(status: int) -> None:
    if status != 0:
        raise SbnError(status, last_error())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require_cuda(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 2 or (t.numel() > 0 and t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")


def _ld(t, width: int) -> int:
    """Leading dimension of a 2-D tensor; for a single row (or none) torch may report any stride."""
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), width)


def quantize_act(x, out_q=None, out_absmax=None, stream=None):
    """x: bf16 (or int16 bit patterns) [T][K] on the device -> (q int8 [T][K], a' fp32 [T])."""
    import torch
    _require_cuda(x, "x")
    if x.dtype not in (torch.bfloat16, torch.int16):
        raise ValueError("x must be bfloat16 (or int16 bf16 bit patterns)")
    T, K = x.shape
    q = out_q if out_q is not None else torch.empty((T, K), dtype=torch.int8, device=x.device)
    a = out_absmax if out_absmax is not None else torch.empty((T,), dtype=torch.float32,
                                                              device=x.device)
    check(lib().sbn_quantize_act(_ptr(x), T, K, _ld(x, K), _ptr(q), _ld(q, K), _ptr(a),
                                 _stream(stream)))
    return q, a


def layernorm_quantize_act(x, eps: float = 1e-5, out_q=None, out_absmax=None, stream=None):
    """Parameter-free LayerNorm, then per-token absmax INT8: x bf16 [T][K] -> (q, a')."""
    import torch
    _require_cuda(x, "x")
    if x.dtype not in (torch.bfloat16, torch.int16):
        raise ValueError("x must be bfloat16 (or int16 bf16 bit patterns)")
    T, K = x.shape
    q = out_q if out_q is not None else torch.empty((T, K), dtype=torch.int8, device=x.device)
    a = out_absmax if out_absmax is not None else torch.empty((T,), dtype=torch.float32,
                                                              device=x.device)
    check(lib().sbn_layernorm_quantize_act(_ptr(x), T, K, _ld(x, K), float(eps), _ptr(q),
                                           _ld(q, K), _ptr(a), _stream(stream)))
    return q, a

class PackedWeight:
    """A packed n:m ternary weight (library-owned device memory)."""

    def __init__(self, w, n: int, m: int, stream=None, variance_correction: bool = False,
                 compact: bool = False, outliers: int = 0):
        self._h = ctypes.c_void_p(0)
        self.n, self.m = n, m
        self.variance_correction = variance_correction
        self.compact = compact
        self.outliers = outliers
        self.pack(w, stream)

    def pack(self, w, stream=None, variance_correction=None, compact=None, outliers=None):
        """(Re-)packs from fp32 latent weights [n_out][K]; re-packing reuses the handle. With
        variance_correction, the matmuls use the variance-corrected scale; with compact, the pack
        also writes the compact form that the GEMV launches read; with outliers = k (4, 8, 16),
        the k largest |w| of every 256 along K are kept apart (sbn_pack_nm_ternary_ex)."""
        if variance_correction is not None:
            self.variance_correction = variance_correction
        if compact is not None:
            self.compact = compact
        if outliers is not None:
            self.outliers = outliers
        import torch
        _require_cuda(w, "w")
        if w.dtype != torch.float32:
            raise ValueError("w must be float32")
        n_out, K = w.shape
        flags = ((SBN_PACK_VARIANCE_CORRECTION if self.variance_correction else 0) |
                 (SBN_PACK_COMPACT if self.compact else 0) | (int(self.outliers) << 8))
        check(lib().sbn_pack_nm_ternary_ex(_ptr(w), n_out, K, _ld(w, K), self.n, self.m, flags,
                                           ctypes.byref(self._h), _stream(stream)))
        self.n_out, self.K = n_out, K
        return self

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise ValueError("handle was freed")
        return self._h

    def query(self) -> PackedDesc:
        d = PackedDesc()
        check(lib().sbn_packed_query(self.handle, ctypes.byref(d)))
        return d

    def export(self, stream=None):
        """(codes int8 [n_out][K], keep uint8 [n_out][K], gamma fp32 [1]) on the device."""
        import torch
        dev = torch.device("cuda", torch.cuda.current_device())
        codes = torch.empty((self.n_out, self.K), dtype=torch.int8, device=dev)
        keep = torch.empty((self.n_out, self.K), dtype=torch.uint8, device=dev)
        gamma = torch.empty((1,), dtype=torch.float32, device=dev)
        check(lib().sbn_packed_export(self.handle, _ptr(codes), _ptr(keep), _ptr(gamma),
                                      _stream(stream)))
        return codes, keep, gamma

    def export_rpf(self, stream=None):
        """(code_bytes uint8 [n_out][cb], mask_bytes uint8 [n_out][mb]) on the device."""
        import torch
        d = self.query()
        dev = torch.device("cuda", torch.cuda.current_device())
        cb = torch.zeros((self.n_out, d.code_row_bytes), dtype=torch.uint8, device=dev)
        mb = torch.zeros((self.n_out, d.mask_row_bytes), dtype=torch.uint8, device=dev)
        check(lib().sbn_packed_export_rpf(self.handle, _ptr(cb),
                                          _ptr(mb) if d.mask_row_bytes else ctypes.c_void_p(0),
                                          _stream(stream)))
        return cb, mb

    def export_compact(self, stream=None):
        """The compact form's per-row bit streams (uint8 [n_out][compact_row_bytes], device)."""
        import torch
        d = self.query()
        dev = torch.device("cuda", torch.cuda.current_device())
        out = torch.zeros((self.n_out, d.compact_row_bytes), dtype=torch.uint8, device=dev)
        check(lib().sbn_packed_export_compact(self.handle, _ptr(out), _stream(stream)))
        return out

    def export_rank(self, stream=None):
        """The codes in the rank encoding (uint8 [n_out][rank_row_bytes], device)."""
        import torch
        d = self.query()
        dev = torch.device("cuda", torch.cuda.current_device())
        out = torch.full((self.n_out, d.rank_row_bytes), 0xA5, dtype=torch.uint8, device=dev)
        check(lib().sbn_packed_export_rank(self.handle, _ptr(out), _stream(stream)))
        return out

    def export_outliers(self, stream=None):
        """(positions uint8 [n_out][K/256][k], bf16 values as int16 [n_out][K/256][k]), device."""
        import torch
        k = self.query().outlier_k
        dev = torch.device("cuda", torch.cuda.current_device())
        pos = torch.zeros((self.n_out, self.K // 256, k), dtype=torch.uint8, device=dev)
        val = torch.zeros((self.n_out, self.K // 256, k), dtype=torch.int16, device=dev)
        check(lib().sbn_packed_export_outliers(self.handle, _ptr(pos), _ptr(val), _stream(stream)))
        return pos, val

    def mask_flips(self, stream=None):
        """Keep bits changed by the last pack (int64 tensor [1] on the device)."""
        import torch
        dev = torch.device("cuda", torch.cuda.current_device())
        out = torch.zeros((1,), dtype=torch.int64, device=dev)
        check(lib().sbn_packed_mask_flips(self.handle, _ptr(out), _stream(stream)))
        return out

    def free(self):
        if self._h:
            lib().sbn_free(self._h)
            self._h = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def bitlinear(x_q, x_absmax, w: PackedWeight, out: str = "f32", y=None, stream=None):
    """y [T][n_out] = dequant(x_q @ codes^T); out="i32" returns the raw int32 accumulators."""
    import torch
    _require_cuda(x_q, "x_q")
    T = x_q.shape[0]
    kind = SBN_OUT_F32 if out == "f32" else SBN_OUT_I32_ACC
    if y is None:
        y = torch.empty((T, w.n_out), dtype=torch.float32 if kind == SBN_OUT_F32 else torch.int32,
                        device=x_q.device)
    check(lib().sbn_bitlinear_fwd(w.handle, _ptr(x_q), _ld(x_q, w.K), _ptr(x_absmax), T,
                                  _ptr(y), _ld(y, w.n_out), kind, _stream(stream)))
    return y


def bitlinear_bf16(x, w: PackedWeight, out: str = "f32", y=None, x_q=None, x_absmax=None,
                   stream=None, ln_eps=None):
    """Quantize-and-multiply: x bf16 [T][K] -> (y, x_q int8 [T][K], a' fp32 [T]). With ln_eps,
    the parameter-free LayerNorm runs first (sbn_bitlinear_fwd_ln_bf16)."""
    import torch
    _require_cuda(x, "x")
    if x.dtype not in (torch.bfloat16, torch.int16):
        raise ValueError("x must be bfloat16 (or int16 bf16 bit patterns)")
    T = x.shape[0]
    kind = SBN_OUT_F32 if out == "f32" else SBN_OUT_I32_ACC
    if y is None:
        y = torch.empty((T, w.n_out), dtype=torch.float32 if kind == SBN_OUT_F32 else torch.int32,
                        device=x.device)
    if x_q is None:
        x_q = torch.empty((T, w.K), dtype=torch.int8, device=x.device)
    if x_absmax is None:
        x_absmax = torch.empty((T,), dtype=torch.float32, device=x.device)
    if ln_eps is None:
        check(lib().sbn_bitlinear_fwd_bf16(w.handle, _ptr(x), _ld(x, w.K), T, _ptr(x_q),
                                           _ld(x_q, w.K), _ptr(x_absmax), _ptr(y),
                                           _ld(y, w.n_out), kind, _stream(stream)))
    else:
        check(lib().sbn_bitlinear_fwd_ln_bf16(w.handle, _ptr(x), _ld(x, w.K), T, float(ln_eps),
                                              _ptr(x_q), _ld(x_q, w.K), _ptr(x_absmax), _ptr(y),
                                              _ld(y, w.n_out), kind, _stream(stream)))
    return y, x_q, x_absmax


def bitlinear_bwd_dx(dy, w: PackedWeight, dx=None, stream=None):
    """Straight-through data gradient: dy bf16 [T][n_out] -> dx fp32 [T][K] = gamma * dy @ codes."""
    import torch
    _require_cuda(dy, "dy")
    if dy.dtype not in (torch.bfloat16, torch.int16):
        raise ValueError("dy must be bfloat16 (or int16 bf16 bit patterns)")
    T = dy.shape[0]
    if dx is None:
        dx = torch.empty((T, w.K), dtype=torch.float32, device=dy.device)
    check(lib().sbn_bitlinear_bwd_dx(w.handle, _ptr(dy), _ld(dy, w.n_out), T, _ptr(dx),
                                     _ld(dx, w.K), _stream(stream)))
    return dx


def _group_arrays(ws, ys):
    n = len(ws)
    handles = (ctypes.c_void_p * n)(*[w.handle.value for w in ws])
    outs = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    lds = (ctypes.c_int64 * n)(*[_ld(y, w.n_out) for w, y in zip(ws, ys)])
    return handles, outs, lds


def _group_outputs(ws, T, kind, ys, device):
    import torch
    if ys is not None:
        return list(ys)
    dt = torch.float32 if kind == SBN_OUT_F32 else torch.int32
    return [torch.empty((T, w.n_out), dtype=dt, device=device) for w in ws]


def bitlinear_group(x_q, x_absmax, ws, out: str = "f32", ys=None, stream=None):
    """Grouped forward of several packed weights on the same x_q (sbn_bitlinear_fwd_group):
    returns the list of outputs [T][n_out_i]."""
    _require_cuda(x_q, "x_q")
    T = x_q.shape[0]
    kind = SBN_OUT_F32 if out == "f32" else SBN_OUT_I32_ACC
    ys = _group_outputs(ws, T, kind, ys, x_q.device)
    handles, outs, lds = _group_arrays(ws, ys)
    check(lib().sbn_bitlinear_fwd_group(handles, len(ws), _ptr(x_q), _ld(x_q, ws[0].K),
                                        _ptr(x_absmax), T, outs, lds, kind, _stream(stream)))
    return ys


def bitlinear_group_bf16(x, ws, out: str = "f32", ys=None, x_q=None, x_absmax=None,
                         ln_eps: float = 0.0, stream=None):
    """Grouped quantize-and-multiply (sbn_bitlinear_fwd_group_bf16): x bf16 [T][K] ->
    (list of outputs, x_q, a'). ln_eps > 0 runs the parameter-free LayerNorm first."""
    import torch
    _require_cuda(x, "x")
    if x.dtype not in (torch.bfloat16, torch.int16):
        raise ValueError("x must be bfloat16 (or int16 bf16 bit patterns)")
    T = x.shape[0]
    K = ws[0].K
    kind = SBN_OUT_F32 if out == "f32" else SBN_OUT_I32_ACC
    ys = _group_outputs(ws, T, kind, ys, x.device)
    if x_q is None:
        x_q = torch.empty((T, K), dtype=torch.int8, device=x.device)
    if x_absmax is None:
        x_absmax = torch.empty((T,), dtype=torch.float32, device=x.device)
    handles, outs, lds = _group_arrays(ws, ys)
    check(lib().sbn_bitlinear_fwd_group_bf16(handles, len(ws), _ptr(x), _ld(x, K), T,
                                             float(ln_eps), _ptr(x_q), _ld(x_q, K),
                                             _ptr(x_absmax), outs, lds, kind, _stream(stream)))
    return ys, x_q, x_absmax


def bitlinear_latent_static(w, n: int, m: int, x_q, x_absmax, out: str = "f32", y=None,
                            stream=None):
    """Pack of the latent weights w fp32 [n_out][K] and forward on x_q, with no device allocation
    in the library (sbn_bitlinear_fwd_latent_static: its fixed workspace holds the packed planes).
    Returns y [T][n_out]."""
    import torch
    _require_cuda(w, "w")
    _require_cuda(x_q, "x_q")
    n_out, K = w.shape
    T = x_q.shape[0]
    kind = SBN_OUT_F32 if out == "f32" else SBN_OUT_I32_ACC
    if y is None:
        y = torch.empty((T, n_out), dtype=torch.float32 if kind == SBN_OUT_F32 else torch.int32,
                        device=x_q.device)
    check(lib().sbn_bitlinear_fwd_latent_static(_ptr(w), n_out, K, _ld(w, K), n, m, _ptr(x_q),
                                                _ld(x_q, K), _ptr(x_absmax), T, _ptr(y),
                                                _ld(y, n_out), kind, _stream(stream)))
    return y
