"""Python binding of librkv, the ResidualKV cache-write path for MI355X.

Argument marshalling only: every function forwards to the C entry point of
the same name in ``librkv.so`` (declared in ``include/rkv.h``).  Tensors are
passed as device pointers (``tensor.data_ptr()``) and streams as raw HIP
stream handles; PyTorch is used by callers for device memory and streams.

There is no fallback: if the compiled library is missing, every call raises.
Build it with ``python -m reference_residual_encoding_amd._build`` or
``__graft_entry__.build()``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librkv.so")

RKV_OK = 0
RKV_ERR_INVALID_ARG = 1
RKV_ERR_UNSUPPORTED = 2
RKV_ERR_WORKSPACE = 3
RKV_ERR_DEVICE = 4

RKV_F32 = 0
RKV_BF16 = 1

# Exported symbols of librkv.so (must match include/rkv.h).
EXPORTS = (
    "rkv_encode_workspace_bytes",
    "rkv_encode",
    "rkv_packed_weights_bytes",
    "rkv_pack_weights",
    "rkv_encode_packed",
    "rkv_dequant_gather",
    "rkv_quantize",
    "rkv_select",
    "rkv_status_str",
    "rkv_last_error",
    "rkv_abi_version",
    "rkv_profile_begin",
    "rkv_profile_read",
    "rkv_restore_workspace_bytes",
    "rkv_restore",
    "rkv_packed_decoder_bytes",
    "rkv_pack_decoder",
    "rkv_restore_packed",
    "rkv_append_workspace_bytes",
    "rkv_append",
    "rkv_append_noalloc",
    "rkv_ref_proj_bytes",
    "rkv_project_refs_workspace_bytes",
    "rkv_append_proj_workspace_bytes",
    "rkv_project_refs",
    "rkv_append_proj",
    "rkv_reference_positions",
    "rkv_store_refs",
)

STAGES = ("pack", "norms", "dist", "merge", "proj", "swiglu", "w3", "quant", "gather", "restore",
          "append", "store")
RKV_ABI_VERSION = 8
RKV_REF_INPUT = 0
RKV_REF_FP8 = 1


class rkv_params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "N", "D", "d_ff", "d_c", "k", "g", "b", "ref_stride")] + \
               [("dtype", ctypes.c_int32), ("n_sink", ctypes.c_int32), ("ref_alpha", ctypes.c_double),
                ("ref_format", ctypes.c_int32)]


class RkvError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {status_name(status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def lib() -> ctypes.CDLL:
    """Load librkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"librkv.so not built at {LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(rkv_params)
        vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
        L.rkv_encode_workspace_bytes.argtypes = [P]
        L.rkv_encode_workspace_bytes.restype = sz
        L.rkv_encode.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.rkv_encode.restype = ctypes.c_int
        L.rkv_packed_weights_bytes.argtypes = [P]
        L.rkv_packed_weights_bytes.restype = sz
        L.rkv_pack_weights.argtypes = [P, vp, vp, vp, vp, sz, vp]
        L.rkv_pack_weights.restype = ctypes.c_int
        L.rkv_encode_packed.argtypes = [P, vp, vp, sz, vp, vp, vp, vp, vp, vp, sz, vp]
        L.rkv_encode_packed.restype = ctypes.c_int
        L.rkv_dequant_gather.argtypes = [P, vp, vp, vp, vp, i32, vp, ctypes.c_int, vp]
        L.rkv_dequant_gather.restype = ctypes.c_int
        L.rkv_quantize.argtypes = [P, vp, i64, vp, vp, vp, vp]
        L.rkv_quantize.restype = ctypes.c_int
        L.rkv_select.argtypes = [P, vp, vp, vp, sz, vp]
        L.rkv_select.restype = ctypes.c_int
        L.rkv_status_str.argtypes = [ctypes.c_int]
        L.rkv_status_str.restype = ctypes.c_char_p
        L.rkv_last_error.argtypes = []
        L.rkv_last_error.restype = ctypes.c_char_p
        L.rkv_abi_version.argtypes = []
        L.rkv_abi_version.restype = ctypes.c_int
        L.rkv_profile_begin.argtypes = [ctypes.c_uint32]
        L.rkv_profile_begin.restype = ctypes.c_int
        L.rkv_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64)]
        L.rkv_profile_read.restype = ctypes.c_int
        L.rkv_restore_workspace_bytes.argtypes = [P, i32]
        L.rkv_restore_workspace_bytes.restype = sz
        L.rkv_restore.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, i32, ctypes.c_float, vp,
                                  ctypes.c_int, vp, sz, vp]
        L.rkv_restore.restype = ctypes.c_int
        L.rkv_packed_decoder_bytes.argtypes = [P]
        L.rkv_packed_decoder_bytes.restype = sz
        L.rkv_pack_decoder.argtypes = [P, vp, vp, sz, vp]
        L.rkv_pack_decoder.restype = ctypes.c_int
        L.rkv_restore_packed.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp, i32, ctypes.c_float,
                                         vp, ctypes.c_int, vp, sz, vp]
        L.rkv_restore_packed.restype = ctypes.c_int
        L.rkv_append_workspace_bytes.argtypes = [P]
        L.rkv_append_workspace_bytes.restype = sz
        L.rkv_append.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.rkv_append.restype = ctypes.c_int
        L.rkv_append_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.rkv_append_noalloc.restype = ctypes.c_int
        L.rkv_ref_proj_bytes.argtypes = [P]
        L.rkv_ref_proj_bytes.restype = sz
        L.rkv_project_refs_workspace_bytes.argtypes = [P]
        L.rkv_project_refs_workspace_bytes.restype = sz
        L.rkv_append_proj_workspace_bytes.argtypes = [P]
        L.rkv_append_proj_workspace_bytes.restype = sz
        L.rkv_project_refs.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
        L.rkv_project_refs.restype = ctypes.c_int
        L.rkv_append_proj.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.rkv_append_proj.restype = ctypes.c_int
        L.rkv_reference_positions.argtypes = [P, vp, i32]
        L.rkv_reference_positions.restype = i32
        L.rkv_store_refs.argtypes = [P, vp, vp, vp]
        L.rkv_store_refs.restype = ctypes.c_int
        _lib = L
    return _lib


def status_name(status: int) -> str:
    return lib().rkv_status_str(int(status)).decode()


def _check(fn: str, status: int) -> int:
    if status != RKV_OK:
        raise RkvError(fn, status, lib().rkv_last_error().decode())
    return status


def params(*, B, T, N, D, d_ff, d_c, k, g, b, ref_stride, dtype, n_sink=0,
           ref_alpha=0.0, ref_format=RKV_REF_INPUT) -> rkv_params:
    """Build an rkv_params; dtype is RKV_F32/RKV_BF16 or "f32"/"bf16";
    ref_format RKV_REF_INPUT/RKV_REF_FP8 or "input"/"fp8"."""
    if isinstance(dtype, str):
        dtype = {"f32": RKV_F32, "bf16": RKV_BF16}[dtype]
    if isinstance(ref_format, str):
        ref_format = {"input": RKV_REF_INPUT, "fp8": RKV_REF_FP8}[ref_format]
    return rkv_params(B, T, N, D, d_ff, d_c, k, g, b, ref_stride, dtype, n_sink, ref_alpha,
                      ref_format)


_BF16 = ("torch.bfloat16",)
_F32 = ("torch.float32",)
_I32 = ("torch.int32",)
_U8 = ("torch.uint8",)
_HALF = ("torch.float16", "torch.int16", "torch.uint16")   # fp16 bits of Delta_h, m_h


def _p(x, name: str = "pointer", dtypes=None, nbytes: int = 0) -> Optional[int]:
    """Device pointer of a tensor (or an int / None), checked before any call.

    A tensor must live on the GPU, be contiguous, have one of `dtypes`
    (names as ``str(tensor.dtype)``) when given, and hold at least `nbytes`
    bytes; otherwise ValueError, so that no host address, strided view or
    short buffer reaches a kernel.  A plain int is passed through as a raw
    device address (the caller's responsibility)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise ValueError(f"{name}: tensor must be on the GPU (device {getattr(x, 'device', '?')})")
    if not x.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    if dtypes is not None and str(x.dtype) not in dtypes:
        raise ValueError(f"{name}: dtype {x.dtype} not one of {', '.join(dtypes)}")
    have = x.numel() * x.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: {have} bytes, needs at least {nbytes}")
    return x.data_ptr()


def _elem(p: "rkv_params"):
    """(dtype names, bytes per element) of kv / weights for p.dtype."""
    return (_BF16, 2) if p.dtype == RKV_BF16 else (_F32, 4)


def _out_elem(out_dtype: int):
    return (_BF16, 2) if out_dtype == RKV_BF16 else (_F32, 4)


def _record_sizes(p: "rkv_params", rows: int):
    """Bytes of codes, and of scale / zmin each, for `rows` records."""
    codes = rows * p.d_c * p.b // 8 if p.b > 0 else 0
    groups = 0 if p.b == 16 or p.g <= 0 else p.d_c // p.g
    return max(codes, 0), max(rows * groups * 2, 0)


def _n_ref(p: "rkv_params") -> int:
    n = lib().rkv_reference_positions(ctypes.byref(p), None, 0)
    return max(int(n), 0)


def _ref_store(p: "rkv_params", kv, name="kv"):
    """The stored references: kv [B][T][C] at input precision, or the FP8
    store [B][n_ref][C] of bytes."""
    C = 2 * p.N * p.D
    if p.ref_format == RKV_REF_FP8:
        return _p(kv, name, _U8, p.B * _n_ref(p) * C)
    dt, es = _elem(p)
    return _p(kv, name, dt, p.B * p.T * C * es)


def _s(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# -- entry points, same names as the C ABI ---------------------------------
def rkv_abi_version() -> int:
    return lib().rkv_abi_version()


def rkv_last_error() -> str:
    return lib().rkv_last_error().decode()


def rkv_status_str(status: int) -> str:
    return status_name(status)


def rkv_encode_workspace_bytes(p: rkv_params) -> int:
    return int(lib().rkv_encode_workspace_bytes(ctypes.byref(p)))


def rkv_encode(p: rkv_params, kv, w1, w2, w3, ref_idx, codes, scale, zmin, z, workspace,
               workspace_bytes: int, stream=None, *, check: bool = True) -> int:
    dt, es = _elem(p)
    C, rows = 2 * p.N * p.D, p.B * p.T
    cb, sb = _record_sizes(p, rows)
    args = (_p(kv, "kv", dt, rows * C * es), _p(w1, "w1", dt, C * p.d_ff * es),
            _p(w2, "w2", dt, C * p.d_ff * es), _p(w3, "w3", dt, p.d_ff * p.d_c * es),
            _p(ref_idx, "ref_idx", _I32, rows * p.k * 4), _p(codes, "codes", _U8, cb),
            _p(scale, "scale", _HALF, sb), _p(zmin, "zmin", _HALF, sb),
            _p(z, "z", _F32, rows * p.d_c * 4), _p(workspace, "workspace", None, workspace_bytes))
    st = lib().rkv_encode(ctypes.byref(p), *args, int(workspace_bytes), _s(stream))
    return _check("rkv_encode", st) if check else st


def rkv_packed_weights_bytes(p: rkv_params) -> int:
    return int(lib().rkv_packed_weights_bytes(ctypes.byref(p)))


def rkv_pack_weights(p: rkv_params, w1, w2, w3, packed, packed_bytes: int, stream=None, *,
                     check: bool = True) -> int:
    dt, es = _elem(p)
    C = 2 * p.N * p.D
    st = lib().rkv_pack_weights(ctypes.byref(p), _p(w1, "w1", dt, C * p.d_ff * es),
                                _p(w2, "w2", dt, C * p.d_ff * es),
                                _p(w3, "w3", dt, p.d_ff * p.d_c * es),
                                _p(packed, "packed", None, packed_bytes), int(packed_bytes),
                                _s(stream))
    return _check("rkv_pack_weights", st) if check else st


def rkv_encode_packed(p: rkv_params, kv, packed, packed_bytes: int, ref_idx, codes, scale, zmin,
                      z, workspace, workspace_bytes: int, stream=None, *,
                      check: bool = True) -> int:
    dt, es = _elem(p)
    C, rows = 2 * p.N * p.D, p.B * p.T
    cb, sb = _record_sizes(p, rows)
    args = (_p(kv, "kv", dt, rows * C * es), _p(packed, "packed", None, packed_bytes),
            int(packed_bytes), _p(ref_idx, "ref_idx", _I32, rows * p.k * 4),
            _p(codes, "codes", _U8, cb), _p(scale, "scale", _HALF, sb),
            _p(zmin, "zmin", _HALF, sb), _p(z, "z", _F32, rows * p.d_c * 4),
            _p(workspace, "workspace", None, workspace_bytes))
    st = lib().rkv_encode_packed(ctypes.byref(p), *args, int(workspace_bytes), _s(stream))
    return _check("rkv_encode_packed", st) if check else st


def rkv_dequant_gather(p: rkv_params, codes, scale, zmin, idx, n_idx: int, out, out_dtype,
                       stream=None, *, check: bool = True) -> int:
    if isinstance(out_dtype, str):
        out_dtype = {"f32": RKV_F32, "bf16": RKV_BF16}[out_dtype]
    rows, n = p.B * p.T, max(int(n_idx), 0)
    cb, sb = _record_sizes(p, rows)
    odt, oes = _out_elem(out_dtype)
    st = lib().rkv_dequant_gather(ctypes.byref(p), _p(codes, "codes", _U8, cb),
                                  _p(scale, "scale", _HALF, sb), _p(zmin, "zmin", _HALF, sb),
                                  _p(idx, "idx", _I32, n * 4), int(n_idx),
                                  _p(out, "out", odt, n * p.d_c * oes), int(out_dtype),
                                  _s(stream))
    return _check("rkv_dequant_gather", st) if check else st


def rkv_quantize(p: rkv_params, z, rows: int, codes, scale, zmin, stream=None, *,
                 check: bool = True) -> int:
    n = max(int(rows), 0)
    cb, sb = _record_sizes(p, n)
    st = lib().rkv_quantize(ctypes.byref(p), _p(z, "z", _F32, n * p.d_c * 4), int(rows),
                            _p(codes, "codes", _U8, cb), _p(scale, "scale", _HALF, sb),
                            _p(zmin, "zmin", _HALF, sb), _s(stream))
    return _check("rkv_quantize", st) if check else st


def rkv_select(p: rkv_params, kv, ref_idx, workspace, workspace_bytes: int, stream=None, *,
               check: bool = True) -> int:
    dt, es = _elem(p)
    rows = p.B * p.T
    st = lib().rkv_select(ctypes.byref(p), _p(kv, "kv", dt, rows * 2 * p.N * p.D * es),
                          _p(ref_idx, "ref_idx", _I32, rows * p.k * 4),
                          _p(workspace, "workspace", None, workspace_bytes),
                          int(workspace_bytes), _s(stream))
    return _check("rkv_select", st) if check else st


def rkv_profile_begin(stage_mask: int) -> int:
    return _check("rkv_profile_begin", lib().rkv_profile_begin(int(stage_mask)))


def rkv_profile_read(stage: int):
    """Returns (total_ms, launches) of one stage since rkv_profile_begin."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check("rkv_profile_read", lib().rkv_profile_read(int(stage), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def rkv_restore_workspace_bytes(p: rkv_params, n_idx: int) -> int:
    return int(lib().rkv_restore_workspace_bytes(ctypes.byref(p), int(n_idx)))


def rkv_restore(p: rkv_params, codes, scale, zmin, ref_idx, kv, wd, idx, n_idx: int,
                rope_theta: float, out, out_dtype, workspace, workspace_bytes: int, stream=None,
                *, check: bool = True) -> int:
    if isinstance(out_dtype, str):
        out_dtype = {"f32": RKV_F32, "bf16": RKV_BF16}[out_dtype]
    dt, es = _elem(p)
    C, rows, n = 2 * p.N * p.D, p.B * p.T, max(int(n_idx), 0)
    cb, sb = _record_sizes(p, rows)
    odt, oes = _out_elem(out_dtype)
    st = lib().rkv_restore(ctypes.byref(p), _p(codes, "codes", _U8, cb),
                           _p(scale, "scale", _HALF, sb), _p(zmin, "zmin", _HALF, sb),
                           _p(ref_idx, "ref_idx", _I32, rows * p.k * 4), _ref_store(p, kv),
                           _p(wd, "wd", dt, p.d_c * C * es), _p(idx, "idx", _I32, n * 4),
                           int(n_idx), float(rope_theta), _p(out, "out", odt, n * C * oes),
                           int(out_dtype), _p(workspace, "workspace", None, workspace_bytes),
                           int(workspace_bytes), _s(stream))
    return _check("rkv_restore", st) if check else st


def rkv_packed_decoder_bytes(p: rkv_params) -> int:
    return int(lib().rkv_packed_decoder_bytes(ctypes.byref(p)))


def rkv_pack_decoder(p: rkv_params, wd, packed, packed_bytes: int, stream=None, *,
                     check: bool = True) -> int:
    dt, es = _elem(p)
    C = 2 * p.N * p.D
    st = lib().rkv_pack_decoder(ctypes.byref(p), _p(wd, "wd", dt, p.d_c * C * es),
                                _p(packed, "packed", None, packed_bytes), int(packed_bytes),
                                _s(stream))
    return _check("rkv_pack_decoder", st) if check else st


def rkv_restore_packed(p: rkv_params, codes, scale, zmin, ref_idx, kv, packed,
                       packed_bytes: int, idx, n_idx: int, rope_theta: float, out, out_dtype,
                       workspace, workspace_bytes: int, stream=None, *,
                       check: bool = True) -> int:
    if isinstance(out_dtype, str):
        out_dtype = {"f32": RKV_F32, "bf16": RKV_BF16}[out_dtype]
    C, rows, n = 2 * p.N * p.D, p.B * p.T, max(int(n_idx), 0)
    cb, sb = _record_sizes(p, rows)
    odt, oes = _out_elem(out_dtype)
    st = lib().rkv_restore_packed(ctypes.byref(p), _p(codes, "codes", _U8, cb),
                                  _p(scale, "scale", _HALF, sb), _p(zmin, "zmin", _HALF, sb),
                                  _p(ref_idx, "ref_idx", _I32, rows * p.k * 4),
                                  _ref_store(p, kv), _p(packed, "packed", None, packed_bytes),
                                  int(packed_bytes), _p(idx, "idx", _I32, n * 4), int(n_idx),
                                  float(rope_theta), _p(out, "out", odt, n * C * oes),
                                  int(out_dtype),
                                  _p(workspace, "workspace", None, workspace_bytes),
                                  int(workspace_bytes), _s(stream))
    return _check("rkv_restore_packed", st) if check else st


def rkv_append_workspace_bytes(p: rkv_params) -> int:
    return int(lib().rkv_append_workspace_bytes(ctypes.byref(p)))


def rkv_append(p: rkv_params, kv, kv_new, pos, w1, w2, w3, ref_idx, codes, scale, zmin, z,
               workspace, workspace_bytes: int, stream=None, *, check: bool = True) -> int:
    dt, es = _elem(p)
    C, rows = 2 * p.N * p.D, p.B * p.T
    cb, sb = _record_sizes(p, rows)
    st = lib().rkv_append(ctypes.byref(p), _ref_store(p, kv), _p(kv_new, "kv_new", dt, p.B * C * es),
                          _p(pos, "pos", _I32, p.B * 4), _p(w1, "w1", dt, C * p.d_ff * es),
                          _p(w2, "w2", dt, C * p.d_ff * es), _p(w3, "w3", dt, p.d_ff * p.d_c * es),
                          _p(ref_idx, "ref_idx", _I32, rows * p.k * 4), _p(codes, "codes", _U8, cb),
                          _p(scale, "scale", _HALF, sb), _p(zmin, "zmin", _HALF, sb),
                          _p(z, "z", _F32, rows * p.d_c * 4),
                          _p(workspace, "workspace", None, workspace_bytes),
                          int(workspace_bytes), _s(stream))
    return _check("rkv_append", st) if check else st


def rkv_append_noalloc(p: rkv_params, kv, kv_new, pos, w1, w2, w3, ref_idx, codes, scale, zmin,
                       z, stream=None, *, check: bool = True) -> int:
    """rkv_append on the library's fixed device scratch (no workspace)."""
    dt, es = _elem(p)
    C, rows = 2 * p.N * p.D, p.B * p.T
    cb, sb = _record_sizes(p, rows)
    st = lib().rkv_append_noalloc(
        ctypes.byref(p), _ref_store(p, kv), _p(kv_new, "kv_new", dt, p.B * C * es),
        _p(pos, "pos", _I32, p.B * 4), _p(w1, "w1", dt, C * p.d_ff * es),
        _p(w2, "w2", dt, C * p.d_ff * es), _p(w3, "w3", dt, p.d_ff * p.d_c * es),
        _p(ref_idx, "ref_idx", _I32, rows * p.k * 4), _p(codes, "codes", _U8, cb),
        _p(scale, "scale", _HALF, sb), _p(zmin, "zmin", _HALF, sb),
        _p(z, "z", _F32, rows * p.d_c * 4), _s(stream))
    return _check("rkv_append_noalloc", st) if check else st


def rkv_ref_proj_bytes(p: rkv_params) -> int:
    return int(lib().rkv_ref_proj_bytes(ctypes.byref(p)))


def rkv_project_refs_workspace_bytes(p: rkv_params) -> int:
    return int(lib().rkv_project_refs_workspace_bytes(ctypes.byref(p)))


def rkv_append_proj_workspace_bytes(p: rkv_params) -> int:
    return int(lib().rkv_append_proj_workspace_bytes(ctypes.byref(p)))


def rkv_project_refs(p: rkv_params, kv, w1, w2, ref_proj, workspace, workspace_bytes: int,
                     stream=None, *, check: bool = True) -> int:
    dt, es = _elem(p)
    C = 2 * p.N * p.D
    st = lib().rkv_project_refs(ctypes.byref(p), _ref_store(p, kv), _p(w1, "w1", dt, C * p.d_ff * es),
                                _p(w2, "w2", dt, C * p.d_ff * es),
                                _p(ref_proj, "ref_proj", _F32, rkv_ref_proj_bytes(p)),
                                _p(workspace, "workspace", None, workspace_bytes),
                                int(workspace_bytes), _s(stream))
    return _check("rkv_project_refs", st) if check else st


def rkv_append_proj(p: rkv_params, kv, ref_proj, kv_new, pos, w1, w2, w3, ref_idx, codes, scale,
                    zmin, z, workspace, workspace_bytes: int, stream=None, *,
                    check: bool = True) -> int:
    dt, es = _elem(p)
    C, rows = 2 * p.N * p.D, p.B * p.T
    cb, sb = _record_sizes(p, rows)
    st = lib().rkv_append_proj(ctypes.byref(p), _ref_store(p, kv),
                               _p(ref_proj, "ref_proj", _F32, rkv_ref_proj_bytes(p)),
                               _p(kv_new, "kv_new", dt, p.B * C * es),
                               _p(pos, "pos", _I32, p.B * 4), _p(w1, "w1", dt, C * p.d_ff * es),
                               _p(w2, "w2", dt, C * p.d_ff * es), _p(w3, "w3", dt, p.d_ff * p.d_c * es),
                               _p(ref_idx, "ref_idx", _I32, rows * p.k * 4), _p(codes, "codes", _U8, cb),
                               _p(scale, "scale", _HALF, sb), _p(zmin, "zmin", _HALF, sb),
                               _p(z, "z", _F32, rows * p.d_c * 4),
                               _p(workspace, "workspace", None, workspace_bytes),
                               int(workspace_bytes), _s(stream))
    return _check("rkv_append_proj", st) if check else st


def rkv_reference_positions(p: rkv_params):
    """The schedule's reference positions (host query): a list of ints."""
    n = lib().rkv_reference_positions(ctypes.byref(p), None, 0)
    if n < 0:
        raise RkvError("rkv_reference_positions", RKV_ERR_INVALID_ARG, rkv_last_error())
    buf = (ctypes.c_int32 * max(n, 1))()
    lib().rkv_reference_positions(ctypes.byref(p), ctypes.cast(buf, ctypes.c_void_p), n)
    return list(buf[:n])


def rkv_store_refs(p: rkv_params, kv, ref_store, stream=None, *, check: bool = True) -> int:
    dt, es = _elem(p)
    C = 2 * p.N * p.D
    st = lib().rkv_store_refs(ctypes.byref(p), _p(kv, "kv", dt, p.B * p.T * C * es),
                              _p(ref_store, "ref_store", _U8, p.B * _n_ref(p) * C), _s(stream))
    return _check("rkv_store_refs", st) if check else st
