"""Thin ctypes binding of the FP8 exponent codec in libk3huf.so (include/e8huf.h):
argument marshalling only. Every decode step runs in the library's HIP
kernel; there is no fallback path."""

from __future__ import annotations

import ctypes

import numpy as np

from . import k3huf

LUT_MAX = 256 * 18        # E8HUF_LUT_MAX
HDR_BYTES = 128
DEV_HEADER, DEV_INDEX, DEV_CODE, DEV_LANE_END = 1, 4, 8, 16
OUT_BF16, OUT_F16 = 1, 2  # E8HUF_OUT_*
EXPORTS = ("e8huf_build_table", "e8huf_layer_info", "e8huf_encode_bound", "e8huf_encode",
           "e8huf_decode", "e8huf_decode_widen")


class Info(ctypes.Structure):
    _fields_ = [("n_values", ctypes.c_uint64), ("n_bits", ctypes.c_uint64),
                ("container_bytes", ctypes.c_uint64), ("n_blocks", ctypes.c_uint32),
                ("exp_bits", ctypes.c_uint32), ("codelen", ctypes.c_uint8 * 32)]


_ready = False


def lib() -> ctypes.CDLL:
    global _ready
    L = k3huf.lib()
    if not _ready:
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.e8huf_build_table.argtypes = [vp, ctypes.c_int, vp, ctypes.POINTER(ctypes.c_int)]
        L.e8huf_build_table.restype = ctypes.c_int
        L.e8huf_layer_info.argtypes = [vp, sz, ctypes.POINTER(Info)]
        L.e8huf_layer_info.restype = ctypes.c_int
        L.e8huf_encode_bound.argtypes = [ctypes.c_uint64]
        L.e8huf_encode_bound.restype = ctypes.c_int64
        L.e8huf_encode.argtypes = [vp, ctypes.c_uint64, ctypes.c_int, vp, ctypes.c_uint64, ctypes.c_int]
        L.e8huf_encode.restype = ctypes.c_int64
        L.e8huf_decode.argtypes = [vp, sz, vp, ctypes.c_int, vp, ctypes.c_uint64, vp, vp]
        L.e8huf_decode.restype = ctypes.c_int
        L.e8huf_decode_widen.argtypes = [vp, sz, vp, ctypes.c_int, vp, ctypes.c_uint64, ctypes.c_int,
                                         ctypes.c_float, vp, vp]
        L.e8huf_decode_widen.restype = ctypes.c_int
        _ready = True
    return L


def build_table_rc(codelen, exp_bits: int):
    """(return code, table[LUT_MAX] u16, entries used)."""
    cl = np.zeros(32, np.uint8)
    c = np.asarray(codelen, dtype=np.uint8)
    cl[: c.size] = c
    lut = np.zeros(LUT_MAX, np.uint16)
    n = ctypes.c_int()
    rc = lib().e8huf_build_table(cl.ctypes.data, exp_bits, lut.ctypes.data, ctypes.byref(n))
    return rc, lut, n.value


def build_table(codelen, exp_bits: int) -> np.ndarray:
    """The two-level decode table (u16), trimmed to the entries used."""
    rc, lut, n = build_table_rc(codelen, exp_bits)
    k3huf._check(rc, "e8huf_build_table")
    return lut[:n].copy()


def layer_info(blob) -> dict:
    b = k3huf._u8(blob)
    info = Info()
    k3huf._check(lib().e8huf_layer_info(b.ctypes.data, b.size, ctypes.byref(info)), "e8huf_layer_info")
    return dict(n_values=info.n_values, n_bits=info.n_bits, container_bytes=info.container_bytes,
                n_blocks=info.n_blocks, exp_bits=info.exp_bits,
                codelen=np.frombuffer(bytes(info.codelen), np.uint8).copy())


def encode_bound(n: int) -> int:
    return k3huf._check(lib().e8huf_encode_bound(n), "e8huf_encode_bound")


def encode(x, exp_bits: int = 4, n_threads: int = 0) -> np.ndarray:
    """Pack FP8 bytes x (E4M3: exp_bits 4; E5M2: 5) into an E8HF container."""
    r = k3huf._u8(x)
    cap = encode_bound(r.size)
    out = np.empty(cap, np.uint8)
    n = k3huf._check(lib().e8huf_encode(r.ctypes.data, r.size, exp_bits, out.ctypes.data, cap, n_threads),
                     "e8huf_encode")
    return out[:n]


def decode(d_blob, d_lut, d_out, d_status=None, stream=None) -> None:
    """Queue the decode of one container: d_blob uint8 (the container),
    d_lut the table from build_table (16-bit entries), d_out uint8 of the
    tensor's value count, d_status a 32-bit device word or None."""
    k3huf._dev(d_blob, "d_blob")
    k3huf._dev(d_lut, "d_lut", elem=2)
    k3huf._dev(d_out, "d_out")
    rc = lib().e8huf_decode(d_blob.data_ptr(), k3huf._nbytes(d_blob), d_lut.data_ptr(), d_lut.numel(),
                            d_out.data_ptr(), k3huf._nbytes(d_out), k3huf._stream_handle(stream),
                            k3huf._status(d_status))
    k3huf._check(rc, "e8huf_decode")


def decode_raw(blob_ptr, blob_bytes, lut_ptr, lut_entries, out_ptr, n_values, stream, status_ptr) -> int:
    """Unchecked pointer-level call; returns the C return code."""
    return lib().e8huf_decode(blob_ptr, blob_bytes, lut_ptr, lut_entries, out_ptr, n_values, stream,
                              status_ptr)


def decode_widen(d_blob, d_lut, d_out, out_kind=None, scale: float = 1.0, d_status=None, stream=None) -> None:
    """Queue the decode of one container into 16-bit floats: d_out holds the
    tensor's value count of bfloat16 or float16 elements (out_kind defaults
    from its dtype: OUT_BF16, OUT_F16); element i is value i times scale,
    rounded to nearest even."""
    if out_kind is None:
        import torch
        out_kind = {torch.bfloat16: OUT_BF16, torch.float16: OUT_F16}.get(d_out.dtype)
        if out_kind is None:
            raise ValueError("decode_widen: d_out must be bfloat16 or float16 (or give out_kind)")
    k3huf._dev(d_blob, "d_blob")
    k3huf._dev(d_lut, "d_lut", elem=2)
    k3huf._dev(d_out, "d_out", elem=2)
    rc = lib().e8huf_decode_widen(d_blob.data_ptr(), k3huf._nbytes(d_blob), d_lut.data_ptr(), d_lut.numel(),
                                  d_out.data_ptr(), d_out.numel(), out_kind, float(scale),
                                  k3huf._stream_handle(stream), k3huf._status(d_status))
    k3huf._check(rc, "e8huf_decode_widen")


def decode_widen_raw(blob_ptr, blob_bytes, lut_ptr, lut_entries, out_ptr, n_values, out_kind, scale, stream,
                     status_ptr) -> int:
    """Unchecked pointer-level call; returns the C return code."""
    return lib().e8huf_decode_widen(blob_ptr, blob_bytes, lut_ptr, lut_entries, out_ptr, n_values, out_kind, scale,
                                    stream, status_ptr)
