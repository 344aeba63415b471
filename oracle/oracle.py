"""ctypes wrapper around the plain C oracles (k3huf_oracle.c: the bf16
high-byte codec; e8huf_oracle.c: the FP8 exponent codec).

TEST INFRASTRUCTURE ONLY: the product path must never import this module.
Every function here calls straight into the C oracle; see that file's header
for the page sections each step follows.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "k3huf_oracle.c"), os.path.join(_HERE, "e8huf_oracle.c")]
_LIB = os.path.join(_HERE, "_build", "liboracle.so")

OK, E_ARG, E_EMPTY, E_OVERSUB, E_BADLEN, E_OVERLAP, E_FORMAT, E_CORRUPT, E_INDEX = (
    0, -1, -2, -3, -4, -5, -6, -7, -9)

MAXLEN = 12


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into oracle/_build/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(map(os.path.getmtime, _SRCS)):
        os.makedirs(os.path.dirname(_LIB), exist_ok=True)
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC",
                               "-o", tmp, *_SRCS, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        L.oh_huffman_depths.argtypes = [u64p, u8p]
        L.oh_huffman_depths.restype = ctypes.c_int
        L.oh_code_lengths.argtypes = [u64p, u8p]
        L.oh_code_lengths.restype = ctypes.c_int
        L.oh_kraft.argtypes = [u8p]
        L.oh_kraft.restype = ctypes.c_int
        L.oh_canonical.argtypes = [u8p, ctypes.POINTER(ctypes.c_uint32)]
        L.oh_canonical.restype = None
        L.oh_check_table.argtypes = [u8p]
        L.oh_check_table.restype = ctypes.c_int
        L.oh_decode_prefix.argtypes = [u8p, ctypes.c_uint32, ctypes.POINTER(ctypes.c_int),
                                       ctypes.POINTER(ctypes.c_int)]
        L.oh_decode_prefix.restype = ctypes.c_int
        L.oh_encode_bound.argtypes = [ctypes.c_uint64]
        L.oh_encode_bound.restype = ctypes.c_int64
        L.oh_encode_bound_lanes.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
        L.oh_encode_bound_lanes.restype = ctypes.c_int64
        L.oh_encode_layer_lanes.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p,
                                            ctypes.c_uint64]
        L.oh_encode_layer_lanes.restype = ctypes.c_int64
        L.oh_encode_layer.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_uint64]
        L.oh_encode_layer.restype = ctypes.c_int64
        L.oh_decode_layer.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_uint64]
        L.oh_decode_layer.restype = ctypes.c_int
        L.oh_decode_stripes.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32,
                                        ctypes.c_uint32, ctypes.c_void_p, ctypes.c_uint64]
        L.oh_decode_stripes.restype = ctypes.c_int
        L.oh_check_index.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
        L.oh_check_index.restype = ctypes.c_int
        L.oh_raw_bytes.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
        L.oh_raw_bytes.restype = ctypes.c_int64
        L.e8_kraft.argtypes = [u8p]
        L.e8_kraft.restype = ctypes.c_int64
        L.e8_code_lengths.argtypes = [u64p, u8p]
        L.e8_code_lengths.restype = ctypes.c_int
        L.e8_canonical.argtypes = [u8p, ctypes.POINTER(ctypes.c_uint32)]
        L.e8_canonical.restype = None
        L.e8_check_table.argtypes = [u8p]
        L.e8_check_table.restype = ctypes.c_int
        L.e8_decode_prefix.argtypes = [u8p, ctypes.c_uint32, ctypes.POINTER(ctypes.c_int),
                                       ctypes.POINTER(ctypes.c_int)]
        L.e8_decode_prefix.restype = ctypes.c_int
        L.e8_encode_bound.argtypes = [ctypes.c_uint64]
        L.e8_encode_bound.restype = ctypes.c_int64
        L.e8_encode.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_uint64]
        L.e8_encode.restype = ctypes.c_int64
        L.e8_decode.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64]
        L.e8_decode.restype = ctypes.c_int
        L.e8_check_index.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
        L.e8_check_index.restype = ctypes.c_int
        L.e8_n_values.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
        L.e8_n_values.restype = ctypes.c_int64
        L.e8_widen.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                               ctypes.c_void_p]
        L.e8_widen.restype = ctypes.c_int
        _lib = L
    return _lib


def _u8(a) -> np.ndarray:
    return np.ascontiguousarray(np.frombuffer(a, dtype=np.uint8) if isinstance(a, (bytes, bytearray))
                                else a, dtype=np.uint8)


def _p(a: np.ndarray, t=ctypes.c_uint8):
    return a.ctypes.data_as(ctypes.POINTER(t))


def huffman_depths(counts) -> np.ndarray:
    """Leaf depths of the plain (unlimited) Huffman tree over 256 counts."""
    c = np.zeros(256, np.uint64)
    c[: len(counts)] = counts
    d = np.zeros(256, np.uint8)
    lib().oh_huffman_depths(_p(c, ctypes.c_uint64), _p(d))
    return d


def code_lengths(counts) -> np.ndarray:
    """Encoder code lengths: Huffman depths, clamp, lengthen, repay."""
    c = np.zeros(256, np.uint64)
    c[: len(counts)] = counts
    d = np.zeros(256, np.uint8)
    lib().oh_code_lengths(_p(c, ctypes.c_uint64), _p(d))
    return d


def kraft(lengths) -> int:
    ln = np.zeros(256, np.uint8)
    ln[: len(lengths)] = lengths
    return lib().oh_kraft(_p(ln))


def canonical(lengths) -> np.ndarray:
    ln = np.zeros(256, np.uint8)
    ln[: len(lengths)] = lengths
    c = np.zeros(256, np.uint32)
    lib().oh_canonical(_p(ln), _p(c, ctypes.c_uint32))
    return c


def check_table(lengths) -> int:
    ln = np.zeros(256, np.uint8)
    ln[: len(lengths)] = lengths
    return lib().oh_check_table(_p(ln))


def decode_prefix(lengths, bits12: int):
    """(symbol, code length) of the code that prefixes the 12-bit string, or None."""
    ln = np.zeros(256, np.uint8)
    ln[: len(lengths)] = lengths
    s, l = ctypes.c_int(), ctypes.c_int()
    if lib().oh_decode_prefix(_p(ln), bits12, ctypes.byref(s), ctypes.byref(l)) < 0:
        return None
    return s.value, l.value


def encode_bound(raw_bytes: int, lane_syms: int = 256) -> int:
    n = lib().oh_encode_bound_lanes(raw_bytes, lane_syms)
    if n < 0:
        raise ValueError("oracle encode bound: lane_syms %d" % lane_syms)
    return n


def encode_layer(raw, lane_syms: int = 256) -> np.ndarray:
    """Container bytes (uint8 array) for one layer of bf16 bytes, with lane
    chunks of lane_syms symbols (256, or 64)."""
    r = _u8(raw)
    cap = encode_bound(r.size, lane_syms)
    out = np.empty(cap, np.uint8)
    n = lib().oh_encode_layer_lanes(r.ctypes.data, r.size, lane_syms, out.ctypes.data, cap)
    if n < 0:
        raise ValueError("oracle encode failed: %d" % n)
    return out[:n]


def decode_layer(blob) -> np.ndarray:
    b = _u8(blob)
    raw = lib().oh_raw_bytes(b.ctypes.data, b.size)
    if raw < 0:
        raise ValueError("oracle: bad container header: %d" % raw)
    out = np.empty(raw, np.uint8)
    rc = lib().oh_decode_layer(b.ctypes.data, b.size, out.ctypes.data, raw)
    if rc:
        raise ValueError("oracle decode failed: %d" % rc)
    return out


def decode_layer_rc(blob) -> int:
    """Status code of a full decode (0 or a negative error), output discarded."""
    b = _u8(blob)
    raw = lib().oh_raw_bytes(b.ctypes.data, b.size)
    if raw < 0:
        return int(raw)
    out = np.empty(raw, np.uint8)
    return lib().oh_decode_layer(b.ctypes.data, b.size, out.ctypes.data, raw)


def decode_stripes(blob, first: int, count: int, out_cap: int) -> np.ndarray:
    b = _u8(blob)
    out = np.empty(out_cap, np.uint8)
    rc = lib().oh_decode_stripes(b.ctypes.data, b.size, first, count, out.ctypes.data, out_cap)
    if rc:
        raise ValueError("oracle stripe decode failed: %d" % rc)
    return out


def check_index(blob) -> int:
    b = _u8(blob)
    return lib().oh_check_index(b.ctypes.data, b.size)


# ---------------------------------------------------------------------------
# FP8 exponent codec (e8huf_oracle.c)

E8_MAXLEN = 16


def _len32(lengths) -> np.ndarray:
    ln = np.zeros(32, np.uint8)
    ln[: len(lengths)] = lengths
    return ln


def e8_code_lengths(counts):
    """(code lengths[32], smoothing rounds) for up to 32 exponent counts."""
    c = np.zeros(32, np.uint64)
    c[: len(counts)] = counts
    d = np.zeros(32, np.uint8)
    rounds = lib().e8_code_lengths(_p(c, ctypes.c_uint64), _p(d))
    return d, rounds


def e8_kraft(lengths) -> int:
    return lib().e8_kraft(_p(_len32(lengths)))


def e8_canonical(lengths) -> np.ndarray:
    c = np.zeros(32, np.uint32)
    lib().e8_canonical(_p(_len32(lengths)), _p(c, ctypes.c_uint32))
    return c


def e8_check_table(lengths) -> int:
    return lib().e8_check_table(_p(_len32(lengths)))


def e8_decode_prefix(lengths, bits16: int):
    """(symbol, code length) of the code that prefixes the 16-bit string, or None."""
    s, l = ctypes.c_int(), ctypes.c_int()
    if lib().e8_decode_prefix(_p(_len32(lengths)), bits16, ctypes.byref(s), ctypes.byref(l)) < 0:
        return None
    return s.value, l.value


def e8_encode(x, exp_bits: int = 4) -> np.ndarray:
    """Container bytes for FP8 bytes x (E4M3: exp_bits 4, E5M2: 5)."""
    r = _u8(x)
    cap = lib().e8_encode_bound(r.size)
    if cap < 0:
        raise ValueError("oracle e8 encode: bad size")
    out = np.empty(cap, np.uint8)
    n = lib().e8_encode(r.ctypes.data, r.size, exp_bits, out.ctypes.data, cap)
    if n < 0:
        raise ValueError("oracle e8 encode failed: %d" % n)
    return out[:n]


def e8_decode(blob) -> np.ndarray:
    b = _u8(blob)
    n = lib().e8_n_values(b.ctypes.data, b.size)
    if n < 0:
        raise ValueError("oracle e8: bad container header: %d" % n)
    out = np.empty(n, np.uint8)
    rc = lib().e8_decode(b.ctypes.data, b.size, out.ctypes.data, n)
    if rc:
        raise ValueError("oracle e8 decode failed: %d" % rc)
    return out


def e8_decode_rc(blob) -> int:
    b = _u8(blob)
    n = lib().e8_n_values(b.ctypes.data, b.size)
    if n < 0:
        return int(n)
    out = np.empty(n, np.uint8)
    return lib().e8_decode(b.ctypes.data, b.size, out.ctypes.data, n)


def e8_check_index(blob) -> int:
    b = _u8(blob)
    return lib().e8_check_index(b.ctypes.data, b.size)


E8_OUT_BF16, E8_OUT_F16 = 1, 2


def e8_widen(x, exp_bits: int, scale: float, out_kind: int) -> np.ndarray:
    """16-bit output words (bfloat16: out_kind 1, IEEE half: 2) of
    value(x[i]) * scale in single precision, rounded to nearest even."""
    r = _u8(x)
    out = np.empty(r.size, np.uint16)
    rc = lib().e8_widen(r.ctypes.data, r.size, exp_bits, float(scale), out_kind, out.ctypes.data)
    if rc:
        raise ValueError("oracle e8 widen: bad arguments (%d)" % rc)
    return out
