"""Thin Python binding of libk3huf.so (ctypes): argument marshalling only.

Every step of decoding runs in the library's HIP kernels; this module only
passes pointers, sizes and stream handles. PyTorch supplies device memory and
streams. If the library has not been built, every call raises -- there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libk3huf.so")

OK = 0
HDR_BYTES = 304   # layer header size (K3HUF_HDR_BYTES)
LUT_ENTRIES = 4096   # decode table entries (K3HUF_LUT_ENTRIES)
E_ARG, E_EMPTY, E_OVERSUB, E_BADLEN, E_OVERLAP, E_FORMAT, E_CORRUPT, E_HIP = range(-1, -9, -1)
DEV_HEADER, DEV_STRIPE, DEV_INDEX, DEV_CODE, DEV_LANE_END = 1, 2, 4, 8, 16

# names the C header declares, checked by the ABI test
EXPORTS = ("k3huf_build_table", "k3huf_layer_info", "k3huf_decode_layer", "k3huf_decode_ring",
           "k3huf_decode_ring_host", "k3huf_encode_bound", "k3huf_encode_layer",
           "k3huf_encode_bound_lanes", "k3huf_encode_layer_lanes", "k3huf_lane_syms_for",
           "k3huf_encode_work_bytes", "k3huf_encode_layer_dev", "k3huf_encode_work_bytes_lanes",
           "k3huf_encode_layer_dev_lanes", "k3huf_encode_layer_dev_static",
           "k3huf_stream_ref", "k3huf_strerror")
STATIC_MAX_RAW = 1 << 32   # K3HUF_STATIC_MAX_RAW


class K3HufError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s: %s (%d)" % (what, strerror(code) if _lib else "error", code))


class Info(ctypes.Structure):
    _fields_ = [("raw_bytes", ctypes.c_uint64), ("container_bytes", ctypes.c_uint64),
                ("n_stripes", ctypes.c_uint32), ("n_subblocks", ctypes.c_uint32),
                ("codelen", ctypes.c_uint8 * 256), ("lane_syms", ctypes.c_uint32)]


class RingLayer(ctypes.Structure):
    _fields_ = [("d_blob", ctypes.c_void_p), ("blob_bytes", ctypes.c_size_t),
                ("d_lut", ctypes.c_void_p), ("raw_bytes", ctypes.c_size_t)]


class HostLayer(ctypes.Structure):
    _fields_ = [("h_blob", ctypes.c_void_p), ("blob_bytes", ctypes.c_size_t),
                ("d_lut", ctypes.c_void_p), ("raw_bytes", ctypes.c_size_t)]


RING_CB = ctypes.CFUNCTYPE(None, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                           ctypes.c_void_p)

_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libk3huf.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.k3huf_build_table.argtypes = [vp, vp]
        L.k3huf_build_table.restype = ctypes.c_int
        L.k3huf_layer_info.argtypes = [vp, sz, ctypes.POINTER(Info)]
        L.k3huf_layer_info.restype = ctypes.c_int
        L.k3huf_decode_layer.argtypes = [vp, sz, vp, vp, sz, vp, vp]
        L.k3huf_decode_layer.restype = ctypes.c_int
        L.k3huf_decode_ring.argtypes = [ctypes.POINTER(RingLayer), ctypes.c_int,
                                        ctypes.POINTER(vp), ctypes.c_int, sz,
                                        ctypes.POINTER(vp), ctypes.c_int, RING_CB, vp, vp]
        L.k3huf_decode_ring.restype = ctypes.c_int
        L.k3huf_decode_ring_host.argtypes = [ctypes.POINTER(HostLayer), ctypes.c_int,
                                             ctypes.POINTER(vp), ctypes.c_int, sz,
                                             ctypes.POINTER(vp), ctypes.c_int, sz, vp,
                                             ctypes.POINTER(vp), ctypes.c_int, RING_CB, vp, vp]
        L.k3huf_decode_ring_host.restype = ctypes.c_int
        L.k3huf_encode_bound.argtypes = [ctypes.c_uint64]
        L.k3huf_encode_bound.restype = ctypes.c_int64
        L.k3huf_encode_layer.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_uint64, ctypes.c_int]
        L.k3huf_encode_layer.restype = ctypes.c_int64
        L.k3huf_encode_bound_lanes.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
        L.k3huf_encode_bound_lanes.restype = ctypes.c_int64
        L.k3huf_encode_layer_lanes.argtypes = [vp, ctypes.c_uint64, ctypes.c_uint32, vp, ctypes.c_uint64,
                                               ctypes.c_int]
        L.k3huf_encode_layer_lanes.restype = ctypes.c_int64
        L.k3huf_lane_syms_for.argtypes = [ctypes.c_uint64]
        L.k3huf_lane_syms_for.restype = ctypes.c_uint32
        L.k3huf_encode_work_bytes.argtypes = [ctypes.c_uint64]
        L.k3huf_encode_work_bytes.restype = ctypes.c_int64
        L.k3huf_encode_layer_dev.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_uint64, vp,
                                             ctypes.c_uint64, vp]
        L.k3huf_encode_layer_dev.restype = ctypes.c_int64
        L.k3huf_encode_work_bytes_lanes.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
        L.k3huf_encode_work_bytes_lanes.restype = ctypes.c_int64
        L.k3huf_encode_layer_dev_lanes.argtypes = [vp, ctypes.c_uint64, ctypes.c_uint32, vp, ctypes.c_uint64, vp,
                                                   ctypes.c_uint64, vp]
        L.k3huf_encode_layer_dev_lanes.restype = ctypes.c_int64
        L.k3huf_encode_layer_dev_static.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_uint64, vp]
        L.k3huf_encode_layer_dev_static.restype = ctypes.c_int64
        L.k3huf_stream_ref.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                       vp]
        L.k3huf_stream_ref.restype = ctypes.c_int
        L.k3huf_strerror.argtypes = [ctypes.c_int]
        L.k3huf_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().k3huf_strerror(code).decode()


def _check(rc: int, what: str) -> int:
    if rc < 0:
        raise K3HufError(int(rc), what)
    return rc


def _u8(a) -> np.ndarray:
    if isinstance(a, (bytes, bytearray, memoryview)):
        return np.frombuffer(a, dtype=np.uint8)
    return np.ascontiguousarray(a, dtype=np.uint8)


def build_table(codelen) -> np.ndarray:
    """4096-entry u16 decode table ((symbol << 4) | length) for codelen[256]."""
    cl = np.zeros(256, np.uint8)
    c = np.asarray(codelen, dtype=np.uint8)
    cl[: c.size] = c
    lut = np.zeros(4096, np.uint16)
    _check(lib().k3huf_build_table(cl.ctypes.data, lut.ctypes.data), "k3huf_build_table")
    return lut


def build_table_rc(codelen) -> int:
    """Return code of k3huf_build_table (0 or a negative error)."""
    cl = np.zeros(256, np.uint8)
    c = np.asarray(codelen, dtype=np.uint8)
    cl[: c.size] = c
    lut = np.zeros(4096, np.uint16)
    return lib().k3huf_build_table(cl.ctypes.data, lut.ctypes.data)


def layer_info(blob) -> dict:
    b = _u8(blob)
    info = Info()
    _check(lib().k3huf_layer_info(b.ctypes.data, b.size, ctypes.byref(info)), "k3huf_layer_info")
    return dict(raw_bytes=info.raw_bytes, container_bytes=info.container_bytes,
                n_stripes=info.n_stripes, n_subblocks=info.n_subblocks,
                codelen=np.frombuffer(bytes(info.codelen), np.uint8).copy(), lane_syms=info.lane_syms)


def encode_bound(raw_bytes: int, lane_syms: int = 256) -> int:
    return _check(lib().k3huf_encode_bound_lanes(raw_bytes, lane_syms), "k3huf_encode_bound_lanes")


def lane_syms_for(raw_bytes: int) -> int:
    """The lane-chunk length the library picks for a layer of raw_bytes
    (k3huf_lane_syms_for: 64 up to 16 MiB, else 256)."""
    return int(lib().k3huf_lane_syms_for(raw_bytes))


def encode_layer(raw, n_threads: int = 0, lane_syms: int = 256) -> np.ndarray:
    """Pack one bf16 layer (bytes) into a container (numpy uint8) with lane
    chunks of lane_syms symbols (256, or 64 for small layers)."""
    r = _u8(raw)
    cap = encode_bound(r.size, lane_syms)
    out = np.empty(cap, np.uint8)
    n = _check(lib().k3huf_encode_layer_lanes(r.ctypes.data, r.size, lane_syms, out.ctypes.data, cap,
                                              n_threads), "k3huf_encode_layer_lanes")
    return out[:n]


def encode_work_bytes(raw_bytes: int, lane_syms: int = 256) -> int:
    return _check(lib().k3huf_encode_work_bytes_lanes(raw_bytes, lane_syms), "k3huf_encode_work_bytes_lanes")


def encode_layer_dev(d_raw, d_out=None, d_work=None, stream=None, lane_syms: int = 256):
    """Pack the bf16 layer in device uint8 tensor ``d_raw`` on the GPU, with
    lane chunks of lane_syms symbols (256, or 64). ``d_out`` (device uint8, at
    least encode_bound bytes) and ``d_work`` (device uint8, at least
    encode_work_bytes) are allocated when None. Returns the container as a
    view of d_out (synchronous call)."""
    import torch
    n = _nbytes(_dev(d_raw, "d_raw"))
    if d_out is None:
        d_out = torch.empty(encode_bound(n, lane_syms), dtype=torch.uint8, device=d_raw.device)
    if d_work is None:
        d_work = torch.empty(encode_work_bytes(n, lane_syms), dtype=torch.uint8, device=d_raw.device)
    _dev(d_out, "d_out")
    _dev(d_work, "d_work")
    size = _check(lib().k3huf_encode_layer_dev_lanes(d_raw.data_ptr(), n, lane_syms, d_out.data_ptr(),
                                                     _nbytes(d_out), d_work.data_ptr(), _nbytes(d_work),
                                                     _stream_handle(stream)), "k3huf_encode_layer_dev_lanes")
    return d_out[:size]


def encode_layer_dev_static(d_raw, d_out=None, stream=None):
    """The GPU packer without allocation inside the library (its work buffer
    and host staging are library-owned arrays; layers up to STATIC_MAX_RAW
    bytes). ``d_out`` is allocated here when None. Returns the container as a
    view of d_out (synchronous call)."""
    import torch
    n = _nbytes(_dev(d_raw, "d_raw"))
    if d_out is None:
        d_out = torch.empty(encode_bound(n), dtype=torch.uint8, device=d_raw.device)
    _dev(d_out, "d_out")
    size = _check(lib().k3huf_encode_layer_dev_static(d_raw.data_ptr(), n, d_out.data_ptr(),
                                                      _nbytes(d_out), _stream_handle(stream)),
                  "k3huf_encode_layer_dev_static")
    return d_out[:size]


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _dev(t, what: str, min_bytes: int = 0, elem: int = 0):
    """Check a tensor handed to a kernel as a device pointer: a contiguous
    GPU tensor of at least min_bytes (and elements of elem bytes when
    given). The library reads or writes exactly what the call's sizes say,
    so a host tensor, a strided view or a short buffer is refused here."""
    if not getattr(t, "is_cuda", False):
        raise ValueError("%s: a GPU tensor is needed (got %s)" % (what, getattr(t, "device", type(t).__name__)))
    if not t.is_contiguous():
        raise ValueError("%s: a contiguous tensor is needed" % what)
    if elem and t.element_size() != elem:
        raise ValueError("%s: elements of %d bytes are needed (got %d)" % (what, elem, t.element_size()))
    if _nbytes(t) < min_bytes:
        raise ValueError("%s: at least %d bytes are needed (got %d)" % (what, min_bytes, _nbytes(t)))
    return t


def _status(d_status):
    return _dev(d_status, "d_status", 4).data_ptr() if d_status is not None else None


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def decode_layer(d_blob, d_lut, d_out, d_status=None, stream=None) -> None:
    """Queue the decode of one layer. Tensors: d_blob uint8 (the blob),
    d_lut 4096 16-bit entries, d_out uint8 of the layer's raw size, d_status
    a 32-bit device word or None. Runs on ``stream`` (default: torch's
    current stream)."""
    _dev(d_blob, "d_blob")
    _dev(d_lut, "d_lut", 2 * LUT_ENTRIES)
    _dev(d_out, "d_out")
    rc = lib().k3huf_decode_layer(
        d_blob.data_ptr(), _nbytes(d_blob), d_lut.data_ptr(),
        d_out.data_ptr(), _nbytes(d_out), _stream_handle(stream), _status(d_status))
    _check(rc, "k3huf_decode_layer")


def decode_layer_raw(blob_ptr: int, blob_bytes: int, lut_ptr: int, out_ptr: int, out_bytes: int,
                     stream: int, status_ptr) -> int:
    """Unchecked pointer-level call; returns the C return code."""
    return lib().k3huf_decode_layer(blob_ptr, blob_bytes, lut_ptr, out_ptr, out_bytes, stream,
                                    status_ptr)


def stream_ref(d_in, d_out, grid: int, nontemporal: bool = False, stream=None) -> None:
    """Queue the streaming reference kernel (k3huf_stream_ref): read all of
    ``d_in`` (uint8 tensor, or None), write all of ``d_out``."""
    if d_in is not None:
        _dev(d_in, "d_in")
    _dev(d_out, "d_out")
    _check(lib().k3huf_stream_ref(d_in.data_ptr() if d_in is not None else None,
                                  _nbytes(d_in) if d_in is not None else 0, d_out.data_ptr(), _nbytes(d_out),
                                  int(grid), int(bool(nontemporal)), _stream_handle(stream)),
           "k3huf_stream_ref")


def decode_ring(layers, slots, streams, cb=None, d_status=None) -> None:
    """Decode ``layers`` (a list of (d_blob, d_lut, raw_bytes)) in order into
    the ring of ``slots`` (uint8 tensors of equal size) on ``streams``. ``cb``
    (optional) is called as cb(k, slot_index, stream_handle) right after layer
    k is queued, to queue its consumer."""
    n = len(layers)
    arr = (RingLayer * max(n, 1))()
    for k, (blob, lut, raw) in enumerate(layers):
        _dev(blob, "layer %d blob" % k)
        _dev(lut, "layer %d table" % k, 2 * LUT_ENTRIES)
        arr[k] = RingLayer(blob.data_ptr(), _nbytes(blob), lut.data_ptr(), raw)
    for i, sl in enumerate(slots):
        _dev(sl, "slot %d" % i)
    slot_ptrs = (ctypes.c_void_p * len(slots))(*[s.data_ptr() for s in slots])
    stream_ptrs = (ctypes.c_void_p * len(streams))(*[_stream_handle(s) for s in streams])
    slot_bytes = min(_nbytes(s) for s in slots)
    c_cb = _ring_cb(cb, slots)
    rc = lib().k3huf_decode_ring(arr, n, slot_ptrs, len(slots), slot_bytes, stream_ptrs,
                                 len(streams), c_cb, None, _status(d_status))
    _check(rc, "k3huf_decode_ring")


def _ring_cb(cb, slots):
    if cb is None:
        return RING_CB()
    index = {s.data_ptr(): i for i, s in enumerate(slots)}

    def _tramp(k, slot, raw, stream, user):
        cb(k, index[slot], stream)
    return RING_CB(_tramp)


def decode_ring_host(layers, stages, slots, copy_stream, streams, cb=None, d_status=None) -> None:
    """The host-fed ring: ``layers`` is a list of (h_blob, d_lut, raw_bytes)
    with h_blob a host uint8 tensor (pinned for overlapped copies); each
    container is copied into stage buffer k % len(stages) (device uint8
    tensors) on ``copy_stream``, then decoded into slot k % len(slots) on
    streams[k % len(streams)]. ``cb`` as for decode_ring."""
    n = len(layers)
    arr = (HostLayer * max(n, 1))()
    for k, (blob, lut, raw) in enumerate(layers):
        if getattr(blob, "is_cuda", True) or not blob.is_contiguous():
            raise ValueError("layer %d blob: a contiguous host tensor is needed" % k)
        _dev(lut, "layer %d table" % k, 2 * LUT_ENTRIES)
        arr[k] = HostLayer(blob.data_ptr(), _nbytes(blob), lut.data_ptr(), raw)
    for i, t in enumerate(list(stages) + list(slots)):
        _dev(t, "stage %d" % i if i < len(stages) else "slot %d" % (i - len(stages)))
    stage_ptrs = (ctypes.c_void_p * len(stages))(*[s.data_ptr() for s in stages])
    slot_ptrs = (ctypes.c_void_p * len(slots))(*[s.data_ptr() for s in slots])
    stream_ptrs = (ctypes.c_void_p * len(streams))(*[_stream_handle(s) for s in streams])
    c_cb = _ring_cb(cb, slots)
    rc = lib().k3huf_decode_ring_host(arr, n, stage_ptrs, len(stages), min(_nbytes(s) for s in stages),
                                      slot_ptrs, len(slots), min(_nbytes(s) for s in slots),
                                      _stream_handle(copy_stream), stream_ptrs, len(streams), c_cb,
                                      None, _status(d_status))
    _check(rc, "k3huf_decode_ring_host")
