"""CPU-side checks of the C-ABI library: it loads, exports what include/k3huf.h
declares, and its host functions (decode-table build, header parse, packer)
agree with the oracle. No GPU compute is called here."""

import os
import re

import numpy as np
import pytest

import oracle as O
from goldens import limiter_goldens
from lossless_huffman_decoding_amd import k3huf, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    txt = open(os.path.join(ROOT, "include", "k3huf.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(k3huf_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = k3huf.lib()
    names = _declared_functions()
    assert set(names) == set(k3huf.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def _tables():
    rng = np.random.default_rng(11)
    yield [1]                                  # lone symbol (Kraft 2048)
    yield [1, 1]
    yield [2, 2, 2]                            # under-full, prefix-free
    yield [8] * 256
    yield list(O.code_lengths(synth._fibonacci(40)))
    for _ in range(40):
        n = int(rng.integers(2, 257))
        counts = np.zeros(256, np.int64)
        idx = rng.permutation(256)[:n]
        counts[idx] = np.maximum(1, rng.geometric(rng.uniform(0.05, 0.5), n) ** 3)
        yield list(O.code_lengths(counts))


def test_build_table_matches_oracle_bit_by_bit_decode():
    """Every one of the 4096 slots equals the oracle's bit-by-bit decode of
    that 12-bit string (symbol << 4 | length), or 0 where no code applies."""
    for lens in _tables():
        lut = k3huf.build_table(lens)
        want = np.zeros(4096, np.uint16)
        for i in range(4096):
            r = O.decode_prefix(lens, i)
            if r is not None:
                want[i] = (r[0] << 4) | r[1]
        assert (lut == want).all(), lens[:16]


def test_build_table_rejections_match_page_rules():
    assert k3huf.build_table_rc([0] * 256) == k3huf.E_EMPTY
    assert k3huf.build_table_rc([1, 1, 1]) == k3huf.E_OVERSUB
    assert k3huf.build_table_rc([13, 1]) == k3huf.E_BADLEN
    assert k3huf.build_table_rc([1, 2]) == k3huf.E_OVERLAP
    for lens in ([1, 1, 1], [13, 1], [1, 2], [0] * 256, [1], [2, 2, 2]):
        rc = k3huf.build_table_rc(lens)
        orc = O.check_table(lens)
        assert (rc == 0) == (orc == 0)
    with pytest.raises(k3huf.K3HufError):
        k3huf.build_table([1, 1, 1])


def test_layer_info_parses_oracle_container():
    x = synth.small_random(3, 3 * 65536 + 514)
    blob = O.encode_layer(x)
    info = k3huf.layer_info(blob)
    assert info["raw_bytes"] == x.size
    assert info["container_bytes"] == blob.size
    assert info["n_stripes"] == 1 and info["n_subblocks"] == 4
    bad = blob.copy()
    bad[0] ^= 1
    with pytest.raises(k3huf.K3HufError):
        k3huf.layer_info(bad)
    bad = blob.copy()
    bad[26] ^= 0x10                                 # raw_bytes no longer matches n_subblocks
    with pytest.raises(k3huf.K3HufError):
        k3huf.layer_info(bad)


@pytest.mark.parametrize("n_bytes", [2, 1026, 65536, 3 * 65536 + 514])
def test_packer_matches_oracle_encoder(n_bytes):
    x = synth.small_random(n_bytes + 7, n_bytes)
    a = O.encode_layer(x)
    b = k3huf.encode_layer(x)
    assert a.size == b.size and (a == b).all()
    assert O.check_index(b) == O.OK


def test_packer_edge_layers_decode_with_oracle():
    for name, gen in synth.CONFIGS["edge"]:
        x = gen()
        b = k3huf.encode_layer(x)
        assert O.check_index(b) == O.OK, name
        assert (O.decode_layer(b) == x).all(), name
        a = O.encode_layer(x)
        assert a.size == b.size and (a == b).all(), name


def test_packer_mixed_spans_matches_oracle():
    x = synth.mixed_spans(77, (8 << 20) + 2 * 65536 + 118)
    a = O.encode_layer(x)
    b = k3huf.encode_layer(x)
    assert a.size == b.size and (a == b).all()


def _layer_with_counts(counts, seed):
    """bf16 layer bytes whose odd (high) bytes hold symbol v exactly counts[v]
    times, in a seeded order; even bytes seeded at random."""
    rng = np.random.default_rng(seed)
    odd = rng.permutation(np.repeat(np.arange(len(counts), dtype=np.uint8), counts))
    x = np.empty(2 * odd.size, np.uint8)
    x[1::2] = odd
    x[0::2] = rng.integers(0, 256, odd.size, dtype=np.uint8)
    return x


def test_packer_code_lengths_match_limiter_goldens():
    """The native packer's codelen[256] (as written into its container header)
    equals the hand-derived length-limit cases of tests/golden/limiter_cases.txt,
    and so does the oracle's (K3 page, section "canonical code assignment and
    Kraft check")."""
    for i, (name, counts, want) in enumerate(limiter_goldens()):
        x = _layer_with_counts(counts, 500 + i)
        b = k3huf.encode_layer(x)
        got = k3huf.layer_info(b)["codelen"]
        assert list(got[: len(counts)]) == want, name
        assert (got[len(counts):] == 0).all(), name
        a = O.encode_layer(x)
        assert a.size == b.size and (a == b).all(), name
        assert (O.decode_layer(b) == x).all(), name


def test_packer_bad_args():
    assert k3huf.lib().k3huf_encode_bound(3) == k3huf.E_ARG
    assert k3huf.lib().k3huf_encode_bound(0) == k3huf.E_ARG
    assert k3huf.encode_bound(2) == O.encode_bound(2)


def test_decode_layer_rejects_bad_arguments_before_any_device_call():
    """The launcher validates sizes and alignment on the host and returns
    K3HUF_E_ARG without touching the device (so this runs without a GPU).
    The pointers are never dereferenced on these paths."""
    raw = k3huf.decode_layer_raw
    blob, lut, out = 1 << 20, 1 << 21, 1 << 22          # 16-byte aligned fake addresses
    good = 304 + 8
    assert raw(0, good, lut, out, 2, 0, None) == k3huf.E_ARG              # null blob
    assert raw(blob, good, 0, out, 2, 0, None) == k3huf.E_ARG             # null table
    assert raw(blob, good, lut, 0, 2, 0, None) == k3huf.E_ARG             # null output
    assert raw(blob + 8, good, lut, out, 2, 0, None) == k3huf.E_ARG       # blob not 16-aligned
    assert raw(blob, good, lut, out + 4, 2, 0, None) == k3huf.E_ARG       # output not 16-aligned
    assert raw(blob, good, lut + 1, out, 2, 0, None) == k3huf.E_ARG       # table not 2-aligned
    assert raw(blob, good, lut, out, 3, 0, None) == k3huf.E_ARG           # odd raw size
    assert raw(blob, good, lut, out, 0, 0, None) == k3huf.E_ARG           # empty layer
    assert raw(blob, 303, lut, out, 2, 0, None) == k3huf.E_ARG            # shorter than a header
    # 3 stripes need 3 stripe offsets after the 304-byte header
    three = 2 * (1 << 26) + 2
    assert raw(blob, 304 + 16, lut, out, three, 0, None) == k3huf.E_ARG
    # offsets are kept in 16-byte units by the kernel: blobs stop below 64 GiB
    assert raw(blob, 1 << 36, lut, out, 2, 0, None) == k3huf.E_ARG
    # a blob holds its layer's even plane (raw / 2 bytes): no blob of 1 KiB
    # decodes to 4 KiB
    assert raw(blob, 1024, lut, out, 4096, 0, None) == k3huf.E_ARG


def test_host_ring_rejects_bad_arguments_before_any_device_call():
    """k3huf_decode_ring_host checks counts, sizes and alignment on the host
    and returns K3HUF_E_ARG before creating events or queuing work (so this
    runs without a GPU; no pointer is dereferenced on these paths)."""
    import ctypes
    L = k3huf.lib()
    vp = ctypes.c_void_p
    lay = (k3huf.HostLayer * 1)(k3huf.HostLayer(1 << 20, 4096, 1 << 21, 8192))
    stage = (vp * 2)(1 << 24, 1 << 25)
    slots = (vp * 2)(1 << 26, 1 << 27)
    streams = (vp * 1)(None)
    cb = k3huf.RING_CB()

    def call(layers=lay, n=1, st=stage, n_st=2, st_bytes=4096, sl=slots, n_sl=2, sl_bytes=8192,
             strm=streams, n_strm=1):
        return L.k3huf_decode_ring_host(layers, n, st, n_st, st_bytes, sl, n_sl, sl_bytes, None,
                                        strm, n_strm, cb, None, None)
    assert call(layers=None) == k3huf.E_ARG
    assert call(n=-1) == k3huf.E_ARG
    assert call(n_st=0) == k3huf.E_ARG
    assert call(n_sl=0) == k3huf.E_ARG
    assert call(n_strm=0) == k3huf.E_ARG
    assert call(st_bytes=4095) == k3huf.E_ARG               # container larger than a stage
    assert call(sl_bytes=8190) == k3huf.E_ARG               # layer larger than a slot
    assert call(st=(vp * 2)(1 << 24, (1 << 25) + 8)) == k3huf.E_ARG   # stage not 16-aligned
    assert call(st=(vp * 2)(1 << 24, None)) == k3huf.E_ARG
    assert call(sl=(vp * 2)(None, 1 << 27)) == k3huf.E_ARG
    assert call(layers=(k3huf.HostLayer * 1)(k3huf.HostLayer(None, 4096, 1 << 21, 8192))) == k3huf.E_ARG
    assert call(layers=(k3huf.HostLayer * 1)(k3huf.HostLayer(1 << 20, 4096, None, 8192))) == k3huf.E_ARG


def test_gpu_encoder_rejects_bad_arguments_before_any_device_call():
    """k3huf_encode_layer_dev validates sizes, alignment and capacities on the
    host before any HIP call (so this runs without a GPU)."""
    L = k3huf.lib()
    raw, out, work = 1 << 20, 1 << 24, 1 << 28     # 16-byte aligned fake addresses
    n = 3 * 65536 + 514
    cap, wb = k3huf.encode_bound(n), k3huf.encode_work_bytes(n)
    assert L.k3huf_encode_work_bytes(3) == k3huf.E_ARG
    assert L.k3huf_encode_work_bytes(0) == k3huf.E_ARG
    f = L.k3huf_encode_layer_dev
    assert f(None, n, out, cap, work, wb, None) == k3huf.E_ARG
    assert f(raw, n, None, cap, work, wb, None) == k3huf.E_ARG
    assert f(raw, n, out, cap, None, wb, None) == k3huf.E_ARG
    assert f(raw, n + 1, out, cap, work, wb, None) == k3huf.E_ARG       # odd size
    assert f(raw, 0, out, cap, work, wb, None) == k3huf.E_ARG
    assert f(raw + 8, n, out, cap, work, wb, None) == k3huf.E_ARG       # misaligned input
    assert f(raw, n, out + 4, cap, work, wb, None) == k3huf.E_ARG       # misaligned output
    assert f(raw, n, out, cap - 1, work, wb, None) == k3huf.E_ARG       # output too small
    assert f(raw, n, out, cap, work, wb - 1, None) == k3huf.E_ARG       # work too small


def test_static_gpu_encoder_rejects_bad_arguments_before_any_device_call():
    """k3huf_encode_layer_dev_static checks sizes (including its
    K3HUF_STATIC_MAX_RAW limit), alignment and capacity on the host before
    any HIP call (so this runs without a GPU)."""
    L = k3huf.lib()
    raw, out = 1 << 20, 1 << 24
    f = L.k3huf_encode_layer_dev_static
    n = k3huf.STATIC_MAX_RAW + 2
    assert f(raw, n, out, k3huf.encode_bound(n), None) == k3huf.E_ARG     # above the limit
    n = 3 * 65536 + 514
    cap = k3huf.encode_bound(n)
    assert f(None, n, out, cap, None) == k3huf.E_ARG
    assert f(raw, n, None, cap, None) == k3huf.E_ARG
    assert f(raw, n + 1, out, cap, None) == k3huf.E_ARG                   # odd size
    assert f(raw, 0, out, cap, None) == k3huf.E_ARG
    assert f(raw + 8, n, out, cap, None) == k3huf.E_ARG                   # misaligned input
    assert f(raw, n, out + 4, cap, None) == k3huf.E_ARG                   # misaligned output
    assert f(raw, n, out, cap - 1, None) == k3huf.E_ARG                   # output too small


def test_packer_fuzz_matches_oracle():
    """The native packer against the oracle's encoder on the seeded random
    sweep of the GPU tests (random sizes and high-byte laws)."""
    for seed in range(48):
        x, what = synth.fuzz_layer(seed)
        a = O.encode_layer(x)
        b = k3huf.encode_layer(x)
        assert a.size == b.size and (a == b).all(), (seed, what)
        assert O.check_index(b) == O.OK, (seed, what)


def test_stream_ref_rejects_bad_arguments_before_any_device_call():
    """The bandwidth reference kernel's launcher checks its arguments first:
    these calls return K3HUF_E_ARG without touching a device."""
    L = k3huf.lib()
    good = 1 << 12   # a 4 KiB-aligned fake address; never dereferenced here
    assert L.k3huf_stream_ref(good, 16, None, 16, 1, 0, None) == k3huf.E_ARG        # no output
    assert L.k3huf_stream_ref(None, 16, good, 16, 1, 0, None) == k3huf.E_ARG        # input bytes, no input
    assert L.k3huf_stream_ref(good, 16, good, 0, 1, 0, None) == k3huf.E_ARG         # empty output
    assert L.k3huf_stream_ref(good, 24, good, 16, 1, 0, None) == k3huf.E_ARG        # not whole units
    assert L.k3huf_stream_ref(good, 16, good, 40, 1, 0, None) == k3huf.E_ARG
    assert L.k3huf_stream_ref(good + 8, 16, good, 16, 1, 0, None) == k3huf.E_ARG    # misaligned
    assert L.k3huf_stream_ref(good, 16, good + 4, 16, 1, 0, None) == k3huf.E_ARG
    assert L.k3huf_stream_ref(good, 16, good, 16, 0, 0, None) == k3huf.E_ARG        # grid
    assert L.k3huf_stream_ref(good, 16, good, 16, (1 << 20) + 1, 0, None) == k3huf.E_ARG


@pytest.mark.parametrize("n_bytes", [2, 130, 16382, 16384, 16386, 3 * 16384 + 514, (1 << 20) + 6,
                                     (1 << 26) + 3 * 16384 + 66])
def test_packer_short_lane_chunks_equal_oracle(n_bytes):
    """The host packer's 64-symbol lane-chunk layout equals the oracle's
    container byte for byte, and layer_info reports its geometry."""
    x = synth.small_random(n_bytes + 5, n_bytes)
    got = k3huf.encode_layer(x, lane_syms=64)
    want = O.encode_layer(x, 64)
    assert got.size == want.size and (got == want).all()
    info = k3huf.layer_info(got)
    assert info["lane_syms"] == 64 and info["n_subblocks"] == -(-n_bytes // 16384)
    assert k3huf.layer_info(k3huf.encode_layer(x))["lane_syms"] == 256
    assert k3huf.encode_bound(n_bytes, 64) == O.encode_bound(n_bytes, 64) >= got.size


def test_lane_syms_other_than_64_or_256_rejected():
    x = synth.small_random(6, 4096)
    L = k3huf.lib()
    for bad in (0, 32, 128, 512):
        assert L.k3huf_encode_bound_lanes(x.size, bad) == k3huf.E_ARG
        with pytest.raises(k3huf.K3HufError):
            k3huf.encode_layer(x, lane_syms=bad)
    blob = k3huf.encode_layer(x, lane_syms=64).copy()
    blob[16:20] = np.frombuffer(np.uint32(128).tobytes(), np.uint8)   # lane_syms 128
    with pytest.raises(k3huf.K3HufError):
        k3huf.layer_info(blob)


def test_lane_syms_for_layer_sizes():
    assert k3huf.lane_syms_for(2) == 64
    assert k3huf.lane_syms_for(16 << 20) == 64
    assert k3huf.lane_syms_for((16 << 20) + 2) == 256
    assert k3huf.lane_syms_for(1_170_000_000) == 256


def test_gpu_packer_lane_syms_checked_before_any_device_call():
    L = k3huf.lib()
    good = 1 << 12
    for bad in (0, 32, 128):
        assert L.k3huf_encode_work_bytes_lanes(1024, bad) == k3huf.E_ARG
        assert L.k3huf_encode_layer_dev_lanes(good, 1024, bad, good, 1 << 20, good, 1 << 20, None) == k3huf.E_ARG
    assert k3huf.encode_work_bytes(1 << 20, 64) > k3huf.encode_work_bytes(1 << 20)


def test_bindings_refuse_host_and_short_tensors_before_any_device_call():
    """The Python calls hand tensors to the kernels as device pointers: host
    tensors, strided views, a table shorter than 4096 entries and tables of
    other than 16-bit elements are refused with ValueError before the
    library is called (CPU tensors here, so nothing reaches a GPU)."""
    import torch
    from lossless_huffman_decoding_amd import e8huf
    blob = torch.zeros(4096, dtype=torch.uint8)
    lut = torch.zeros(4096, dtype=torch.int16)
    out = torch.zeros(4096, dtype=torch.uint8)
    st = torch.zeros(1, dtype=torch.int32)
    for call in (lambda: k3huf.decode_layer(blob, lut, out, st),
                 lambda: k3huf.decode_ring([(blob, lut, 4096)], [out], [None]),
                 lambda: k3huf.stream_ref(blob, out, 1),
                 lambda: k3huf.encode_layer_dev(blob, out, out),
                 lambda: k3huf.encode_layer_dev_static(blob, out),
                 lambda: e8huf.decode(blob, lut, out, st),
                 lambda: e8huf.decode_widen(blob, lut, out.view(torch.int16), out_kind=e8huf.OUT_BF16)):
        with pytest.raises(ValueError, match="GPU tensor"):
            call()
    # the checks themselves, on stand-ins that report a GPU device
    class Fake:
        def __init__(self, n, elem=1, contiguous=True):
            self.is_cuda, self.n, self.elem, self.c = True, n, elem, contiguous

        def is_contiguous(self):
            return self.c

        def element_size(self):
            return self.elem

        def numel(self):
            return self.n
    with pytest.raises(ValueError, match="at least 8192 bytes"):
        k3huf._dev(Fake(4095, 2), "d_lut", 2 * k3huf.LUT_ENTRIES)
    with pytest.raises(ValueError, match="contiguous"):
        k3huf._dev(Fake(4096, 2, contiguous=False), "d_lut", 2 * k3huf.LUT_ENTRIES)
    with pytest.raises(ValueError, match="elements of 2 bytes"):
        k3huf._dev(Fake(8192, 1), "d_lut", elem=2)
    with pytest.raises(ValueError, match="at least 4 bytes"):
        k3huf._status(Fake(3, 1))
    k3huf._dev(Fake(4096, 2), "d_lut", 2 * k3huf.LUT_ENTRIES, elem=2)
