"""GPU parity of the FP8 decoder's 16-bit output (e8huf_decode_widen, HIP,
gfx950) against the CPU oracle. ECF8 page (pwwt.cn/news/2030120): FP8
weights (section 1.2) decoded on the GPU, the decoder handing its values over
as 16-bit floats (section 2.2). Expected words come from the oracle's
widening (oracle/e8huf_oracle.c: the FP8 value times the scale in single
precision, rounded to nearest even) of the generated tensor, which the
lossless decode gives back byte for byte. The bar is equality of every
16-bit word; where the oracle's word is a NaN the kernel's must be a NaN (its
payload is not specified). Every case prints its name before touching the
GPU.
"""

import struct

import numpy as np
import pytest
import torch

import oracle as O
from lossless_huffman_decoding_amd import e8huf, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KINDS = {"bf16": e8huf.OUT_BF16, "f16": e8huf.OUT_F16}


def say(*a):
    print("[gpu-case]", *a, flush=True)


def _f32(bits):
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def gpu_widen(blob, kind, scale, n=None, lut=None, prefill=0x5A5A):
    info = e8huf.layer_info(blob) if (n is None or lut is None) else None
    n = info["n_values"] if n is None else n
    lut = e8huf.build_table(info["codelen"], info["exp_bits"]) if lut is None else lut
    d_blob = torch.from_numpy(np.ascontiguousarray(blob)).to(DEV)
    d_lut = torch.from_numpy(np.ascontiguousarray(lut).view(np.int16)).to(DEV)
    d_out = torch.full((n,), prefill, dtype=torch.int16, device=DEV)
    d_status = torch.zeros(1, dtype=torch.int32, device=DEV)
    e8huf.decode_widen(d_blob, d_lut, d_out, out_kind=kind, scale=scale, d_status=d_status)
    torch.cuda.synchronize()
    return d_out.cpu().numpy().view(np.uint16), int(d_status.item())


def is_nan(w, kind):
    w = w.astype(np.uint32)
    ex, fr = (0x7F80, 0x007F) if kind == e8huf.OUT_BF16 else (0x7C00, 0x03FF)
    return ((w & ex) == ex) & ((w & fr) != 0)


def assert_words(got, want, kind):
    nan = is_nan(want, kind)
    assert got.shape == want.shape
    bad = np.flatnonzero((got != want) & ~nan)
    assert bad.size == 0, "first differing words at %s: got %s want %s" % (
        bad[:4], [hex(v) for v in got[bad[:4]]], [hex(v) for v in want[bad[:4]]])
    assert is_nan(got[nan], kind).all()


SIZES = [1, 2, 15, 16, 17, 255, 256, 4095, 16383, 16384, 16385, 3 * 16384 + 77, 64 * 16384 + 5]


@pytest.mark.parametrize("kind", sorted(KINDS))
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("n", SIZES)
def test_widen_sizes(n, fmt, kind):
    """Normal values with a per-tensor amax scale undone by the scale
    argument, at sizes with partial lane chunks, phases and blocks."""
    eb = synth.FP8_EXP_BITS[fmt]
    x = synth.e8_small(n + 31, n, fmt)
    blob = O.e8_encode(x, eb)
    scale = 0.02 / synth.FP8_MAX[fmt]
    say("e8 widen sizes", fmt, kind, n)
    got, st = gpu_widen(blob, KINDS[kind], scale)
    assert st == 0
    assert (O.e8_decode(blob) == x).all()
    assert_words(got, O.e8_widen(x, eb, scale, KINDS[kind]), KINDS[kind])


SCALES = [0x3F800000,   # 1: exact widening
          0xBF400000,   # -0.75
          0x3F808000,   # 1 + 2^-8: bfloat16 ties
          0x3F801000,   # 1 + 2^-11: half ties
          0x00800000,   # 2^-126: subnormal products
          0x1E3CE508,   # 1e-20: half underflow
          0x47000000,   # 2^15: half overflow
          0x7F7FFFFF,   # the largest float: overflow in both
          0x7F800000,   # infinity: 0 * inf is NaN
          0x7FC00000]   # NaN


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_widen_every_byte_and_special_scales(fmt):
    """Uniform random bytes (every FP8 byte, NaN and infinity codes
    included; every block's codes exceed the wave's buffer, so lanes decode
    in passes and the output goes through the checked store path) times
    special scales, into both output kinds."""
    eb = synth.FP8_EXP_BITS[fmt]
    n = 12 * 16384 + 301
    x = synth.e8_uniform_bytes(41 + eb, n)
    blob = O.e8_encode(x, eb)
    for bits in SCALES:
        for kind in sorted(KINDS):
            say("e8 widen specials", fmt, kind, hex(bits))
            got, st = gpu_widen(blob, KINDS[kind], _f32(bits))
            assert st == 0
            assert_words(got, O.e8_widen(x, eb, _f32(bits), KINDS[kind]), KINDS[kind])


@pytest.mark.parametrize("case", ["fib_e5m2", "long_codes_in_passes", "one_exponent"])
def test_widen_edge_tensors(case):
    """Codes of 13-16 bits through the second-level table, long codes in
    passes, and one exponent value (1-bit codes)."""
    n = 40 * 16384 + 123
    x, eb = {"fib_e5m2": (synth.e8_fib_exponents(15, n), 5),
             "long_codes_in_passes": (synth.e8_long_codes_in_passes(16, n), 5),
             "one_exponent": (synth.e8_one_exponent(11, n), 4)}[case]
    blob = O.e8_encode(x, eb)
    for kind in sorted(KINDS):
        say("e8 widen edge", case, kind)
        got, st = gpu_widen(blob, KINDS[kind], 1.0)
        assert st == 0
        assert_words(got, O.e8_widen(x, eb, 1.0, KINDS[kind]), KINDS[kind])


def test_widen_trunk():
    """The FP8 trunk tensor (585,000,000 E4M3 values, the decode bench's
    workload and launch) widened to bfloat16 with a scale: every word against
    the oracle's widening of the generated tensor (each word is a function of
    its byte alone, so the oracle widens the 256 byte values once and the
    expected words are looked up), and the first 2^20 words against the
    oracle's widening of those values directly."""
    x = synth.e8_trunk()
    blob = O.e8_encode(x, 4)
    scale = 0.05 / 448.0
    say("e8 widen trunk", x.size)
    got, st = gpu_widen(blob, e8huf.OUT_BF16, scale)
    assert st == 0
    per_byte = O.e8_widen(np.arange(256, dtype=np.uint8), 4, scale, e8huf.OUT_BF16)
    assert_words(got, per_byte[x], e8huf.OUT_BF16)
    assert_words(got[: 1 << 20], O.e8_widen(x[: 1 << 20], 4, scale, e8huf.OUT_BF16), e8huf.OUT_BF16)


def test_widen_corrupt_header_is_flagged_and_nothing_written():
    x = synth.e8_small(22, 3 * 16384 + 5)
    good = O.e8_encode(x)
    info = e8huf.layer_info(good)
    lut = e8huf.build_table(info["codelen"], 4)
    bad = good.copy()
    bad[0] ^= 0xFF
    say("e8 widen corrupt header")
    got, st = gpu_widen(bad, e8huf.OUT_BF16, 1.0, n=x.size, lut=lut)
    assert st & e8huf.DEV_HEADER and (got == 0x5A5A).all()


def test_widen_matches_the_fp8_decode_widened_by_torch():
    """The same tensor through e8huf_decode (FP8 bytes) and a torch widening
    on the GPU, against e8huf_decode_widen: one definition, two paths (the
    oracle remains the reference; this ties the two entry points)."""
    x = synth.e8_small(77, 5 * 16384 + 9)
    blob = O.e8_encode(x)
    info = e8huf.layer_info(blob)
    lut = e8huf.build_table(info["codelen"], 4)
    d_blob = torch.from_numpy(blob).to(DEV)
    d_lut = torch.from_numpy(lut.view(np.int16)).to(DEV)
    d8 = torch.empty(x.size, dtype=torch.uint8, device=DEV)
    d16 = torch.empty(x.size, dtype=torch.bfloat16, device=DEV)
    say("e8 widen vs decode + torch")
    e8huf.decode(d_blob, d_lut, d8)
    e8huf.decode_widen(d_blob, d_lut, d16, scale=0.25)
    torch.cuda.synchronize()
    ref = (d8.view(torch.float8_e4m3fn).to(torch.float32) * 0.25).to(torch.bfloat16)
    assert torch.equal(d16.view(torch.int16), ref.view(torch.int16))
