"""GPU parity of the FP8 exponent decoder (e8huf_decode, HIP, gfx950) against
the CPU oracle (ECF8 page, pwwt.cn/news/2030120, sections 2.1-2.2).

Containers come from the oracle's encoder; the expected bytes are the
generated FP8 tensor itself (decode(encode(x)) = x) and the oracle's
bit-by-bit decode. The bar is byte equality. Every case prints its name
before touching the GPU.
"""

import numpy as np
import pytest
import torch

import oracle as O
from lossless_huffman_decoding_amd import e8huf, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
_cache = {}


def say(*a):
    print("[gpu-case]", *a, flush=True)


def container(name, gen, exp_bits):
    if name not in _cache:
        x = gen()
        _cache[name] = (x, O.e8_encode(x, exp_bits))
    return _cache[name]


def gpu_decode(blob, n=None, lut=None, stream=None):
    info = e8huf.layer_info(blob) if (n is None or lut is None) else None
    n = info["n_values"] if n is None else n
    lut = e8huf.build_table(info["codelen"], info["exp_bits"]) if lut is None else lut
    d_blob = torch.from_numpy(np.ascontiguousarray(blob)).to(DEV)
    d_lut = torch.from_numpy(np.ascontiguousarray(lut).view(np.int16)).to(DEV)
    d_out = torch.full((n,), 0xA5, dtype=torch.uint8, device=DEV)
    d_status = torch.zeros(1, dtype=torch.int32, device=DEV)
    if stream is not None:
        stream.wait_stream(torch.cuda.current_stream())
    e8huf.decode(d_blob, d_lut, d_out, d_status, stream)
    torch.cuda.synchronize()
    return d_out.cpu().numpy(), int(d_status.item())


SIZES = [1, 2, 3, 15, 16, 17, 255, 256, 257, 4095, 16383, 16384, 16385, 3 * 16384 + 77,
         64 * 16384 + 5, 300 * 16384 + 9]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("n", SIZES)
def test_sizes_parity(n, fmt):
    eb = synth.FP8_EXP_BITS[fmt]
    x = synth.e8_small(n + 17, n, fmt)
    blob = O.e8_encode(x, eb)
    say("e8 sizes", fmt, n)
    got, st = gpu_decode(blob)
    assert st == 0
    want = O.e8_decode(blob)
    assert (want == x).all()
    assert (got == want).all()


def test_tiny_parity():
    x, blob = container("tiny", synth.e8_tiny, 4)
    say("e8 tiny", x.size)
    got, st = gpu_decode(blob)
    assert st == 0 and (got == O.e8_decode(blob)).all() and (got == x).all()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_heavy_parity(fmt):
    x, blob = container("heavy_" + fmt, lambda: synth.e8_heavy(fmt=fmt), synth.FP8_EXP_BITS[fmt])
    say("e8 heavy", fmt, x.size)
    got, st = gpu_decode(blob)
    assert st == 0 and (got == x).all()


def test_trunk_parity():
    """The FP8 trunk layer (585,000,000 values) from the oracle's container,
    compared with the generated tensor and, on its first and last 2^22
    values, with the oracle's own bit-by-bit decode of that container."""
    x, blob = container("trunk", synth.e8_trunk, 4)
    say("e8 trunk", x.size)
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got == x).all()
    want = O.e8_decode(blob)
    assert (got[: 1 << 22] == want[: 1 << 22]).all() and (got[-(1 << 22):] == want[-(1 << 22):]).all()


@pytest.mark.parametrize("case", ["one_exponent", "one_exponent_e5m2", "uniform_e4m3", "uniform_e5m2",
                                  "fib_e5m2", "long_codes_in_passes"])
def test_edge_parity(case):
    """One exponent value (1-bit codes); uniform bytes (every block's codes
    exceed the wave's 6 KiB buffer, so lanes decode in passes); Fibonacci
    exponent counts over 18 E5M2 fields (smoothed codes up to 16 bits, taken
    through the second-level table); and both at once: E5M2 blocks whose
    codes exceed the buffer (decoded in passes) holding codes of 13-16 bits."""
    n = 40 * 16384 + 123
    x, eb = {"one_exponent": (synth.e8_one_exponent(11, n), 4),
             "one_exponent_e5m2": (synth.e8_one_exponent(12, n, "e5m2"), 5),
             "uniform_e4m3": (synth.e8_uniform_bytes(13, n), 4),
             "uniform_e5m2": (synth.e8_uniform_bytes(14, n), 5),
             "fib_e5m2": (synth.e8_fib_exponents(15, n), 5),
             "long_codes_in_passes": (synth.e8_long_codes_in_passes(16, n), 5)}[case]
    blob = O.e8_encode(x, eb)
    say("e8 edge", case, n)
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got == x).all()
    if case in ("fib_e5m2", "long_codes_in_passes"):
        assert e8huf.layer_info(blob)["codelen"].max() > 12      # escapes were taken
    if case in ("uniform_e4m3", "uniform_e5m2", "long_codes_in_passes"):
        info = e8huf.layer_info(blob)
        assert info["n_bits"] / info["n_blocks"] > 6144 * 8      # blocks decode in passes


def test_long_codes_at_chunk_and_phase_edges():
    """Codes longer than 12 bits (taken through the second-level table) at
    the first and last values of lane chunks, on both sides of the edge
    between a lane's two 128-value halves (alone and in pairs), and at the
    end of a partial block's last lane: the cases where such a code meets a
    lookup that ran past a half or past the lane's count."""
    x, pos = synth.e8_rare_at_edges(1)
    blob = O.e8_encode(x, 4)
    cl = e8huf.layer_info(blob)["codelen"]
    assert cl[0] > 12 and cl[1] > 12
    say("e8 long codes at edges", x.size)
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got[pos] == x[pos]).all()
    assert (got == x).all()


def test_packer_container_decodes_on_gpu():
    x = synth.e8_small(77, 5 * 16384 + 3)
    blob = e8huf.encode(x)
    say("e8 packer container")
    got, st = gpu_decode(blob)
    assert st == 0 and (got == x).all()


def test_stream_invariance():
    x, blob = container("tiny", synth.e8_tiny, 4)
    s = torch.cuda.Stream()
    say("e8 stream invariance")
    a, sa = gpu_decode(blob)
    b, sb = gpu_decode(blob, stream=s)
    assert sa == sb == 0 and (a == b).all() and (a == x).all()


def _u64(blob, off):
    return int(np.frombuffer(bytes(blob[off: off + 8]), "<u8")[0])


def test_corrupt_header_is_flagged_and_nothing_written():
    x = synth.e8_small(21, 3 * 16384 + 5)
    good = O.e8_encode(x)
    info = e8huf.layer_info(good)
    lut = e8huf.build_table(info["codelen"], 4)
    bad = good.copy()
    bad[0] ^= 0xFF
    say("e8 corrupt header")
    got, st = gpu_decode(bad, n=x.size, lut=lut)
    assert st & e8huf.DEV_HEADER and (got == 0xA5).all()
    say("e8 wrong value count")
    got, st = gpu_decode(good, n=x.size + 1, lut=lut)
    assert st & e8huf.DEV_HEADER
    bad = good.copy()
    bad[48:56] = np.frombuffer(np.uint64(good.size + 256).tobytes(), np.uint8)   # nibble plane past the blob
    say("e8 nibble plane out of the blob")
    got, st = gpu_decode(bad, n=x.size, lut=lut)
    assert st & e8huf.DEV_HEADER


def test_graph_replays_beside_an_eager_decode():
    """An FP8 decode captured into a graph on stream s and replayed on the
    default stream while another FP8 decode runs on s: both tensors come
    back on every replay (eager fills and synchronization between replays;
    the kernel keeps no state between launches)."""
    x1 = synth.e8_small(26, 70 * 16384 + 19)
    x2 = synth.e8_small(27, 50 * 16384 + 3, "e5m2")
    b1, b2 = O.e8_encode(x1, 4), O.e8_encode(x2, 5)
    dev = []
    for b, eb in ((b1, 4), (b2, 5)):
        lut = e8huf.build_table(e8huf.layer_info(b)["codelen"], eb)
        dev.append((torch.from_numpy(b).to(DEV), torch.from_numpy(lut.view(np.int16)).to(DEV)))
    out1 = torch.empty(x1.size, dtype=torch.uint8, device=DEV)
    out2 = torch.empty(x2.size, dtype=torch.uint8, device=DEV)
    st1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    st2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    say("e8 graph capture of a decode")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        e8huf.decode(dev[0][0], dev[0][1], out1, st1)
    for rep in range(3):
        out1.fill_(0xA5)
        out2.fill_(0x5A)
        st1.zero_()
        st2.zero_()
        torch.cuda.synchronize()
        say("e8 graph replay beside a decode", rep)
        with torch.cuda.stream(s):
            e8huf.decode(dev[1][0], dev[1][1], out2, st2)
        g.replay()
        torch.cuda.synchronize()
        assert int(st1.item()) == 0 and int(st2.item()) == 0
        assert (out1.cpu().numpy() == x1).all(), rep
        assert (out2.cpu().numpy() == x2).all(), rep


def test_null_status_word():
    """The status word is optional (include/e8huf.h): a decode without one
    gives a valid tensor back, and a corrupt one (noise in the bitstream, a
    bad lane count) completes with nothing to report, after which a valid
    decode still gives its tensor back."""
    x = synth.e8_small(24, 5 * 16384 + 77)
    blob = O.e8_encode(x)
    info = e8huf.layer_info(blob)
    d_lut = torch.from_numpy(e8huf.build_table(info["codelen"], 4).view(np.int16)).to(DEV)

    def run(b):
        d_blob = torch.from_numpy(np.ascontiguousarray(b)).to(DEV)
        d_out = torch.full((x.size,), 0xA5, dtype=torch.uint8, device=DEV)
        e8huf.decode(d_blob, d_lut, d_out, None)
        torch.cuda.synchronize()
        return d_out.cpu().numpy()

    say("e8 null status: valid")
    assert (run(blob) == x).all()
    bad = blob.copy()
    boff, noff = _u64(blob, 40), _u64(blob, 48)
    bad[boff: noff] = np.random.default_rng(25).integers(0, 256, noff - boff, dtype=np.uint8)
    bad[128 + 136 * 2 + 8 + 2 * 5] ^= 1       # and a lane count of block 2
    say("e8 null status: corrupt")
    run(bad)
    say("e8 null status: valid again")
    assert (run(blob) == x).all()


def test_corrupt_index_and_bits_are_flagged():
    x = synth.e8_small(22, 3 * 16384 + 5)
    blob = O.e8_encode(x)
    b1 = blob.copy()
    b1[128 + 136 * 1 + 8 + 2 * 9] ^= 1        # lane 9 of block 1
    say("e8 corrupt lane bits")
    got, st = gpu_decode(b1)
    assert st & e8huf.DEV_INDEX
    assert (got[:16384] == x[:16384]).all() and (got[2 * 16384:] == x[2 * 16384:]).all()
    b2 = blob.copy()
    boff = _u64(blob, 40)
    noff = _u64(blob, 48)
    rng = np.random.default_rng(23)
    b2[boff: noff] = rng.integers(0, 256, noff - boff, dtype=np.uint8)
    say("e8 noise bitstream")
    got, st = gpu_decode(b2)
    assert st & (e8huf.DEV_CODE | e8huf.DEV_LANE_END)
    one = synth.e8_one_exponent(24, 20000)
    b3 = O.e8_encode(one).copy()
    b3[_u64(b3, 40)] = 0x80          # a one-symbol table has only the code '0'
    say("e8 uncovered code")
    got, st = gpu_decode(b3)
    assert st & e8huf.DEV_CODE


def test_concurrent_decodes_on_streams():
    xs = [synth.e8_small(30 + k, (k + 1) * 40000 + k) for k in range(6)]
    blobs = [O.e8_encode(x) for x in xs]
    outs, args = [], []
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    for x, b in zip(xs, blobs):
        info = e8huf.layer_info(b)
        lut = e8huf.build_table(info["codelen"], 4)
        args.append((torch.from_numpy(b).to(DEV), torch.from_numpy(lut.view(np.int16)).to(DEV)))
        outs.append(torch.full((x.size,), 0xA5, dtype=torch.uint8, device=DEV))
    streams = [torch.cuda.Stream() for _ in range(3)]
    torch.cuda.synchronize()
    say("e8 concurrent streams")
    for k, (db, dl) in enumerate(args):
        e8huf.decode(db, dl, outs[k], status, streams[k % 3])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for k, x in enumerate(xs):
        assert (outs[k].cpu().numpy() == x).all(), k
