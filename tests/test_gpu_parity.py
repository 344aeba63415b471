"""GPU parity: k3huf_decode_layer (HIP, gfx950) against the CPU oracle.

Containers come from the oracle's encoder; the expected bytes are the
generated layer itself (decode(encode(x)) = x, K3 trunk-compression page,
"verification results") and the oracle's bit-by-bit decode. The bar is byte
equality. Every case prints its name before touching the GPU.
"""

import numpy as np
import pytest
import torch

import oracle as O
from lossless_huffman_decoding_amd import k3huf, synth

pytestmark = pytest.mark.gpu
from oracle_cache import oracle_container

DEV = "cuda:0"


def say(*a):
    print("[gpu-case]", *a, flush=True)


def to_dev(blob, lut):
    d_blob = torch.from_numpy(np.ascontiguousarray(blob)).to(DEV)
    d_lut = torch.from_numpy(np.ascontiguousarray(lut).view(np.int16)).to(DEV)
    return d_blob, d_lut


def gpu_decode(blob, lut=None, out_bytes=None, stream=None):
    if lut is None or out_bytes is None:
        info = k3huf.layer_info(blob)
        lut = k3huf.build_table(info["codelen"]) if lut is None else lut
        out_bytes = info["raw_bytes"] if out_bytes is None else out_bytes
    d_blob, d_lut = to_dev(blob, lut)
    n = out_bytes
    d_out = torch.full((n,), 0xA5, dtype=torch.uint8, device=DEV)  # poison
    d_status = torch.zeros(1, dtype=torch.int32, device=DEV)
    if stream is not None:
        # the poison and the cleared status are queued on the current stream
        stream.wait_stream(torch.cuda.current_stream())
    k3huf.decode_layer(d_blob, d_lut, d_out, d_status, stream)
    torch.cuda.synchronize()
    return d_out.cpu().numpy(), int(d_status.item())


@pytest.mark.parametrize("n_bytes", [2, 4, 16, 1022, 1024, 1026, 1040, 65534, 65536, 65538,
                                     3 * 65536 + 514, 64 * 65536 - 2, (1 << 26), (1 << 26) + 2])
def test_sizes_parity(n_bytes):
    x = synth.small_random(n_bytes, n_bytes)
    blob = O.encode_layer(x)
    say("sizes", n_bytes)
    got, st = gpu_decode(blob)
    assert st == 0
    want = O.decode_layer(blob)
    assert (want == x).all()
    assert (got == want).all()


def test_tiny_parity():
    x, blob = oracle_container("tiny", synth.tiny)
    say("tiny", x.size)
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got == O.decode_layer(blob)).all()


@pytest.mark.parametrize("layer", ["edge_fib40", "edge_single", "edge_uniform"])
def test_edge_parity(layer):
    gen = dict(synth.CONFIGS["edge"])[layer]
    x, blob = oracle_container(layer, gen)
    say("edge", layer, x.size)
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got == x).all()
    want = O.decode_layer(blob)
    assert (got == want).all()


# The decode kernel's per-wave bitstream buffer (7,680 bytes), in 16-byte
# units: a full unit whose code span fits it is copied into LDS whole; a
# larger one takes the per-lane gather path; the layer's partial last unit
# runs in passes over lane ranges whose span fits the buffer.
KERNEL_BUF_UNITS = 7680 // 16


def unit_paths(blob):
    """Each 256-symbol-layout unit's decode path, from the container's index
    as include/k3huf.h lays it out: 'fill' or 'gather' for a full unit
    (32,768 output bytes), ('tail', passes) for a partial one. A unit's span
    runs from the 16 bytes holding the bit before its first code to two
    dwords past the dword of its last bit, rounded up to 16 bytes."""
    info = k3huf.layer_info(blob)
    assert info["lane_syms"] == 256
    first16 = lambda p: ((p - 1) >> 5) & ~3          # noqa: E731  (dwords)
    end16 = lambda p: (((p - 1) >> 5) + 6) & ~3      # noqa: E731
    paths = []
    for s in range(info["n_stripes"]):
        so = int(np.frombuffer(bytes(blob[304 + 8 * s: 312 + 8 * s]), "<u8")[0])
        n_sub = int(np.frombuffer(bytes(blob[so + 20: so + 24]), "<u4")[0])
        for j in range(n_sub):
            r = so + 32 + 264 * j
            start, nsyms = (int(v) for v in np.frombuffer(bytes(blob[r: r + 8]), "<u4"))
            lb = np.frombuffer(bytes(blob[r + 8: r + 264]), "<u2").astype(np.int64)
            for half in (0, 1):
                syms = min(max(nsyms - half * 16384, 0), 16384)
                if syms == 0:
                    continue
                ends = start + np.cumsum(lb)[64 * half: 64 * half + 64]
                starts = ends - lb[64 * half: 64 * half + 64]
                if syms == 16384:
                    units = (end16(int(ends[63])) - first16(int(starts[0]))) // 4
                    paths.append("fill" if units <= KERNEL_BUF_UNITS else "gather")
                else:
                    l0, passes = 0, 0
                    while l0 < 64:
                        j0 = first16(int(starts[l0]))
                        l1 = l0 + 1
                        while l1 < 64 and end16(int(ends[l1])) - j0 <= 4 * KERNEL_BUF_UNITS:
                            l1 += 1
                        l0, passes = l1, passes + 1
                    paths.append(("tail", passes))
    return paths


@pytest.mark.parametrize("n_bytes", [65536, 65536 + 2 * 12000, 3 * 65536 + 2 * 20000 + 2,
                                     2 * 65536 - 2, 4 * 65536 + 2 * 7000])
def test_units_over_the_lds_buffer(n_bytes):
    """Uniform high bytes take 8-bit codes, so a full unit's codes (16 KiB)
    exceed the kernel's 7.5 KiB bitstream buffer (each lane then gathers its
    codes phase by phase), and a partial last unit of more than 7680 symbols
    decodes in several passes over lane ranges."""
    x = synth.edge_uniform(seed=700 + n_bytes % 97, n_bytes=n_bytes)
    blob = O.encode_layer(x)
    paths = unit_paths(blob)
    assert "gather" in paths and "fill" not in paths
    assert paths[-1] in ("gather", ("tail", 1), ("tail", 2), ("tail", 3))
    say("over buffer", n_bytes, paths[-1])
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got == x).all()
    assert (got == O.decode_layer(blob)).all()


def test_some_units_over_the_lds_buffer():
    """Weights with two half-subblocks of uniform high bytes: those units'
    codes are long (the rare symbols get codes of 11-12 bits) and exceed the
    buffer, while their neighbours fit it."""
    x = synth.small_random(21, 8 * 65536 + 4098).copy()
    rng = np.random.default_rng(5)
    for start in (65536 + 32768, 5 * 65536):   # a second-half and a first-half unit
        x[start + 1: start + 32768: 2] = rng.integers(0, 256, 16384, dtype=np.uint8)
    blob = O.encode_layer(x)
    paths = unit_paths(blob)
    assert paths.count("gather") == 2 and paths.count("fill") == len(paths) - 3
    say("some units over buffer")
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got == x).all()


@pytest.mark.parametrize("tail_syms", [3000, 9000, 12000, 15000, 16382])
def test_partial_last_unit_in_passes(tail_syms):
    """Weights, then a partial last unit of uniform high bytes (rare symbols
    with codes of 11-12 bits, so 3-4 times the 8-bit case's bits per symbol):
    it decodes in one pass when its codes fit the buffer and in two to four
    passes over lane ranges when they do not; full units of such bytes, or
    of half such bytes, before it take the gather path."""
    x = synth.small_random(31, 10 * 65536 + 2 * tail_syms).copy()
    rng = np.random.default_rng(tail_syms)
    x[10 * 65536 + 1::2] = rng.integers(0, 256, tail_syms, dtype=np.uint8)
    x[9 * 65536 + 32768 + 1: 10 * 65536: 2] = rng.integers(0, 256, 16384, dtype=np.uint8)
    x[8 * 65536 + 1: 8 * 65536 + 16384: 2] = rng.integers(0, 256, 8192, dtype=np.uint8)
    blob = O.encode_layer(x)
    paths = unit_paths(blob)
    want = 1 if tail_syms * 12 <= 7680 * 8 - 64 else 2
    assert paths[-1][0] == "tail" and paths[-1][1] >= want
    assert paths.count("gather") == 2
    say("partial last unit in passes", tail_syms, paths[-1])
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got == x).all()
    assert (got == O.decode_layer(blob)).all()


def _shift_first_stripe(blob, pad=256):
    """The same container with its stripe records and planes moved `pad`
    bytes further from the header (stripe offsets and container size
    adjusted): the format gives each stripe record's offset explicitly, so
    it stays a valid container of the same layer."""
    info = k3huf.layer_info(blob)
    ns = info["n_stripes"]
    so = np.frombuffer(bytes(blob[304: 304 + 8 * ns]), "<u8").astype(np.uint64)
    out = np.concatenate([blob[: int(so[0])], np.zeros(pad, np.uint8), blob[int(so[0]):]])
    out[304: 304 + 8 * ns] = np.frombuffer((so + np.uint64(pad)).tobytes(), np.uint8)
    out[40:48] = np.frombuffer(np.uint64(blob.size + pad).tobytes(), np.uint8)
    return out


@pytest.mark.parametrize("n_bytes,lanes", [(3 * 65536 + 514, 256), (3 * 65536 + 514, 64),
                                           ((1 << 26) + 4 * 65536 + 6, 256)])
def test_first_stripe_record_elsewhere(n_bytes, lanes):
    """The packers put the first stripe record right after the padded
    offset table, but the format gives each stripe record's offset
    explicitly: a container that keeps them elsewhere (here 256 bytes
    further) decodes through its stored offsets, in one-stripe and
    two-stripe layers and both lane-chunk layouts."""
    x = synth.small_random(n_bytes % 1000 + lanes, n_bytes)
    blob = _shift_first_stripe(O.encode_layer(x, lanes))
    assert (O.decode_layer(blob) == x).all()
    say("first stripe record elsewhere", n_bytes, lanes)
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got == x).all()


def test_heavy_parity():
    x, blob = oracle_container("heavy", synth.heavy)
    say("heavy", x.size)
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got == x).all()
    # oracle bit-by-bit decode of the first and last stripes, compared in place
    first = O.decode_stripes(blob, 0, 1, 1 << 26)
    last = O.decode_stripes(blob, 3, 1, 1 << 26)
    assert (got[: 1 << 26] == first).all() and (got[3 << 26:] == last).all()


def test_trunk_layer_parity():
    x, blob = oracle_container("trunk", synth.trunk_layer)
    say("trunk", x.size)
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got == x).all()
    n_str = -(-x.size // (1 << 26))
    for s in (0, n_str - 1):
        size = min(1 << 26, x.size - (s << 26))
        want = O.decode_stripes(blob, s, 1, size)
        assert (got[s << 26: (s << 26) + size] == want).all()


def test_packer_containers_decode_on_gpu():
    for name, gen in (("tiny", synth.tiny), ("edge_fib40", synth.edge_fib40)):
        x = gen()
        blob = k3huf.encode_layer(x)
        say("packer", name)
        got, st = gpu_decode(blob)
        assert st == 0 and (got == x).all()


def test_repeat_and_stream_invariance():
    x, blob = oracle_container("tiny", synth.tiny)
    s = torch.cuda.Stream()
    say("stream invariance")
    a, sa = gpu_decode(blob)
    b, sb = gpu_decode(blob, stream=s)
    c, sc = gpu_decode(blob, stream=s)
    assert sa == sb == sc == 0
    assert (a == b).all() and (b == c).all() and (a == x).all()


# ---------------------------------------------------------------------------
# corrupted containers: flagged through d_status, never a fault

def _hdr_field_off(blob, s):
    return int(np.frombuffer(bytes(blob[304 + 8 * s: 312 + 8 * s]), "<u8")[0])


def test_corrupt_header_is_flagged_and_nothing_written():
    x = synth.small_random(9, 3 * 65536 + 514)
    good = O.encode_layer(x)
    lut = k3huf.build_table(k3huf.layer_info(good)["codelen"])
    blob = good.copy()
    blob[0] ^= 0xFF
    say("corrupt header")
    got, st = gpu_decode(blob, lut=lut, out_bytes=x.size)
    assert st & k3huf.DEV_HEADER
    assert (got == 0xA5).all()


def test_decode_without_a_status_word():
    """d_status may be null: a good layer decodes, and a corrupt header
    (which the kernel would flag) leaves the output unwritten."""
    x = synth.small_random(19, 3 * 65536 + 514)
    good = O.encode_layer(x)
    lut = k3huf.build_table(k3huf.layer_info(good)["codelen"])
    bad = good.copy()
    bad[0] ^= 0xFF
    for blob, ok in ((good, True), (bad, False)):
        d_blob, d_lut = to_dev(blob, lut)
        d_out = torch.full((x.size,), 0xA5, dtype=torch.uint8, device=DEV)
        say("no status word", "good" if ok else "corrupt header")
        k3huf.decode_layer(d_blob, d_lut, d_out, None)
        torch.cuda.synchronize()
        got = d_out.cpu().numpy()
        assert (got == x).all() if ok else (got == 0xA5).all()


def test_wrong_out_size_is_flagged():
    x = synth.small_random(10, 65536 * 2)
    blob = O.encode_layer(x)
    lut = k3huf.build_table(k3huf.layer_info(blob)["codelen"])
    say("wrong out size")
    got, st = gpu_decode(blob, lut=lut, out_bytes=65536 * 2 + 2)
    assert st & k3huf.DEV_HEADER


def test_corrupt_index_and_stripe_are_flagged():
    x = synth.small_random(11, 3 * 65536)
    blob = O.encode_layer(x)
    off = _hdr_field_off(blob, 0)
    b1 = blob.copy()
    b1[off + 32 + 264 * 1 + 8 + 2 * 5] ^= 1        # lane 5 of subblock 1
    say("corrupt lane bits")
    got, st = gpu_decode(b1)
    assert st & k3huf.DEV_INDEX
    assert (got[:65536] == x[:65536]).all()          # the other subblocks still decode
    assert (got[2 * 65536:] == x[2 * 65536:]).all()
    b2 = blob.copy()
    b2[304: 312] = np.frombuffer(np.uint64(b2.size + 4096).tobytes(), np.uint8)
    say("corrupt stripe offset")
    got, st = gpu_decode(b2, lut=k3huf.build_table(k3huf.layer_info(blob)["codelen"]),
                         out_bytes=x.size)
    assert st & k3huf.DEV_STRIPE


def test_corrupt_bits_are_detectable():
    x = synth.small_random(12, 2 * 65536)
    blob = O.encode_layer(x)
    st0 = blob.copy()
    off = _hdr_field_off(blob, 0)
    bits_off = int(np.frombuffer(bytes(blob[off + 24: off + 28]), "<u4")[0])
    st0[off + bits_off + 333] ^= 0x24
    say("corrupt bits")
    got, st = gpu_decode(st0)
    assert st != 0 or not (got == x).all()


def test_bitstream_of_noise_is_flagged():
    """Every code bit replaced by noise over a 16 MiB layer: every unit's
    lanes end off their index; the kernel flags it and finishes (status is
    set once per wave, not once per lane)."""
    x = synth.small_random(14, 16 << 20)
    blob = O.encode_layer(x).copy()
    off = _hdr_field_off(blob, 0)
    bits_off = int(np.frombuffer(bytes(blob[off + 24: off + 28]), "<u4")[0])
    even_off = int(np.frombuffer(bytes(blob[off + 28: off + 32]), "<u4")[0])
    rng = np.random.default_rng(15)
    blob[off + bits_off: off + even_off] = rng.integers(0, 256, even_off - bits_off, dtype=np.uint8)
    say("noise bitstream")
    got, st = gpu_decode(blob)
    assert st & (k3huf.DEV_CODE | k3huf.DEV_LANE_END)


def test_unused_slot_is_flagged():
    # one-symbol table: codes are '0'; a '1' bit hits an unused slot
    x = synth.edge_single(n_bytes=65536)
    blob = O.encode_layer(x).copy()
    off = _hdr_field_off(blob, 0)
    bits_off = int(np.frombuffer(bytes(blob[off + 24: off + 28]), "<u4")[0])
    blob[off + bits_off] = 0x80
    say("unused slot")
    got, st = gpu_decode(blob)
    assert st & k3huf.DEV_CODE


def test_bad_arguments_raise_before_launch():
    x = synth.small_random(13, 4096)
    blob = O.encode_layer(x)
    lut = k3huf.build_table(k3huf.layer_info(blob)["codelen"])
    d_blob, d_lut = to_dev(blob, lut)
    d_out = torch.empty(4096 + 16, dtype=torch.uint8, device=DEV)
    say("bad args")
    with pytest.raises(k3huf.K3HufError):
        k3huf.decode_layer(d_blob, d_lut, d_out[1: 4097])       # misaligned output
    with pytest.raises(k3huf.K3HufError):
        k3huf.decode_layer(d_blob, d_lut, d_out[:4095])         # odd size
    with pytest.raises(k3huf.K3HufError):
        k3huf.decode_layer(d_blob[:100], d_lut, d_out[:4096])   # blob shorter than a header
    with pytest.raises(k3huf.K3HufError):
        k3huf.decode_layer(d_blob[:1024], d_lut, d_out[:4096])  # output above twice the blob


def test_layer_at_the_start_of_a_buffer_over_8_gib():
    """A two-stripe container at the start of a 9 GiB device buffer, decoded
    with blob_bytes set to the whole buffer: every stripe's bitstream starts
    more than 8 GiB before the blob's end. The kernel bounds its bitstream
    reads by each stripe's own planes, in 64-bit offsets (the read bounds are
    checked on the CPU up to 2^36 bytes by tests/test_read_bounds.py), so the
    layer decodes exactly."""
    x = synth.small_random(655, (1 << 26) + 3 * 65536 + 514)
    blob = O.encode_layer(x)
    lut = k3huf.build_table(k3huf.layer_info(blob)["codelen"])
    big = (9 << 30) + 4096
    say("layer in a buffer of", big, "bytes")
    d_buf = torch.zeros(big, dtype=torch.uint8, device=DEV)
    d_buf[: blob.size].copy_(torch.from_numpy(blob))
    d_lut = torch.from_numpy(lut.view(np.int16)).to(DEV)
    d_out = torch.full((x.size,), 0xA5, dtype=torch.uint8, device=DEV)
    d_status = torch.zeros(1, dtype=torch.int32, device=DEV)
    k3huf.decode_layer(d_buf, d_lut, d_out, d_status)
    torch.cuda.synchronize()
    assert int(d_status.item()) == 0
    assert (d_out.cpu().numpy() == x).all()
    del d_buf
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# layer ring (K3 TUNING page, section 2: a two-slot trunk ring)

@pytest.mark.parametrize("n_slots,n_streams", [(2, 2), (1, 1), (3, 2), (2, 1)])
def test_ring_decodes_layers_in_order(n_slots, n_streams):
    sizes = [3 * 65536 + 514, 65536, 2 * 65536 + 2, 5 * 65536, 1026, 4 * 65536 + 100]
    xs = [synth.small_random(100 + k, n) for k, n in enumerate(sizes)]
    blobs = [O.encode_layer(x) for x in xs]
    luts = [k3huf.build_table(k3huf.layer_info(b)["codelen"]) for b in blobs]
    dev = [to_dev(b, l) for b, l in zip(blobs, luts)]
    layers = [(db, dl, x.size) for (db, dl), x in zip(dev, xs)]
    slot_bytes = max(sizes)
    slots = [torch.empty(slot_bytes, dtype=torch.uint8, device=DEV) for _ in range(n_slots)]
    streams = [torch.cuda.Stream() for _ in range(n_streams)]
    by_handle = {s.cuda_stream: s for s in streams}
    results = [torch.empty(n, dtype=torch.uint8, device=DEV) for n in sizes]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def consume(k, slot, handle):
        with torch.cuda.stream(by_handle[handle]):
            results[k].copy_(slots[slot][: sizes[k]])

    torch.cuda.synchronize()   # buffers prepared on the current stream
    say("ring", n_slots, n_streams)
    k3huf.decode_ring(layers, slots, streams, consume, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for k in range(len(xs)):
        assert (results[k].cpu().numpy() == xs[k]).all(), k


def test_ring_streamed_trunk_layers_full_size():
    """The streamed-trunk ring at its real shape: six 1.17 GB trunk layers
    (per-layer seeds, as layers 0..5 of the 93-layer pass) decoded in fixed
    order into two slots on two streams (K3 page, "background": layers are
    visited in order 0..92; K3 TUNING page, section 2: a two-slot ring). Each
    layer is copied out of its slot on the slot's stream before the slot is
    released, and every layer is compared byte for byte with its generated
    bytes."""
    n = 6
    xs = [synth.streamed_layer(k) for k in range(n)]
    blobs = [k3huf.encode_layer(x) for x in xs]
    luts = [k3huf.build_table(k3huf.layer_info(b)["codelen"]) for b in blobs]
    dev = [to_dev(b, l) for b, l in zip(blobs, luts)]
    del blobs
    layers = [(db, dl, x.size) for (db, dl), x in zip(dev, xs)]
    slots = [torch.empty(max(x.size for x in xs), dtype=torch.uint8, device=DEV) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    by_handle = {s.cuda_stream: s for s in streams}
    results = [torch.full((x.size,), 0xA5, dtype=torch.uint8, device=DEV) for x in xs]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def consume(k, slot, handle):
        with torch.cuda.stream(by_handle[handle]):
            results[k].copy_(slots[slot][: xs[k].size])

    torch.cuda.synchronize()   # buffers prepared on the current stream
    say("streamed ring, full-size trunk layers", n)
    k3huf.decode_ring(layers, slots, streams, consume, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for k, x in enumerate(xs):
        assert torch.equal(results[k], torch.from_numpy(x).to(DEV)), k
    del results, slots, dev, layers
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# host-fed ring (K3 page, "background": the trunk streams from storage in the
# fixed layer order; K3 TUNING page, section 5: extra ring slots hold reads in
# flight)

def _pinned(a):
    t = torch.empty(a.size, dtype=torch.uint8, pin_memory=True)
    t.numpy()[:] = a
    return t


@pytest.mark.parametrize("n_stage,n_slots,n_streams", [(2, 2, 2), (1, 1, 1), (3, 2, 2), (2, 3, 1)])
def test_host_ring_decodes_layers_in_order(n_stage, n_slots, n_streams):
    sizes = [3 * 65536 + 514, 65536, 2 * 65536 + 2, 5 * 65536, 1026, 4 * 65536 + 100, 70000]
    xs = [synth.small_random(300 + k, n) for k, n in enumerate(sizes)]
    blobs = [O.encode_layer(x) for x in xs]
    luts = [k3huf.build_table(k3huf.layer_info(b)["codelen"]) for b in blobs]
    h_blobs = [_pinned(b) for b in blobs]
    d_luts = [torch.from_numpy(l.view(np.int16)).to(DEV) for l in luts]
    layers = [(hb, dl, x.size) for hb, dl, x in zip(h_blobs, d_luts, xs)]
    stages = [torch.empty(max(b.size for b in blobs), dtype=torch.uint8, device=DEV)
              for _ in range(n_stage)]
    slots = [torch.empty(max(sizes), dtype=torch.uint8, device=DEV) for _ in range(n_slots)]
    copy_stream = torch.cuda.Stream()
    streams = [torch.cuda.Stream() for _ in range(n_streams)]
    by_handle = {s.cuda_stream: s for s in streams}
    results = [torch.empty(n, dtype=torch.uint8, device=DEV) for n in sizes]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def consume(k, slot, handle):
        with torch.cuda.stream(by_handle[handle]):
            results[k].copy_(slots[slot][: sizes[k]])

    torch.cuda.synchronize()   # buffers prepared on the current stream
    say("host ring", n_stage, n_slots, n_streams)
    k3huf.decode_ring_host(layers, stages, slots, copy_stream, streams, consume, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for k in range(len(xs)):
        assert (results[k].cpu().numpy() == xs[k]).all(), k


def test_host_ring_repeated_containers_and_pageable_memory():
    """The same host container fed several times (stage reuse), and a
    pageable (not pinned) host container: both decode exactly."""
    x = synth.small_random(77, 6 * 65536 + 6)
    blob = O.encode_layer(x)
    lut = torch.from_numpy(k3huf.build_table(k3huf.layer_info(blob)["codelen"]).view(np.int16)).to(DEV)
    pinned = _pinned(blob)
    pageable = torch.from_numpy(blob.copy())
    layers = [(pinned, lut, x.size), (pageable, lut, x.size), (pinned, lut, x.size),
              (pinned, lut, x.size)]
    stages = [torch.empty(blob.size, dtype=torch.uint8, device=DEV) for _ in range(2)]
    slots = [torch.empty(x.size, dtype=torch.uint8, device=DEV) for _ in range(2)]
    copy_stream = torch.cuda.Stream()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    by_handle = {s.cuda_stream: s for s in streams}
    results = [torch.empty(x.size, dtype=torch.uint8, device=DEV) for _ in layers]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def consume(k, slot, handle):
        with torch.cuda.stream(by_handle[handle]):
            results[k].copy_(slots[slot])

    torch.cuda.synchronize()   # buffers prepared on the current stream
    say("host ring repeat/pageable")
    k3huf.decode_ring_host(layers, stages, slots, copy_stream, streams, consume, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for k, r in enumerate(results):
        assert (r.cpu().numpy() == x).all(), k


def test_concurrent_decodes_on_many_streams():
    """Decodes queued on six streams at once (three layers each, every
    stream with its own work-counter slot) all give their layers back."""
    sizes = [2 * 65536 + 10, 5 * 65536 + 4, 3 * 65536 + 514]
    xs = [synth.small_random(500 + k, sizes[k % 3]) for k in range(18)]
    blobs = [O.encode_layer(x) for x in xs]
    dev = [to_dev(b, k3huf.build_table(k3huf.layer_info(b)["codelen"])) for b in blobs]
    outs = [torch.full((x.size,), 0xA5, dtype=torch.uint8, device=DEV) for x in xs]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    streams = [torch.cuda.Stream() for _ in range(6)]
    torch.cuda.synchronize()   # poison and status prepared on the current stream
    say("concurrent streams", len(streams), len(xs))
    for k, (db, dl) in enumerate(dev):
        k3huf.decode_layer(db, dl, outs[k], status, streams[k % 6])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for k, x in enumerate(xs):
        assert (outs[k].cpu().numpy() == x).all(), k


def _hip_runtime():
    """The HIP runtime torch has loaded (same soname, so dlopen returns it)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipStreamCreate.restype = ctypes.c_int
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    hip.hipStreamDestroy.restype = ctypes.c_int
    return hip


@pytest.fixture(scope="module")
def many_streams():
    """300 raw HIP streams (hipStreamCreate; torch's own Stream() objects
    come from a pool of 32 and repeat), all alive at once, each registered by
    a decode. The library gives work-counter slots to the first 256 distinct
    streams of a device it sees and none to later ones, so at least the last
    44 of these 300 distinct handles have no slot, whatever streams earlier
    tests registered: decodes on them hand out units from workgroup
    counters."""
    import ctypes
    torch.cuda.init()
    hip = _hip_runtime()
    handles = []
    for _ in range(300):
        h = ctypes.c_void_p()
        assert hip.hipStreamCreate(ctypes.byref(h)) == 0
        handles.append(h.value)
    assert len(set(handles)) == 300 > 256
    streams = [torch.cuda.ExternalStream(h, device=DEV) for h in handles]
    x = synth.small_random(611, 3 * 65536 + 514)
    blob = O.encode_layer(x)
    db, dl = to_dev(blob, k3huf.build_table(k3huf.layer_info(blob)["codelen"]))
    outs = [torch.full((x.size,), 0xA5, dtype=torch.uint8, device=DEV) for _ in streams]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()   # poison and status prepared on the current stream
    say("register 300 raw streams")
    for s, o in zip(streams, outs):
        k3huf.decode_layer(db, dl, o, status, s)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for k, o in enumerate(outs):
        assert (o.cpu().numpy() == x).all(), k
    yield streams
    torch.cuda.synchronize()
    for h in handles:
        assert hip.hipStreamDestroy(h) == 0


def test_concurrent_decodes_past_the_counter_slots(many_streams):
    """Decodes queued at once on a stream with a counter slot (layers of
    more than five rounds of units take its counters) and on streams past the
    slot limit (workgroup counters) all give their layers back."""
    xs = [synth.small_random(620 + k, (330 << 20) + 2 * k * 65536 + 6) for k in range(3)]
    blobs = [O.encode_layer(x) for x in xs]
    dev = [to_dev(b, k3huf.build_table(k3huf.layer_info(b)["codelen"])) for b in blobs]
    outs = [torch.empty(x.size, dtype=torch.uint8, device=DEV) for x in xs]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    streams = [many_streams[0], many_streams[-1], many_streams[-2]]
    for rep in range(3):
        for o in outs:
            o.fill_(0xA5)
        torch.cuda.synchronize()
        say("concurrent past the slot limit, round", rep)
        for k in range(3):
            k3huf.decode_layer(dev[k][0], dev[k][1], outs[k], status, streams[k])
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        for k, x in enumerate(xs):
            assert (outs[k].cpu().numpy() == x).all(), (rep, k)


@pytest.mark.parametrize("kind", ["weights", "mixed_spans"])
def test_ticketed_schedule_parity(kind):
    """Layers of more than five rounds of units (about 12,800 units against
    1,792 wave slots) take their later units from the device counters;
    ragged tails, six stripes plus a partial one."""
    n = (400 << 20) + 2 * 65536 + 514
    x = synth.small_random(641, n) if kind == "weights" else synth.mixed_spans(642, n)
    blob = O.encode_layer(x)
    say("ticketed schedule", kind, x.size)
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got == x).all()


@pytest.mark.parametrize("layer", ["tiny", "edge_fib40", "edge_single", "edge_uniform", "heavy", "trunk"])
def test_unslotted_stream_parity(many_streams, layer):
    """Every config decodes right on a stream past the counter slots (each
    workgroup's share of units handed to its waves from its own counter);
    the trunk layer is the case of more than five rounds of units without
    device counters."""
    gen = {"tiny": synth.tiny, "heavy": synth.heavy, "trunk": synth.trunk_layer,
           **dict(synth.CONFIGS["edge"])}[layer]
    x, blob = oracle_container(layer, gen)
    say("unslotted stream", layer, x.size)
    got, st = gpu_decode(blob, stream=many_streams[-1])
    assert st == 0
    assert (got == x).all()


def test_graph_replays_beside_decodes_on_the_capture_stream():
    """A decode captured into a graph on stream s, replayed on the default
    stream while another decode runs on s: both layers come back, on every
    replay (eager work and synchronization between replays)."""
    x1 = synth.small_random(631, (16 << 20) + 2 * 65536 + 18)
    x2 = synth.small_random(632, (24 << 20) + 6)
    b1, b2 = O.encode_layer(x1), O.encode_layer(x2)
    d1 = to_dev(b1, k3huf.build_table(k3huf.layer_info(b1)["codelen"]))
    d2 = to_dev(b2, k3huf.build_table(k3huf.layer_info(b2)["codelen"]))
    out1 = torch.empty(x1.size, dtype=torch.uint8, device=DEV)
    out2 = torch.empty(x2.size, dtype=torch.uint8, device=DEV)
    st1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    st2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()   # status words cleared on the current stream
    say("graph capture of a decode")
    with torch.cuda.stream(s):
        k3huf.decode_layer(d2[0], d2[1], out2, st2)     # the stream's first decode takes its slot
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        k3huf.decode_layer(d1[0], d1[1], out1, st1)
    for rep in range(3):
        out1.fill_(0xA5)
        out2.fill_(0x5A)
        st1.zero_()
        st2.zero_()
        torch.cuda.synchronize()
        say("graph replay beside a decode on the capture stream", rep)
        with torch.cuda.stream(s):
            k3huf.decode_layer(d2[0], d2[1], out2, st2)
        g.replay()
        torch.cuda.synchronize()
        assert int(st1.item()) == 0 and int(st2.item()) == 0
        assert (out1.cpu().numpy() == x1).all(), rep
        assert (out2.cpu().numpy() == x2).all(), rep
