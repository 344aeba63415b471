"""GPU parity for the 64-symbol lane-chunk layout (lane_syms = 64, 16 KiB
subblocks of 128 chunks), the container option for small layers: the
kernel reads the layout from the header. Containers come from the oracle's
encoder (the host packer's for the two largest layers, which equals the
oracle's byte for byte on every size the CPU tests cover); the bar is byte
equality with the generated layer and with the oracle's bit-by-bit decode.
Every case prints its name before touching the GPU."""

import numpy as np
import pytest
import torch

import oracle as O
from lossless_huffman_decoding_amd import k3huf, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[gpu-case]", *a, flush=True)


def to_dev(blob, lut):
    return (torch.from_numpy(np.ascontiguousarray(blob)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(lut).view(np.int16)).to(DEV))


def gpu_decode(blob, out_bytes=None):
    info = k3huf.layer_info(blob)
    d_blob, d_lut = to_dev(blob, k3huf.build_table(info["codelen"]))
    n = info["raw_bytes"] if out_bytes is None else out_bytes
    d_out = torch.full((n,), 0xA5, dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    k3huf.decode_layer(d_blob, d_lut, d_out, st)
    torch.cuda.synchronize()
    return d_out, int(st.item())


@pytest.mark.parametrize("n_bytes", [2, 4, 126, 128, 130, 1022, 8190, 8192, 8194, 16382, 16384, 16386,
                                     3 * 16384 + 514, 64 * 16384 - 2, 4 << 20, (1 << 26) - 2, 1 << 26,
                                     (1 << 26) + 3 * 16384 + 2])
def test_sizes_parity(n_bytes):
    x = synth.small_random(n_bytes + 11, n_bytes)
    blob = O.encode_layer(x, 64)
    assert k3huf.layer_info(blob)["lane_syms"] == 64
    say("short lanes sizes", n_bytes)
    got, st = gpu_decode(blob)
    assert st == 0
    want = O.decode_layer(blob)
    assert (want == x).all()
    assert (got.cpu().numpy() == want).all()


@pytest.mark.parametrize("layer", ["tiny", "edge_fib40", "edge_single", "edge_uniform"])
def test_configs_parity(layer):
    gen = {"tiny": synth.tiny, **dict(synth.CONFIGS["edge"])}[layer]
    x = gen()
    blob = O.encode_layer(x, 64)
    say("short lanes config", layer, x.size)
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got.cpu().numpy() == x).all()


def test_mixed_spans_parity():
    """Dense and sparse stretches of bitstream (uniform-byte spans take 8-bit
    codes: a unit's codes then fill 4 KiB of the 7.5 KiB buffer) across
    three stripes."""
    x = synth.mixed_spans(79, (2 << 26) + 3 * 16384 + 1234)
    blob = O.encode_layer(x, 64)
    say("short lanes mixed", x.size)
    got, st = gpu_decode(blob)
    assert st == 0
    assert (got.cpu().numpy() == x).all()


def test_trunk_layer_parity():
    """The 1.17 GB trunk layer in the short layout: 71,412 subblocks, more
    than five rounds of units, so it runs on the device work counters; the
    decode equals the layer, and the oracle decodes the first and last
    stripes of the same container to the same bytes."""
    x = synth.trunk_layer()
    blob = k3huf.encode_layer(x, lane_syms=64)
    info = k3huf.layer_info(blob)
    assert info["lane_syms"] == 64 and info["n_subblocks"] == -(-x.size // 16384)
    say("short lanes trunk", x.size)
    got, st = gpu_decode(blob)
    assert st == 0
    assert torch.equal(got, torch.from_numpy(x).to(DEV))
    last = info["n_stripes"] - 1
    assert (O.decode_stripes(blob, 0, 1, 1 << 26) == x[: 1 << 26]).all()
    tail = x.size - (last << 26)
    assert (O.decode_stripes(blob, last, 1, tail) == x[last << 26:]).all()


def test_corrupt_lane_bits_flagged():
    x = synth.small_random(13, 5 * 16384)
    blob = O.encode_layer(x, 64).copy()
    off = int(np.frombuffer(bytes(blob[304: 312]), "<u8")[0])
    blob[off + 32 + 264 * 2 + 8 + 2 * 70] ^= 1            # lane 70 of subblock 2 (second unit)
    say("short lanes corrupt lane bits")
    got, st = gpu_decode(blob)
    assert st & k3huf.DEV_INDEX
    got = got.cpu().numpy()
    assert (got[: 2 * 16384] == x[: 2 * 16384]).all()    # the other subblocks still decode
    assert (got[3 * 16384:] == x[3 * 16384:]).all()


def test_header_layout_mismatch_flagged():
    """A header whose lane_syms and subblock_bytes disagree is refused (on
    the host by layer_info; the kernel flags it and writes nothing)."""
    x = synth.small_random(14, 3 * 16384)
    good = O.encode_layer(x, 64)
    lut = k3huf.build_table(k3huf.layer_info(good)["codelen"])
    bad = good.copy()
    bad[12:16] = np.frombuffer(np.uint32(65536).tobytes(), np.uint8)   # subblock_bytes of the 256 layout
    with pytest.raises(k3huf.K3HufError):
        k3huf.layer_info(bad)
    d_blob, d_lut = to_dev(bad, lut)
    d_out = torch.full((x.size,), 0xA5, dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("short lanes header mismatch")
    k3huf.decode_layer(d_blob, d_lut, d_out, st)
    torch.cuda.synchronize()
    assert int(st.item()) & k3huf.DEV_HEADER
    assert (d_out.cpu().numpy() == 0xA5).all()


def test_ring_mixes_layouts():
    """The layer ring with layers of both layouts, in order, two slots on two
    streams."""
    sizes = [3 * 65536 + 514, 16384 * 5 + 2, 2 * 65536 + 2, 130, 4 * 65536 + 100, 7 * 16384]
    xs = [synth.small_random(300 + k, n) for k, n in enumerate(sizes)]
    blobs = [O.encode_layer(x, 64 if k % 2 else 256) for k, x in enumerate(xs)]
    dev = [to_dev(b, k3huf.build_table(k3huf.layer_info(b)["codelen"])) for b in blobs]
    layers = [(db, dl, x.size) for (db, dl), x in zip(dev, xs)]
    slots = [torch.empty(max(sizes), dtype=torch.uint8, device=DEV) for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    by_handle = {s.cuda_stream: s for s in streams}
    results = [torch.empty(n, dtype=torch.uint8, device=DEV) for n in sizes]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def consume(k, slot, handle):
        with torch.cuda.stream(by_handle[handle]):
            results[k].copy_(slots[slot][: sizes[k]])

    torch.cuda.synchronize()
    say("short lanes ring")
    k3huf.decode_ring(layers, slots, streams, consume, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for k in range(len(xs)):
        assert (results[k].cpu().numpy() == xs[k]).all(), k


# ---------------------------------------------------------------------------
# the GPU packer in the 64-symbol layout

def gpu_encode64(x, d_out=None, d_work=None):
    d_x = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    if d_out is None:   # non-zero patterns: a byte the kernels fail to write shows up
        d_out = torch.full((k3huf.encode_bound(x.size, 64),), 0x5A, dtype=torch.uint8, device=DEV)
        d_work = torch.full((k3huf.encode_work_bytes(x.size, 64),), 0xC3, dtype=torch.uint8, device=DEV)
    return k3huf.encode_layer_dev(d_x, d_out, d_work, lane_syms=64), d_x


@pytest.mark.parametrize("n_bytes", [2, 4, 126, 128, 130, 8190, 8192, 8194, 16382, 16384, 16386,
                                     3 * 16384 + 514, 64 * 16384 - 2, (1 << 26) - 2, 1 << 26,
                                     (1 << 26) + 3 * 16384 + 18])
def test_gpu_packer_sizes_match_oracle(n_bytes):
    x = synth.small_random(n_bytes + 17, n_bytes)
    want = O.encode_layer(x, 64)
    say("short lanes GPU packer", n_bytes)
    got, _ = gpu_encode64(x)
    got = got.cpu().numpy()
    assert got.size == want.size and (got == want).all()


@pytest.mark.parametrize("layer", ["tiny", "edge_fib40", "edge_single", "edge_uniform"])
def test_gpu_packer_configs_match_oracle(layer):
    gen = {"tiny": synth.tiny, **dict(synth.CONFIGS["edge"])}[layer]
    x = gen()
    want = O.encode_layer(x, 64)
    say("short lanes GPU packer config", layer)
    got, _ = gpu_encode64(x)
    got = got.cpu().numpy()
    assert got.size == want.size and (got == want).all()


def test_gpu_packer_mixed_spans_and_round_trip():
    """Uniform-byte spans (8-bit codes) among weight spans over three stripes,
    then decoded back on the GPU."""
    x = synth.mixed_spans(80, (2 << 26) + 3 * 16384 + 1234)
    want = O.encode_layer(x, 64)
    say("short lanes GPU packer mixed", x.size)
    got, d_x = gpu_encode64(x)
    assert got.numel() == want.size and (got.cpu().numpy() == want).all()
    out, st = gpu_decode(got.cpu().numpy())
    assert st == 0 and torch.equal(out, d_x)


def test_gpu_packer_reuses_buffers():
    big = synth.small_random(903, 5 * 16384 + 66)
    small = synth.small_random(904, 2 * 16384 + 10)
    d_out = torch.full((k3huf.encode_bound(big.size, 64),), 0x5A, dtype=torch.uint8, device=DEV)
    d_work = torch.full((k3huf.encode_work_bytes(big.size, 64),), 0xC3, dtype=torch.uint8, device=DEV)
    say("short lanes GPU packer reuse")
    a, _ = gpu_encode64(big, d_out, d_work)
    a = a.cpu().numpy()
    b, _ = gpu_encode64(small, d_out, d_work)
    b = b.cpu().numpy()
    assert (a == O.encode_layer(big, 64)).all()
    assert (b == O.encode_layer(small, 64)).all()


def test_gpu_packer_trunk_layer_equals_host_packer():
    x = synth.trunk_layer()
    say("short lanes GPU packer trunk", x.size)
    got, d_x = gpu_encode64(x)
    want = k3huf.encode_layer(x, lane_syms=64)
    assert got.numel() == want.size
    assert torch.equal(got, torch.from_numpy(want).to(DEV))
