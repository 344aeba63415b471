"""GPU encoder (k3huf_encode_layer_dev) against the CPU oracle's encoder.

The container is fully determined by the layer (K3 trunk-compression page:
one histogram and codelen[256] per layer, longest-first canonical codes,
64 MiB stripes, MSB-first bitstream, raw even plane; plus the subblock
index), so the bar is byte equality with the oracle's container. A GPU
round trip (encode, then decode) must give the layer back. Every case prints
its name before touching the GPU.
"""

import numpy as np
import pytest
import torch

import oracle as O
from lossless_huffman_decoding_amd import k3huf, synth
from oracle_cache import oracle_container

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[gpu-case]", *a, flush=True)


def garbage_buffers(n_bytes):
    """Output and work buffers for an encode of n_bytes, filled with a
    non-zero pattern: a container byte the kernels fail to write then shows
    up as a mismatch against the oracle."""
    d_out = torch.full((k3huf.encode_bound(n_bytes),), 0x5A, dtype=torch.uint8, device=DEV)
    d_work = torch.full((k3huf.encode_work_bytes(n_bytes),), 0xC3, dtype=torch.uint8, device=DEV)
    return d_out, d_work


def gpu_encode(x, d_out=None, d_work=None):
    d_x = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    if d_out is None:
        d_out, d_work = garbage_buffers(x.size)
    blob = k3huf.encode_layer_dev(d_x, d_out, d_work)
    return blob.cpu().numpy(), d_x


def gpu_decode_dev(d_blob, raw_bytes):
    lut = k3huf.build_table(k3huf.layer_info(d_blob[:512].cpu().numpy())["codelen"])
    d_lut = torch.from_numpy(lut.view(np.int16)).to(DEV)
    d_out = torch.full((raw_bytes,), 0xA5, dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    k3huf.decode_layer(d_blob, d_lut, d_out, st)
    torch.cuda.synchronize()
    return d_out, int(st.item())


@pytest.mark.parametrize("n_bytes", [2, 4, 16, 18, 510, 512, 514, 1022, 1024, 1026, 65534, 65536,
                                     65538, 3 * 65536 + 514, 64 * 65536 - 2, (1 << 26) - 2,
                                     (1 << 26), (1 << 26) + 2, (1 << 26) + 3 * 65536 + 18])
def test_encode_sizes_match_oracle(n_bytes):
    x = synth.small_random(n_bytes + 7, n_bytes)
    want = O.encode_layer(x)
    say("encode sizes", n_bytes)
    got, _ = gpu_encode(x)
    assert got.size == want.size
    assert (got == want).all()


@pytest.mark.parametrize("layer", ["tiny", "edge_fib40", "edge_single", "edge_uniform", "heavy"])
def test_encode_configs_match_oracle(layer):
    gen = {"tiny": synth.tiny, "heavy": synth.heavy, **dict(synth.CONFIGS["edge"])}[layer]
    x, want = oracle_container(layer, gen)
    say("encode config", layer, x.size)
    got, _ = gpu_encode(x)
    assert got.size == want.size
    assert (got == want).all()


def test_encode_trunk_layer_matches_oracle_and_round_trips():
    x, want = oracle_container("trunk", synth.trunk_layer)
    say("encode trunk", x.size)
    d_x = torch.from_numpy(x).to(DEV)
    d_blob = k3huf.encode_layer_dev(d_x, *garbage_buffers(x.size))
    got = d_blob.cpu().numpy()
    assert got.size == want.size
    assert (got == want).all()
    say("encode trunk: decode back")
    d_dec, st = gpu_decode_dev(d_blob, x.size)
    assert st == 0
    assert torch.equal(d_dec, d_x)


def test_encode_mixed_spans_matches_oracle_and_round_trips():
    """Spans of uniform bytes (units too large for the packing kernel's LDS
    buffer, which pack straight into memory) alternate with weight spans
    (buffered units) across three stripes, so the two kinds of unit meet at
    about 1100 unit boundaries and share their boundary words."""
    x = synth.mixed_spans(78, (2 << 26) + 3 * 65536 + 1234)
    want = O.encode_layer(x)
    say("encode mixed spans", x.size)
    got, d_x = gpu_encode(x)
    assert got.size == want.size
    assert (got == want).all()
    say("encode mixed spans: decode back")
    d_blob = torch.from_numpy(got).to(DEV)
    d_dec, st = gpu_decode_dev(d_blob, x.size)
    assert st == 0
    assert torch.equal(d_dec, d_x)


def test_layer_of_more_than_64_stripes():
    """A 4.36 GB trunk-recipe layer: 65 full stripes and a partial one. The
    decoder keeps stripe values for blocks of 64 stripes and must reload them
    when a unit falls in the next block; the GPU encoder's look-back restarts
    in every stripe. The GPU encoder's container must equal the native
    packer's (which equals the oracle's byte for byte on every other layer
    here; the oracle's encoder needs about two minutes for this size), its
    code lengths, stripe bit counts and three of its stripes are checked
    against the oracle, and decoding it must give the layer back."""
    n = (65 << 26) + 3 * 65536 + 1234
    x = synth.trunk_layer(synth.SEED_BASE + 77, n_bytes=n)
    want = k3huf.encode_layer(x)
    assert k3huf.layer_info(want)["n_stripes"] == 66
    say("encode and decode 66 stripes", x.size)
    d_x = torch.from_numpy(x).to(DEV)
    d_blob = k3huf.encode_layer_dev(d_x, *garbage_buffers(x.size))
    assert d_blob.numel() == want.size
    assert torch.equal(d_blob, torch.from_numpy(want).to(DEV))
    say("66 stripes: decode")
    d_dec, st = gpu_decode_dev(d_blob, x.size)
    assert st == 0
    assert torch.equal(d_dec, d_x)
    # oracle checks of the GPU's container that stay within seconds: its
    # code lengths are the oracle's for the layer's histogram, every stripe's
    # bit count is the closed form sum(count * length), and the oracle's
    # bit-by-bit decode of stripes 0, 64 and 65 gives the layer's bytes
    blob = d_blob.cpu().numpy()
    info = k3huf.layer_info(blob)
    hist = np.bincount(x[1::2], minlength=256)
    assert (info["codelen"] == O.code_lengths(hist)).all()
    lens = info["codelen"].astype(np.int64)
    for s in range(66):
        off = int(np.frombuffer(bytes(blob[304 + 8 * s: 312 + 8 * s]), "<u8")[0])
        n_bits = int(np.frombuffer(bytes(blob[off + 8: off + 12]), "<u4")[0])
        hs = np.bincount(x[(s << 26) + 1: min(x.size, (s + 1) << 26): 2], minlength=256)
        assert n_bits == int((hs * lens).sum()), s
    for s in (0, 64, 65):
        size = min(1 << 26, x.size - (s << 26))
        assert (O.decode_stripes(blob, s, 1, size) == x[s << 26: (s << 26) + size]).all(), s


def test_encode_reuses_buffers_across_calls():
    """Two calls in a row on the same output and work buffers, the second
    with a smaller layer: both containers equal the oracle's (scratch state of
    the first call must not leak into the second)."""
    big = synth.small_random(901, 5 * 65536 + 66)
    small = synth.small_random(902, 2 * 65536 + 10)
    d_out, d_work = garbage_buffers(big.size)
    say("encode reuse")
    a, _ = gpu_encode(big, d_out, d_work)
    b, _ = gpu_encode(small, d_out, d_work)
    assert (a == O.encode_layer(big)).all()
    assert (b == O.encode_layer(small)).all()


def test_encode_round_trip_through_gpu_decode():
    x = synth.small_random(4242, (1 << 26) + 5 * 65536 + 1000)
    say("encode round trip", x.size)
    d_x = torch.from_numpy(x).to(DEV)
    d_blob = k3huf.encode_layer_dev(d_x)
    d_dec, st = gpu_decode_dev(d_blob, x.size)
    assert st == 0 and torch.equal(d_dec, d_x)


def test_encode_bad_arguments_raise():
    d_x = torch.zeros(1024, dtype=torch.uint8, device=DEV)
    say("encode bad args")
    with pytest.raises(k3huf.K3HufError):
        k3huf.encode_layer_dev(d_x[:1023])                                  # odd size
    small_out = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(k3huf.K3HufError):
        k3huf.encode_layer_dev(d_x, d_out=small_out)                        # capacity
    small_work = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(k3huf.K3HufError):
        k3huf.encode_layer_dev(d_x, d_work=small_work)                      # work size
