"""k3huf_encode_layer_dev_static, the GPU encoder that allocates nothing (its
work buffer is a library-owned device array), against k3huf_encode_layer_dev
(caller's work buffer) through the C ABI: two calls in a row, the second on a
smaller layer, so that what the first call left in the array must not leak
into the second container. Both containers must be equal byte for byte, and
equal to the oracle's encoder."""

import numpy as np
import pytest
import torch

import oracle as O
from lossless_huffman_decoding_amd import k3huf, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[gpu-case]", *a, flush=True)


def test_static_encoder_equals_the_allocating_encoder():
    layers = [synth.small_random(801, (1 << 26) + 5 * 65536 + 514),   # two stripes, ragged tail
              synth.small_random(802, 3 * 65536 + 130)]               # then a smaller layer
    for x in layers:
        d_x = torch.from_numpy(x).to(DEV)
        cap = k3huf.encode_bound(x.size)
        d_a = torch.full((cap,), 0x5A, dtype=torch.uint8, device=DEV)
        d_b = torch.full((cap,), 0xA5, dtype=torch.uint8, device=DEV)
        d_work = torch.full((k3huf.encode_work_bytes(x.size),), 0x33, dtype=torch.uint8, device=DEV)
        torch.cuda.synchronize()
        say("static encoder", x.size)
        a = k3huf.encode_layer_dev(d_x, d_a, d_work)
        b = k3huf.encode_layer_dev_static(d_x, d_b)
        assert a.numel() == b.numel()
        assert torch.equal(a, b)
        want = O.encode_layer(x)
        assert b.numel() == want.size and np.array_equal(b.cpu().numpy(), want)
