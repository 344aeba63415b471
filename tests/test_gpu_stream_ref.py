"""The bandwidth reference kernel (k3huf_stream_ref) writes what its header
says: output unit u is input unit u while the input lasts, then
{u mod 2^32, 0, 0, 0}. Every case prints its name before touching the GPU."""

import numpy as np
import pytest
import torch

from lossless_huffman_decoding_amd import k3huf

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[gpu-case]", *a, flush=True)


@pytest.mark.parametrize("in_units,out_units,grid,nt", [(0, 1, 1, 0), (5, 3, 1, 1), (256, 256, 2, 0),
                                                         (1000, 4099, 3, 1), (70000, 65536, 7, 0),
                                                         (50000, 131072, 1024, 1)])
def test_stream_ref_writes_the_documented_units(in_units, out_units, grid, nt):
    rng = np.random.default_rng(in_units * 7 + out_units)
    src = rng.integers(0, 256, 16 * in_units, dtype=np.uint8)
    say("stream ref", in_units, out_units, grid, nt)
    d_in = torch.from_numpy(src).to(DEV) if in_units else None
    d_out = torch.full((16 * out_units,), 0xA5, dtype=torch.uint8, device=DEV)
    k3huf.stream_ref(d_in, d_out, grid, bool(nt))
    torch.cuda.synchronize()
    got = d_out.cpu().numpy().view(np.uint32).reshape(-1, 4)
    want = np.zeros((out_units, 4), np.uint32)
    k = min(in_units, out_units)
    want[:k] = src.view(np.uint32).reshape(-1, 4)[:k]
    want[k:, 0] = np.arange(k, out_units, dtype=np.uint64).astype(np.uint32)
    assert (got == want).all()
