"""Decode-on-demand of module weights (ECF8 page, section 2.2: one buffer the
size of the largest layer, filled by a forward pre-hook before each layer).

The decoded weights are the original bf16 or FP8 bytes, so a forward pass
through the hooked modules must equal the dense forward pass bit for bit. Every case
prints its name before touching the GPU.
"""

import pytest
import torch

from lossless_huffman_decoding_amd import k3huf, synth
from lossless_huffman_decoding_amd.ondemand import OnDemandWeights

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[gpu-case]", *a, flush=True)


def _trunk_like(rows, cols, seed):
    """A bf16 weight drawn like a trunk matrix (N(0, s), s log-uniform in
    [0.005, 0.05]); the generator lives in synth."""
    raw = synth.small_trunk_matrix(seed, rows, cols)
    return torch.from_numpy(raw).view(torch.bfloat16).view(rows, cols)


def _stack(shapes, seed):
    layers = []
    for k, (o, i) in enumerate(shapes):
        lin = torch.nn.Linear(i, o, bias=(k % 2 == 0), dtype=torch.bfloat16, device=DEV)
        with torch.no_grad():
            lin.weight.copy_(_trunk_like(o, i, seed + k).to(DEV))
        layers.append(lin)
    return torch.nn.Sequential(*layers)


@pytest.mark.parametrize("batch,lookahead,n_layers", [(1, False, 4), (7, False, 4), (1, True, 4),
                                                      (7, True, 3), (2, True, 1)])
def test_on_demand_forward_equals_dense(batch, lookahead, n_layers):
    shapes = [(1024, 512), (768, 1024), (1536, 768), (512, 1536)][:n_layers]
    if n_layers < 4:
        shapes[-1] = (512, shapes[-1][1])   # the stack still maps 512 -> 512
    model = _stack(shapes, 600)
    x = torch.randn(batch, 512, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    dense = [m.weight.detach().clone() for m in model]
    say("ondemand dense forward", batch)
    with torch.no_grad():
        want = model(x)
        dense_first = model[0](x)
    od = OnDemandWeights(DEV, lookahead=lookahead)
    for m in model:
        od.attach(m)
    assert od.buffer_bytes == max(o * i for o, i in shapes) * 2 * (2 if lookahead else 1)
    assert od.resident_bytes < sum(o * i for o, i in shapes) * 2
    # modules of a few MB get the 64-symbol lane-chunk layout
    assert all(k3huf.layer_info(g["blob"][: k3huf.HDR_BYTES].cpu().numpy())["lane_syms"] == 64
               for g in od._groups)
    say("ondemand hooked forward", batch, lookahead, n_layers)
    with torch.no_grad():
        got = model(x)
        got2 = model(x)             # buffers reused across passes
        got3 = model[0](x)          # a module out of order
    od.check()
    assert torch.equal(got, want) and torch.equal(got2, want)
    assert torch.equal(got3, dense_first)
    assert torch.equal(model[0].weight, dense[0])


@pytest.mark.parametrize("lookahead", [False, True])
def test_on_demand_on_a_side_stream(lookahead):
    model = _stack([(640, 320), (320, 640)], 700)
    x = torch.randn(3, 320, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16).to(DEV)
    with torch.no_grad():
        want = model(x)
    od = OnDemandWeights(DEV, lookahead=lookahead)
    for m in model:
        od.attach(m)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())   # x and the weights were made on the current stream
    say("ondemand side stream", lookahead)
    with torch.cuda.stream(s), torch.no_grad():
        got = model(x)
    od.check()
    assert torch.equal(got, want)


@pytest.mark.parametrize("weights", ["bf16", "fp8", "fp8_as_bf16"])
def test_on_demand_forward_captured_in_a_graph(weights):
    """The hooked forward (one buffer, decodes on the capturing stream)
    captured once and replayed: every replay equals the dense forward, with
    eager work and synchronizations between replays. fp8: E4M3, E5M2 and
    bf16 modules, so the graph holds both codecs' decodes."""
    shapes = [(1024, 512), (768, 1024), (512, 768)]
    model = (_stack(shapes, 800) if weights == "bf16" else
             _fp8_stack(shapes, ["e4m3", "bf16", "e5m2"], 850))
    x = torch.randn(4, 512, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16).to(DEV)
    with torch.no_grad():
        want = model(x)
    od = OnDemandWeights(DEV, lookahead=False, fp8_as=torch.bfloat16 if weights == "fp8_as_bf16" else None)
    for m in model:
        od.attach(m)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("ondemand graph capture", weights)
    with torch.cuda.stream(s), torch.no_grad():
        model(x)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g), torch.no_grad():
        out = model(x)
    for r in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), r
        with torch.no_grad():
            eager = model(x)        # eager decodes between replays
        torch.cuda.synchronize()
        assert torch.equal(eager, want), r
    od.check()


@pytest.mark.parametrize("lookahead", [False, True])
def test_on_demand_groups(lookahead):
    """Modules packed in groups (one container per group, as a trunk layer
    packs all its tensors with one table): three groups of mixed sizes, run
    twice; every output equals the dense forward."""
    shapes = [(640, 512), (512, 640), (768, 512), (512, 768), (1024, 512), (512, 1024), (512, 512)]
    model = _stack(shapes, 1000)
    x = torch.randn(5, 512, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16).to(DEV)
    with torch.no_grad():
        want = model(x)
    od = OnDemandWeights(DEV, lookahead=lookahead)
    groups = [[model[0], model[1]], [model[2], model[3], model[4]], [model[5], model[6]]]
    for grp in groups:
        od.attach_group(grp)
    biggest = max(sum(m.in_features * m.out_features * 2 for m in grp) for grp in groups)
    assert od.buffer_bytes == biggest * (2 if lookahead else 1)
    say("ondemand groups", lookahead)
    with torch.no_grad():
        a = model(x)
        b = model(x)
    od.check()
    assert torch.equal(a, want) and torch.equal(b, want)


@pytest.mark.parametrize("lookahead", [False, True])
def test_on_demand_attach_after_a_forward(lookahead):
    """Modules attached after forwards have run: a larger group replaces the
    decode buffers, so the groups decoded into the old ones are decoded
    again on their next use rather than read from the new, unwritten
    buffers."""
    model = _stack([(512, 256), (256, 512), (1024, 256), (256, 1024)], 1100)
    x = torch.randn(4, 256, generator=torch.Generator().manual_seed(11)).to(torch.bfloat16).to(DEV)
    with torch.no_grad():
        want01 = model[1](model[0](x))
        want = model(x)
    od = OnDemandWeights(DEV, lookahead=lookahead)
    od.attach_group([model[0], model[1]])
    say("ondemand attach after a forward", lookahead)
    with torch.no_grad():
        first = model[1](model[0](x))
    small = od.buffer_bytes
    od.attach_group([model[2], model[3]])    # twice the bytes: new buffers
    assert od.buffer_bytes == 2 * small
    with torch.no_grad():
        again = model[1](model[0](x))        # group 0 again, into the new buffers
        full = model(x)
    od.check()
    assert torch.equal(first, want01) and torch.equal(again, want01) and torch.equal(full, want)


class _FP8Linear(torch.nn.Module):
    """A weight-only FP8 linear map: y = x (scale * W)^T, W held as FP8 and
    widened to bf16 on use (the ECF8 page's setting: FP8 weights, decoded
    from their compressed form just before the layer runs)."""

    def __init__(self, w, scale):
        super().__init__()
        self.weight = torch.nn.Parameter(w, requires_grad=False)
        self.scale = scale

    def forward(self, x):
        return torch.nn.functional.linear(x, self.weight.to(torch.bfloat16) * self.scale)


def _fp8_stack(shapes, fmts, seed):
    layers = []
    for k, ((o, i), fmt) in enumerate(zip(shapes, fmts)):
        if fmt == "bf16":
            lin = torch.nn.Linear(i, o, bias=False, dtype=torch.bfloat16, device=DEV)
            with torch.no_grad():
                lin.weight.copy_(_trunk_like(o, i, seed + k).to(DEV))
        else:
            dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
            raw = synth.e8_small(seed + k, o * i, fmt)
            w = torch.from_numpy(raw).view(dt).view(o, i).to(DEV)
            lin = _FP8Linear(w, 0.03 / synth.FP8_MAX[fmt])
        layers.append(lin)
    return torch.nn.Sequential(*layers)


@pytest.mark.parametrize("fp8_as", [None, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("lookahead", [False, True])
def test_on_demand_fp8_weights(lookahead, fp8_as):
    """FP8 weights (E4M3 and E5M2 groups) beside a bf16 group: each FP8
    group is one E8HF container decoded into the shared buffers, as FP8
    bytes (e8huf_decode) or widened to 16-bit floats (e8huf_decode_widen;
    the modules' own widening is then a no-op or exact). Every forward equals
    the dense one bit for bit, the views hold the original values, and the
    containers are smaller than the weights."""
    shapes = [(1024, 512), (768, 1024), (512, 768), (640, 512), (512, 640)]
    fmts = ["e4m3", "e4m3", "bf16", "e5m2", "e5m2"]
    model = _fp8_stack(shapes, fmts, 1100)
    x = torch.randn(3, 512, generator=torch.Generator().manual_seed(11)).to(torch.bfloat16).to(DEV)
    dense = [m.weight.detach().clone() for m in model]
    say("ondemand fp8 dense forward", lookahead, fp8_as)
    with torch.no_grad():
        want = model(x)
        want_last = model[4](model[3](torch.ones(2, 512, dtype=torch.bfloat16, device=DEV)))
    od = OnDemandWeights(DEV, lookahead=lookahead, fp8_as=fp8_as)
    od.attach_group([model[0], model[1]])
    od.attach(model[2])
    od.attach_group([model[3], model[4]])
    weight_bytes = [1024 * 512 + 768 * 1024, 512 * 768 * 2, 640 * 512 * 2]
    wide = 1 if fp8_as is None else 2
    buffer_bytes = [weight_bytes[0] * wide, weight_bytes[1], weight_bytes[2] * wide]
    assert od.buffer_bytes == max(buffer_bytes) * (2 if lookahead else 1)
    assert od._groups[0]["blob"][:4].cpu().numpy().tobytes() == b"E8HF"
    assert od._groups[1]["blob"][:4].cpu().numpy().tobytes() == b"K3HF"
    fp8_blobs = od._groups[0]["blob"].numel() + od._groups[2]["blob"].numel()
    assert fp8_blobs < weight_bytes[0] + weight_bytes[2] // 2
    say("ondemand fp8 hooked forward", lookahead, fp8_as)
    with torch.no_grad():
        got = model(x)
        got2 = model(x)
        got_last = model[4](model[3](torch.ones(2, 512, dtype=torch.bfloat16, device=DEV)))
    od.check()
    assert torch.equal(got, want) and torch.equal(got2, want)
    assert torch.equal(got_last, want_last)
    # the weight each module sees right after its own decode (the buffers are
    # shared, so an earlier module's view holds a later group's bytes)
    for (o, i), m, d in zip(shapes, model, dense):
        with torch.no_grad():
            m(torch.ones(1, i, dtype=torch.bfloat16, device=DEV))
        assert m.weight.shape == (o, i)
        if d.dtype == torch.bfloat16 or fp8_as is None:
            assert m.weight.dtype == d.dtype
            assert torch.equal(m.weight.view(torch.uint8), d.view(torch.uint8))
        else:
            assert m.weight.dtype == fp8_as
            assert torch.equal(m.weight.view(torch.int16), d.to(fp8_as).view(torch.int16))
    od.check()


def test_on_demand_rejects_what_it_cannot_hold():
    """Argument errors are raised at attach time, before any weight is
    touched: a group mixing dtypes, an unsupported dtype, a weight on the
    host, an empty group and an unsupported fp8_as."""
    say("ondemand argument errors")
    with pytest.raises(ValueError):
        OnDemandWeights(DEV, fp8_as=torch.float32)
    od = OnDemandWeights(DEV)
    a = torch.nn.Linear(64, 32, bias=False, dtype=torch.bfloat16, device=DEV)
    b = _FP8Linear(torch.zeros(32, 64, dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn), 1.0)
    with pytest.raises(ValueError):
        od.attach_group([a, b])
    with pytest.raises(ValueError):
        od.attach(torch.nn.Linear(64, 32, bias=False, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        od.attach(torch.nn.Linear(64, 32, bias=False, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        od.attach_group([])
    assert od.resident_bytes == 0 and a.weight is not None and b.weight is not None
