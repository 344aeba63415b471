"""Decode-on-demand of compressed bf16 and FP8 module weights.

The ECF8 page (pwwt.cn/news/2030120), section 2.2 ("zero-copy tensor
management"), keeps weights compressed in device memory, pre-allocates a
decompression buffer the size of the largest layer, and decodes a layer's
weights into it from a forward pre-hook just before the layer runs. This
module does that with this library's codec. A group of modules (a trunk
layer: the K3 page packs each layer's tensors together, with one code table
per layer) is packed on the GPU as one container (k3huf_encode_layer_dev_lanes,
in the lane-chunk layout k3huf_lane_syms_for picks for its size) of its
weights laid end to end; only the container and its 4096-entry table stay
resident. When a member module is about to run, its group is decoded (once)
into a buffer and every member's weight becomes a view of its slice.

FP8 weights (float8_e4m3fn, float8_e5m2: the ECF8 page's case) are packed
instead in the FP8 exponent format (e8huf_encode, the library's native host
packer: the group's bytes go to the host once, at attach time) with its
two-level table, and decoded by e8huf_decode into the same buffers. The
members of one group share one dtype; groups of either kind mix freely.
With fp8_as=torch.bfloat16 (or torch.float16) FP8 groups are decoded by
e8huf_decode_widen straight into that type instead (scale 1: every E4M3 and
E5M2 value is exact in bfloat16, and every E5M2 value in half), as the
page's decoder hands over 16-bit floats: members then see 16-bit weights
holding their FP8 values, and no widening pass runs before their products.

Two schedules:
  - lookahead=False (default): one buffer; the group's decode is queued on
    the current stream. Work on one stream runs in order, so a decode never
    overwrites weights an earlier module is still reading.
  - lookahead=True: two buffers used in turn, groups in attach
    order (the two-slot ring of the K3 TUNING page, section 2, applied to
    module groups). When group k starts, group k + 1 (after the last group:
    group 0) is decoded into the other buffer on a side stream, once the
    group that last used that buffer has finished (events recorded by forward
    hooks); the current stream waits for group k's decode. A group whose
    decode is not the one pending in its buffer (groups run out of order) is
    decoded in place first. On MI355X this is not faster: the decode kernel
    holds every CU's LDS for its whole grid, so a decode on the side stream
    runs beside the matrix products only at its edges, and both are bound by
    HBM bandwidth anyway.

Everything here is marshalling around the HIP kernels: packing and decoding
run in libk3huf.so; PyTorch supplies device memory, streams, events and the
hooks.
"""

from __future__ import annotations

import numpy as np
import torch

from . import e8huf, k3huf

# FP8 dtypes and the width of their exponent field
_FP8_EXP_BITS = {torch.float8_e4m3fn: 4, torch.float8_e5m2: 5}


class OnDemandWeights:
    """Hold modules' bf16 or FP8 weights compressed in HBM; decode each
    group on use.

    ``attach(module)`` makes a group of one; ``attach_group(modules)`` packs
    the modules' weights together. Attach in the order the groups run. The
    dense weights are freed. ``fp8_as`` (None, torch.bfloat16 or
    torch.float16) is the type FP8 weights are handed to their modules in
    (None: FP8 as stored). ``buffer_bytes`` reports the decode buffers (one
    or two of the largest group's decoded size); ``resident_bytes`` the
    containers and tables kept in HBM. ``status`` is the device word the
    decodes flag malformed input in (read by ``check()``, which
    synchronizes).
    """

    def __init__(self, device="cuda:0", lookahead: bool = False, fp8_as=None):
        if fp8_as not in (None, torch.bfloat16, torch.float16):
            raise ValueError("fp8_as: None (FP8 bytes), torch.bfloat16 or torch.float16")
        self.device = torch.device(device)
        self.lookahead = lookahead
        self.fp8_as = fp8_as
        n = 2 if lookahead else 1
        self._bufs = [torch.empty(0, dtype=torch.uint8, device=self.device) for _ in range(n)]
        self._groups = []
        self._by_module = {}
        self._handles = []
        self._pending = [None] * n   # group whose decode each buffer holds or awaits
        self.status = torch.zeros(1, dtype=torch.int32, device=self.device)
        # decodes may run on any stream: the cleared status must be in place
        torch.cuda.current_stream(self.device).synchronize()
        self._lib = e8huf.lib()   # (loads libk3huf.so and declares both codecs' calls)
        self._decoded = [torch.cuda.Event() for _ in range(n)]
        if lookahead:
            self._side = torch.cuda.Stream(device=self.device)
            self._free = [torch.cuda.Event() for _ in range(n)]

    @property
    def buffer_bytes(self) -> int:
        return sum(b.numel() for b in self._bufs)

    @property
    def resident_bytes(self) -> int:
        return sum(g["blob"].numel() + g["lut"].numel() * 2 for g in self._groups)

    def attach(self, module: torch.nn.Module, name: str = "weight") -> None:
        self.attach_group([module], name)

    def attach_group(self, modules, name: str = "weight") -> None:
        members, parts, off, dtype = [], [], 0, None
        for m in modules:
            w = getattr(m, name)
            if (w is None or w.device != self.device
                    or (w.dtype != torch.bfloat16 and w.dtype not in _FP8_EXP_BITS)):
                raise ValueError("decode-on-demand needs bf16, float8_e4m3fn or float8_e5m2 weights on %s"
                                 % self.device)
            if dtype is not None and w.dtype != dtype:
                raise ValueError("the weights of one group must share a dtype (%s, %s)" % (dtype, w.dtype))
            dtype = w.dtype
            raw = w.detach().contiguous().view(torch.uint8).reshape(-1)
            members.append((m, off, raw.numel(), tuple(w.shape)))
            parts.append(raw)
            off += raw.numel()
        if not members:
            raise ValueError("an empty group")
        raw = parts[0] if len(parts) == 1 else torch.cat(parts)
        if dtype == torch.bfloat16:
            # the lane-chunk layout by the library's rule (64-symbol chunks for
            # containers of up to 16 MiB, whose decode is one lane's chain of
            # lookups); trimmed copy, the bound-sized output is freed
            blob = k3huf.encode_layer_dev(raw, lane_syms=k3huf.lane_syms_for(raw.numel())).clone()
            info = k3huf.layer_info(blob[: k3huf.HDR_BYTES].cpu().numpy())
            lut = torch.from_numpy(k3huf.build_table(info["codelen"]).view(np.int16)).to(self.device)
            fn, fname = self._lib.k3huf_decode_layer, "k3huf_decode_layer"
        else:
            eb = _FP8_EXP_BITS[dtype]
            hblob = e8huf.encode(raw.cpu().numpy(), exp_bits=eb)
            info = e8huf.layer_info(hblob[: e8huf.HDR_BYTES])
            blob = torch.from_numpy(hblob).to(self.device)
            lut = torch.from_numpy(e8huf.build_table(info["codelen"], eb).view(np.int16)).to(self.device)
            if self.fp8_as is None:
                fn, fname = self._lib.e8huf_decode, "e8huf_decode"
            else:
                fn, fname = self._lib.e8huf_decode_widen, "e8huf_decode_widen"
        del raw, parts
        # what the buffer holds for this group: its dtype and bytes per value
        # of the weights (FP8 widened: 2 bytes per FP8 byte)
        out_dtype = dtype if dtype == torch.bfloat16 or self.fp8_as is None else self.fp8_as
        k = 2 if (dtype != torch.bfloat16 and self.fp8_as is not None) else 1
        g = {"blob": blob, "lut": lut, "raw_bytes": off, "name": name, "members": members,
             "index": len(self._groups), "dtype": dtype, "out_dtype": out_dtype, "k": k, "fn": fn,
             "fname": fname}
        self._groups.append(g)
        if any(off * k > b.numel() for b in self._bufs):
            # a larger buffer replaces the old one: decodes and forwards still
            # queued may use the old one (on any stream), and what it holds
            # does not carry over
            torch.cuda.synchronize(self.device)
            for i, b in enumerate(self._bufs):
                if off * k > b.numel():
                    self._bufs[i] = torch.empty(off * k, dtype=torch.uint8, device=self.device)
                    self._pending[i] = None
        # per buffer: the decode call's arguments and the members' weight views
        # (the hooks run per forward, so they only look these up)
        # (every decode call ends in stream, status)
        for x in self._groups:
            x["calls"] = [(x["blob"].data_ptr(), x["blob"].numel(), x["lut"].data_ptr(), b.data_ptr(),
                           x["raw_bytes"]) if x["dtype"] == torch.bfloat16 else
                          (x["blob"].data_ptr(), x["blob"].numel(), x["lut"].data_ptr(), x["lut"].numel(),
                           b.data_ptr(), x["raw_bytes"]) if x["k"] == 1 else
                          (x["blob"].data_ptr(), x["blob"].numel(), x["lut"].data_ptr(), x["lut"].numel(),
                           b.data_ptr(), x["raw_bytes"],
                           e8huf.OUT_BF16 if x["out_dtype"] == torch.bfloat16 else e8huf.OUT_F16, 1.0)
                          for b in self._bufs]
            x["views"] = [[b[o * x["k"]: (o + n) * x["k"]].view(x["out_dtype"]).view(shape)
                           for (_, o, n, shape) in x["members"]] for b in self._bufs]
        for j, (m, _, _, _) in enumerate(members):
            self._by_module[id(m)] = (g, j)
            if name in m._parameters:
                del m._parameters[name]
            setattr(m, name, None)
            self._handles.append(m.register_forward_pre_hook(self._pre_hook))
            if self.lookahead:
                self._handles.append(m.register_forward_hook(self._post_hook))

    def _decode(self, g, slot: int, stream_handle: int) -> None:
        rc = g["fn"](*g["calls"][slot], stream_handle, self.status.data_ptr())
        if rc:
            raise k3huf.K3HufError(rc, g["fname"])

    def _pre_hook(self, module, inputs):
        g, j = self._by_module[id(module)]
        k = g["index"]
        cur = torch.cuda.current_stream(self.device)
        if not self.lookahead:
            # (a stream other than the one that decoded the group waits for it;
            # forwards on different streams must not overlap: one buffer)
            slot = 0
            if self._pending[0] != k:
                self._decode(g, 0, cur.cuda_stream)
                self._decoded[0].record(cur)
                self._pending[0] = k
            else:
                cur.wait_event(self._decoded[0])
        else:
            slot = k % 2
            if self._pending[slot] != k:
                # not prefetched: decode in place after the buffer's last user
                self._side.wait_event(self._free[slot])
                self._decode(g, slot, self._side.cuda_stream)
                self._decoded[slot].record(self._side)
                self._pending[slot] = k
            cur.wait_event(self._decoded[slot])
            # prefetch the next group into the other buffer once its last user
            # is done (not when the wrap-around lands in this group's buffer)
            n = (k + 1) % len(self._groups)
            ns = n % 2
            if ns != slot and self._pending[ns] != n:
                self._side.wait_event(self._free[ns])
                self._decode(self._groups[n], ns, self._side.cuda_stream)
                self._decoded[ns].record(self._side)
                self._pending[ns] = n
        setattr(module, g["name"], g["views"][slot][j])

    def _post_hook(self, module, inputs, output):
        g, _ = self._by_module[id(module)]
        self._free[g["index"] % 2].record(torch.cuda.current_stream(self.device))

    def check(self) -> None:
        """Raise if any decode so far flagged malformed input (synchronizes).
        The word holds the codecs' own device bits (K3HUF_DEV_* from bf16
        groups, E8HUF_DEV_* from FP8 groups), OR-ed together."""
        torch.cuda.synchronize(self.device)
        st = int(self.status.item())
        if st:
            raise k3huf.K3HufError(k3huf.E_CORRUPT, "on-demand decode (device status %#x)" % st)

    def detach(self) -> None:
        for h in self._handles:
            h.remove()
        self._handles.clear()
