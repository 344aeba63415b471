"""MI355X-native lossless decoding of bf16 layers whose high-byte plane is
coded with a 12-bit length-limited canonical Huffman code.

Modules:
  k3huf    -- ctypes binding of the C-ABI library (libk3huf.so, HIP kernels)
  ondemand -- decode-on-demand of compressed module weights (forward pre-hook)
  synth    -- seeded synthetic bf16 layers (inputs for tests and benchmarks)
  _build   -- compiles the library for gfx950
"""

__all__ = ["k3huf", "ondemand", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
