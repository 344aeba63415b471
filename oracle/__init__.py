"""CPU oracle for the bf16 high-byte Huffman codec -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. It shares no code with the product library.
"""
from .oracle import *  # noqa: F401,F403
