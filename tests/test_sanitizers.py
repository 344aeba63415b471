"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU oracle and
of the library's host code (table builders, header parsers, packers), run on
seeded fuzz: truncated containers, random bit flips in headers, records and
bitstreams, random code-length vectors. Host code only: no GPU code is built
with a sanitizer. Each harness must finish clean (any report aborts it)."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=ENV)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.startswith("ok "), r.stdout


@pytest.mark.slow
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "fuzz_oracle")
    subprocess.check_call(["gcc", "-std=c99", "-Wall", *SAN, "-o", exe,
                           os.path.join(ROOT, "tests", "native", "fuzz_oracle.c"),
                           os.path.join(ROOT, "oracle", "k3huf_oracle.c"),
                           os.path.join(ROOT, "oracle", "e8huf_oracle.c")])
    _run(exe)


@pytest.mark.slow
def test_library_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "fuzz_host")
    csrc = os.path.join(ROOT, "lossless_huffman_decoding_amd", "csrc")
    subprocess.check_call(["g++", "-std=c++17", "-Wall", "-pthread", *SAN,
                           "-I" + os.path.join(ROOT, "include"), "-I" + csrc, "-o", exe,
                           os.path.join(ROOT, "tests", "native", "fuzz_host.cpp"),
                           os.path.join(csrc, "k3huf_host.cpp"), os.path.join(csrc, "e8huf_host.cpp")])
    _run(exe)
