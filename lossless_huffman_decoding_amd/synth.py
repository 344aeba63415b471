"""Seeded synthetic bf16 layers for the decoder's workloads.

This module only draws numbers and rounds them to bf16; it holds none of the
codec's arithmetic (no histograms, code lengths or bit packing), so both the
CPU oracle's tests and the GPU path's tests and benchmark may use it.

The shapes and distributions stand in for the real bf16 trunk bytes the pages
measured (Kimi K3 trunk compression page, sections on background and on the
entropy of the bf16 high byte: layers of ~1.17 GB, a high byte of ~2.8 bit);
the heavy-tailed layer follows the ECF8 page's alpha-stable weight model
(section 1.1). The real bytes are not available, so every config is drawn here
from a numpy PCG64 generator with a fixed seed.

Every generator returns a C-contiguous ``numpy.uint8`` array holding the layer's
little-endian bf16 bytes (even offsets: low/mantissa byte, odd offsets: high
sign+exponent byte).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_BASE = 20260729

# one "trunk layer" is 1.17 decimal GB of bf16 (93 layers make 108.81 GB)
TRUNK_LAYER_BYTES = 1_170_000_000

# repeating tensor cycle of a trunk layer: ("W", rows, cols) weight matrices with
# a per-tensor scale, ("g", n) 1-D norm gains around 1.0
TRUNK_CYCLE = (
    ("W", 7168, 7168),
    ("g", 7168),
    ("W", 7168, 2048),
    ("W", 2048, 7168),
    ("W", 7168, 576),
    ("g", 7168),
)


def f64_to_bf16_bytes(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 via float32, round-to-nearest-even on the
    float32 bit pattern, and return the little-endian bf16 bytes (uint8)."""
    f32 = np.ascontiguousarray(x, dtype=np.float32)
    u = f32.view(np.uint32)
    # RNE: add 0x7FFF plus the lowest kept bit, then drop the low 16 bits.
    # Inputs are finite, so u + 0x8000 cannot wrap and no NaN case is needed.
    r = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    return r.view(np.uint8)


# Large layers are drawn in fixed chunks of CHUNK values; chunk c of stream
# `key` uses numpy.random.default_rng(key + (c,)), so chunks are independent
# and can be drawn on several threads without changing the result.
CHUNK = 1 << 22


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill_chunks(out: np.ndarray, v0: int, n: int, key: tuple, draw) -> None:
    """Write n bf16 values starting at value index v0 of ``out``; chunk c gets
    ``draw(rng, m)`` (float64) with rng seeded by key + (c,)."""
    def job(c):
        p = c * CHUNK
        m = min(CHUNK, n - p)
        rng = np.random.default_rng(key + (c,))
        out[2 * (v0 + p): 2 * (v0 + p + m)] = f64_to_bf16_bytes(draw(rng, m))
    nch = -(-n // CHUNK)
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, range(nch)))


def tiny(seed: int = SEED_BASE + 1) -> np.ndarray:
    """4 MiB: 2,097,152 values iid N(0, 0.02) rounded to bf16 (one partial stripe)."""
    rng = np.random.default_rng(seed)
    return f64_to_bf16_bytes(rng.standard_normal(2_097_152) * 0.02)


def trunk_layer(seed: int = SEED_BASE + 2, n_bytes: int = TRUNK_LAYER_BYTES) -> np.ndarray:
    """A trunk-layer-sized buffer: the TRUNK_CYCLE repeated and truncated to
    ``n_bytes``. Tensor t (counting from 0 along the layer) is drawn from
    the streams keyed (seed, t); a weight matrix is N(0, s) with its own s
    log-uniform in [0.005, 0.05] (drawn first from default_rng((seed, t))),
    a gain vector is N(1.0, 0.05)."""
    if n_bytes % 2:
        raise ValueError("bf16 layer needs an even byte count")
    n_vals = n_bytes // 2
    out = np.empty(n_bytes, dtype=np.uint8)
    pos = 0
    t = 0
    lo, hi = math.log(0.005), math.log(0.05)
    while pos < n_vals:
        spec = TRUNK_CYCLE[t % len(TRUNK_CYCLE)]
        cnt = spec[1] * spec[2] if spec[0] == "W" else spec[1]
        take = min(cnt, n_vals - pos)
        if spec[0] == "W":
            s = math.exp(np.random.default_rng((seed, t)).uniform(lo, hi))
            _fill_chunks(out, pos, take, (seed, t, 1),
                         lambda rng, m, s=s: rng.standard_normal(m) * s)
        else:
            _fill_chunks(out, pos, take, (seed, t, 1),
                         lambda rng, m: 1.0 + 0.05 * rng.standard_normal(m))
        pos += take
        t += 1
    return out


def _alpha_stable_sym(rng: np.random.Generator, n: int, alpha: float) -> np.ndarray:
    """Symmetric (beta = 0) alpha-stable draws, unit scale, by the
    Chambers-Mallows-Stuck (1976) construction."""
    v = rng.uniform(-math.pi / 2, math.pi / 2, n)
    w = rng.exponential(1.0, n)
    return (np.sin(alpha * v) / np.cos(v) ** (1.0 / alpha)) * (
        np.cos(v - alpha * v) / w) ** ((1.0 - alpha) / alpha)


def heavy(seed: int = SEED_BASE + 3, n_bytes: int = 256 << 20) -> np.ndarray:
    """256 MiB of symmetric alpha-stable (alpha = 1.7, scale 0.01) weights
    clipped to +-64 and rounded to bf16."""
    out = np.empty(n_bytes, dtype=np.uint8)
    _fill_chunks(out, 0, n_bytes // 2, (seed,),
                 lambda rng, m: np.clip(_alpha_stable_sym(rng, m, 1.7) * 0.01, -64.0, 64.0))
    return out


def _fibonacci(k: int) -> list[int]:
    f = [1, 1]
    while len(f) < k:
        f.append(f[-1] + f[-2])
    return f[:k]


def edge_fib40(seed: int = SEED_BASE + 41, n_bytes: int = 16 << 20) -> np.ndarray:
    """High bytes over 40 seeded distinct values with Fibonacci-like counts
    c_k = max(1, floor(F_k * n / sum F)), the residual going to the largest;
    a seeded shuffle orders them. Low bytes uniform. Unlimited Huffman depth
    on these counts is far above 12."""
    n = n_bytes // 2
    rng = np.random.default_rng(seed)
    vals = rng.permutation(256)[:40].astype(np.uint8)
    fib = _fibonacci(40)
    tot = sum(fib)
    counts = [max(1, (f * n) // tot) for f in fib]
    counts[-1] += n - sum(counts)
    hi = np.repeat(vals, counts)
    rng.shuffle(hi)
    out = np.empty(n_bytes, dtype=np.uint8)
    out[1::2] = hi
    out[0::2] = rng.integers(0, 256, n, dtype=np.uint8)
    return out


def edge_single(seed: int = SEED_BASE + 42, n_bytes: int = 16 << 20) -> np.ndarray:
    """Every high byte 0x3C (a one-symbol alphabet); low bytes uniform."""
    rng = np.random.default_rng(seed)
    out = np.empty(n_bytes, dtype=np.uint8)
    out[1::2] = 0x3C
    out[0::2] = rng.integers(0, 256, n_bytes // 2, dtype=np.uint8)
    return out


def edge_uniform(seed: int = SEED_BASE + 43, n_bytes: int = (64 << 20) + 2) -> np.ndarray:
    """High and low bytes uniform over 0..255; 64 MiB + 2 B, so the second
    64 MiB stripe holds a single bf16 value."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, n_bytes, dtype=np.uint8)


def streamed_layer(k: int, n_bytes: int = TRUNK_LAYER_BYTES) -> np.ndarray:
    """Layer k of the 93-layer streamed trunk: a trunk layer with seed
    SEED_BASE + 5000 + k."""
    return trunk_layer(SEED_BASE + 5000 + k, n_bytes)


# name -> list of (layer name, zero-argument generator)
CONFIGS = {
    "tiny": [("tiny", tiny)],
    "trunk": [("trunk", trunk_layer)],
    "heavy": [("heavy", heavy)],
    "edge": [("edge_fib40", edge_fib40), ("edge_single", edge_single),
             ("edge_uniform", edge_uniform)],
}


def small_random(seed: int, n_bytes: int, sigma: float = 0.02) -> np.ndarray:
    """Small N(0, sigma) bf16 buffers for quick tests of odd sizes."""
    rng = np.random.default_rng(seed)
    if n_bytes % 2:
        raise ValueError("bf16 layer needs an even byte count")
    return f64_to_bf16_bytes(rng.standard_normal(n_bytes // 2) * sigma)


def mixed_spans(seed: int, n_bytes: int, lo: int = 4 << 10, hi: int = 160 << 10) -> np.ndarray:
    """Spans of N(0, 0.02) bf16 values alternating with spans of uniform
    random bytes, span lengths uniform over even sizes in [lo, hi] (the first
    span's kind drawn too). With one code table per layer the uniform spans
    take long codes and the weight spans short ones, so stretches of dense
    and sparse bitstream meet at arbitrary offsets."""
    if n_bytes % 2:
        raise ValueError("bf16 layer needs an even byte count")
    rng = np.random.default_rng(seed)
    out = np.empty(n_bytes, dtype=np.uint8)
    pos, uniform = 0, bool(rng.integers(0, 2))
    while pos < n_bytes:
        m = min(n_bytes - pos, 2 * int(rng.integers(lo // 2, hi // 2 + 1)))
        if uniform:
            out[pos:pos + m] = rng.integers(0, 256, m, dtype=np.uint8)
        else:
            out[pos:pos + m] = f64_to_bf16_bytes(rng.standard_normal(m // 2) * 0.02)
        pos += m
        uniform = not uniform
    return out


def fuzz_layer(seed: int, max_bytes: int = 24 << 20) -> tuple[np.ndarray, str]:
    """A seeded random layer for sweeps: an even size log-uniform in
    [2, max_bytes] and one of several high-byte laws (bf16 normals of very
    different scales, uniform bytes, 1-255 live high bytes with Dirichlet
    weights, a Zipf-like law); low bytes uniform unless drawn from bf16
    values. Returns the bytes and a short description."""
    rng = np.random.default_rng((SEED_BASE, 9000, seed))
    n = 2 * max(1, int(math.exp(rng.uniform(0.0, math.log(max_bytes / 2)))))
    law = int(rng.integers(0, 4))
    if law == 0:
        sigma = float(10.0 ** rng.uniform(-5, 3))
        return f64_to_bf16_bytes(rng.standard_normal(n // 2) * sigma), "normal sigma %.3g, %d B" % (sigma, n)
    if law == 1:
        return rng.integers(0, 256, n, dtype=np.uint8), "uniform bytes, %d B" % n
    out = rng.integers(0, 256, n, dtype=np.uint8)
    if law == 2:
        k = int(rng.choice([1, 2, 3, 5, 17, 64, 255]))
        syms = rng.choice(256, size=k, replace=False)
        w = rng.dirichlet(np.full(k, 0.3))
        out[1::2] = syms[rng.choice(k, size=n // 2, p=w)].astype(np.uint8)
        return out, "%d live high bytes (Dirichlet 0.3), %d B" % (k, n)
    a = float(rng.uniform(1.05, 3.0))
    ranks = np.minimum(rng.zipf(a, size=n // 2), 256) - 1
    perm = rng.permutation(256)
    out[1::2] = perm[ranks].astype(np.uint8)
    return out, "Zipf a=%.2f high bytes, %d B" % (a, n)


def small_trunk_matrix(seed: int, rows: int, cols: int) -> np.ndarray:
    """One rows x cols bf16 weight drawn like a trunk matrix: N(0, s) with s
    log-uniform in [0.005, 0.05], both from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    s = math.exp(rng.uniform(math.log(0.005), math.log(0.05)))
    return f64_to_bf16_bytes(rng.standard_normal(rows * cols) * s)


# ---------------------------------------------------------------------------
# FP8 tensors for the exponent codec (ECF8 page, sections 1.2 and 2.1: FP8
# weights, E4M3 or E5M2, whose exponent field is entropy coded). Values are
# drawn as above, scaled per tensor so that the largest magnitude lands on the
# format's largest finite value (a per-tensor amax scale), and rounded to the
# format (round to nearest even) by torch's float8 conversion.

FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}
FP8_EXP_BITS = {"e4m3": 4, "e5m2": 5}

# values of the FP8 trunk layer: the bf16 trunk layer's 585,000,000 values
FP8_TRUNK_VALUES = TRUNK_LAYER_BYTES // 2


def fp8_bytes(x: np.ndarray, fmt: str = "e4m3", amax: float | None = None) -> np.ndarray:
    """Scale x so that max |x| (or ``amax``) maps to the format's largest
    finite value, round to FP8 and return the bytes (uint8). Large arrays are
    handled in CHUNK-value pieces on several threads (the result does not
    depend on the split)."""
    import torch
    x = np.asarray(x, dtype=np.float64)
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    spans = [(p, min(p + CHUNK, x.size)) for p in range(0, x.size, CHUNK)]
    with ThreadPoolExecutor(_workers()) as ex:
        if amax is None:
            amax = max(ex.map(lambda sp: float(np.abs(x[sp[0]:sp[1]]).max()), spans))
        scale = FP8_MAX[fmt] / amax if amax > 0 else 1.0
        out = np.empty(x.size, dtype=np.uint8)

        def conv(sp):
            t = torch.from_numpy((x[sp[0]:sp[1]] * scale).astype(np.float32))
            out[sp[0]:sp[1]] = t.to(dt).view(torch.uint8).numpy()
        list(ex.map(conv, spans))
    return out


def e8_tiny(seed: int = SEED_BASE + 101, fmt: str = "e4m3") -> np.ndarray:
    """4,194,304 FP8 values: iid N(0, 1), per-tensor amax scale."""
    rng = np.random.default_rng(seed)
    return fp8_bytes(rng.standard_normal(4_194_304), fmt)


def e8_small(seed: int, n: int, fmt: str = "e4m3", sigma: float = 1.0) -> np.ndarray:
    """n FP8 values: iid N(0, sigma), per-tensor amax scale (quick tests)."""
    rng = np.random.default_rng((SEED_BASE, 8100, seed))
    if n == 1:
        return fp8_bytes(np.array([sigma * float(rng.standard_normal())]), fmt)
    return fp8_bytes(rng.standard_normal(n) * sigma, fmt)


def e8_trunk(seed: int = SEED_BASE + 102, n_values: int = FP8_TRUNK_VALUES, fmt: str = "e4m3") -> np.ndarray:
    """The trunk layer's tensor cycle as FP8: tensor t is N(0, s_t) (s_t
    log-uniform in [0.005, 0.05]) or N(1, 0.05) gains, each tensor scaled to
    the format by its own amax; truncated to n_values."""
    out = np.empty(n_values, dtype=np.uint8)
    pos, t = 0, 0
    lo, hi = math.log(0.005), math.log(0.05)
    while pos < n_values:
        spec = TRUNK_CYCLE[t % len(TRUNK_CYCLE)]
        cnt = spec[1] * spec[2] if spec[0] == "W" else spec[1]
        take = min(cnt, n_values - pos)
        vals = np.empty(take, dtype=np.float64)

        def job(c, t=t, spec=spec, vals=vals, take=take):
            p = c * CHUNK
            m = min(CHUNK, take - p)
            rng = np.random.default_rng((seed, t, 1, c))
            if spec[0] == "W":
                s = math.exp(np.random.default_rng((seed, t)).uniform(lo, hi))
                vals[p:p + m] = rng.standard_normal(m) * s
            else:
                vals[p:p + m] = 1.0 + 0.05 * rng.standard_normal(m)
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(job, range(-(-take // CHUNK))))
        out[pos:pos + take] = fp8_bytes(vals, fmt)
        pos += take
        t += 1
    return out


def e8_heavy(seed: int = SEED_BASE + 103, n_values: int = 256 << 20, fmt: str = "e4m3") -> np.ndarray:
    """Symmetric alpha-stable (alpha = 1.7, scale 0.01) values clipped to
    +-64, scaled so that 64 maps to the format's largest value (the clip
    bound as amax), as FP8."""
    vals = np.empty(n_values, dtype=np.float64)

    def job(c):
        p = c * CHUNK
        m = min(CHUNK, n_values - p)
        rng = np.random.default_rng((seed, c))
        vals[p:p + m] = np.clip(_alpha_stable_sym(rng, m, 1.7) * 0.01, -64.0, 64.0)
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, range(-(-n_values // CHUNK))))
    return fp8_bytes(vals, fmt, amax=64.0)


def e8_one_exponent(seed: int, n: int, fmt: str = "e4m3") -> np.ndarray:
    """n FP8 values that all share one exponent field (+-[1, 2) scaled to the
    format), random signs and mantissas: a one-symbol exponent plane."""
    rng = np.random.default_rng((SEED_BASE, 8200, seed))
    m = 3 if fmt == "e4m3" else 2
    e = 7 if fmt == "e4m3" else 15
    sign = rng.integers(0, 2, n, dtype=np.uint8) << 7
    mant = rng.integers(0, 1 << m, n, dtype=np.uint8)
    return (sign | np.uint8(e << m) | mant).astype(np.uint8)


def e8_uniform_bytes(seed: int, n: int) -> np.ndarray:
    """n uniformly random bytes (every exponent field equally likely; in E4M3
    this includes the NaN patterns, which the codec keeps like any byte)."""
    return np.random.default_rng((SEED_BASE, 8300, seed)).integers(0, 256, n, dtype=np.uint8)


def e8_fib_exponents(seed: int, n: int, k: int = 18) -> np.ndarray:
    """n E5M2 bytes whose exponent fields 0..k-1 occur with Fibonacci-like
    counts (as in edge_fib40), random signs and mantissas: the unsmoothed
    Huffman tree is deeper than 16 bits."""
    rng = np.random.default_rng((SEED_BASE, 8400, seed))
    f = np.array(_fibonacci(k), dtype=np.float64)
    c = np.maximum(1, np.floor(f * n / f.sum())).astype(np.int64)
    c[-1] += n - c.sum()
    exps = rng.permutation(np.repeat(np.arange(k, dtype=np.uint8), c))
    sign = rng.integers(0, 2, n, dtype=np.uint8) << 7
    mant = rng.integers(0, 4, n, dtype=np.uint8)
    return (sign | (exps << 2) | mant).astype(np.uint8)


def e8_rare_at_edges(seed: int) -> tuple[np.ndarray, np.ndarray]:
    """8 blocks of 16,384 E4M3 values plus a partial block of 700. Exponent
    field f in 4..15 occurs with probability proportional to 2^(f - 15) (a
    chain of code lengths 1..12); two fields (0 and 1) occur only at 18
    listed positions, so their codes are longer than 12 bits. Those
    positions sit at lane-chunk edges (chunks of 256 values: offsets 0, 1,
    254, 255), at the half-chunk edge (offsets 126-130, pairs across it) and
    at the end of the partial block's last lane. Returns the bytes and the
    positions."""
    rng = np.random.default_rng((SEED_BASE, 8500, seed))
    n = 8 * 16384 + 700
    w = 2.0 ** np.arange(-11, 1, dtype=np.float64)
    exps = rng.choice(np.arange(4, 16, dtype=np.uint8), size=n, p=w / w.sum())
    lanes = [0, 17, 63, 5, 40, 63, 31, 1]
    offs = [[0, 1], [126, 127], [127, 128], [128, 129], [129, 130], [254, 255], [255], [0, 255]]
    pos = [b * 16384 + 256 * lanes[b] + o for b in range(8) for o in offs[b]]
    pos += [8 * 16384 + 256 * 1 + 255, 8 * 16384 + 256 * 2 + 186, 8 * 16384 + 256 * 2 + 187]
    pos = np.array(pos, dtype=np.int64)
    exps[pos] = (np.arange(pos.size) % 2).astype(np.uint8)
    sign = rng.integers(0, 2, n, dtype=np.uint8) << 7
    mant = rng.integers(0, 8, n, dtype=np.uint8)
    return (sign | (exps << 3) | mant).astype(np.uint8), pos


def e8_long_codes_in_passes(seed: int, n: int) -> np.ndarray:
    """n E5M2 bytes whose exponent fields 0..19 have probabilities falling by
    a factor 0.86 each and fields 20..31 by a further factor 2 each: the
    codes average about 4 bits, so a block's codes (about 8 KB) exceed a
    6 KiB buffer, and the rare fields get codes of 13-16 bits."""
    rng = np.random.default_rng((SEED_BASE, 8600, seed))
    w = np.concatenate([0.86 ** np.arange(20), 0.86 ** 19 * 0.5 ** np.arange(1, 13)])
    exps = rng.choice(np.arange(32, dtype=np.uint8), size=n, p=w / w.sum())
    sign = rng.integers(0, 2, n, dtype=np.uint8) << 7
    mant = rng.integers(0, 4, n, dtype=np.uint8)
    return (sign | (exps << 2) | mant).astype(np.uint8)


def e8_fuzz_tensor(seed: int, max_values: int = 4 << 20) -> tuple[np.ndarray, int, str]:
    """A seeded random FP8 tensor for sweeps: a size log-uniform in
    [1, max_values], E4M3 or E5M2, and one of several exponent laws (normal
    values of a random scale, uniform bytes, a few live exponent fields with
    Dirichlet weights, Zipf-like exponent ranks, a chain of fields whose
    probabilities fall by a random factor); signs and mantissas uniform
    unless drawn from the values. Returns the bytes, the exponent width and a
    short description."""
    rng = np.random.default_rng((SEED_BASE, 9100, seed))
    n = max(1, int(math.exp(rng.uniform(0.0, math.log(max_values)))))
    fmt = "e4m3" if rng.integers(0, 2) == 0 else "e5m2"
    eb = FP8_EXP_BITS[fmt]
    m = 7 - eb
    law = int(rng.integers(0, 5))
    if law == 0:
        sigma = float(10.0 ** rng.uniform(-4, 2))
        x = rng.standard_normal(n) * sigma
        return fp8_bytes(x, fmt), eb, "%s normal sigma %.3g, %d values" % (fmt, sigma, n)
    if law == 1:
        return rng.integers(0, 256, n, dtype=np.uint8), eb, "%s uniform bytes, %d values" % (fmt, n)
    nf = 1 << eb
    if law == 2:
        k = int(rng.choice([1, 2, 3, 5, 9, nf]))
        fields = rng.choice(nf, size=k, replace=False)
        w = rng.dirichlet(np.full(k, 0.3))
        exps = fields[rng.choice(k, size=n, p=w)].astype(np.uint8)
        what = "%s %d live exponent fields (Dirichlet 0.3), %d values" % (fmt, k, n)
    elif law == 3:
        a = float(rng.uniform(1.05, 3.0))
        ranks = np.minimum(rng.zipf(a, size=n), nf) - 1
        exps = rng.permutation(nf)[ranks].astype(np.uint8)
        what = "%s Zipf a=%.2f exponent ranks, %d values" % (fmt, a, n)
    else:
        r = float(rng.uniform(0.3, 0.9))
        w = r ** np.arange(nf)
        exps = rng.permutation(nf)[rng.choice(nf, size=n, p=w / w.sum())].astype(np.uint8)
        what = "%s exponent chain r=%.2f, %d values" % (fmt, r, n)
    sign = rng.integers(0, 2, n, dtype=np.uint8) << 7
    mant = rng.integers(0, 1 << m, n, dtype=np.uint8)
    return (sign | (exps << m) | mant).astype(np.uint8), eb, what

