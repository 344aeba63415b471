/*
 * e8huf_oracle.c -- plain, slow CPU oracle for the FP8 exponent Huffman codec
 * (the ECF8-style variant).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library. The product path
 * must never call it, and it shares no source, header, table or constant with
 * the product library: it restates the container layout from its written
 * specification.
 *
 * Source: the ECF8 page ("指数集中现象：GenAI模型权重压缩的理论基础",
 * pwwt.cn/news/2030120):
 *   - section 1.2: the base format is FP8, E4M3 or E5M2 (byte aligned);
 *   - section 2.1 (encoding stage): per layer, count the frequencies of the
 *     exponent values; smooth the frequency distribution so that no code gets
 *     extremely long; build a Huffman tree; the longest code is 16 bits; the
 *     codes come out ordered by (code length, symbol); a two-level table: the
 *     first level handles an 8-bit prefix and either decodes directly or
 *     points to a second-level table, which handles the next 8 bits; metadata
 *     per thread block: its bit offset and its start in the symbol stream;
 *   - section 1.1: the sign and mantissa bits carry the rest of the value
 *     (only the exponent is concentrated), so they are kept as they are.
 *
 * Readings where the page is silent (each also listed in the design notes):
 *   - symbols are the exponent fields: 16 of them for E4M3 (bits 6..3), 32 for
 *     E5M2 (bits 6..2); sign and mantissa form a nibble (sign << m | mantissa,
 *     m = mantissa bits) stored raw, two per byte, value 2i in the low nibble;
 *   - Huffman ties: merge the two lightest nodes, equal weights to the lower
 *     node id (leaves 0.. by symbol, merged nodes the following ids);
 *   - smoothing: while the deepest code is longer than 16 bits, every live
 *     count c becomes c / 2 + 1 (integer division) and the tree is rebuilt; a
 *     lone symbol gets length 1;
 *   - codes: canonical, shortest length first (the page's order by length,
 *     then symbol): first[1] = 0, first[l] = (first[l-1] + count[l-1]) << 1,
 *     symbols of one length take consecutive codes in ascending order; codes
 *     are read most-significant bit first;
 *   - a thread block's unit is 16,384 values (64 lane chunks of 256): its
 *     record holds its start bit and the code bits of each lane chunk; its
 *     start in the symbol stream is its index times 16,384.
 *
 * Container ("E8HF"), little-endian:
 *   header, 128 bytes: magic "E8HF", u16 version 1, u8 exp_bits (4 or 5),
 *     u8 maxlen 16, u64 n_values, u32 block_values 16384, u32 lane_values
 *     256, u32 n_blocks = ceil(n / 16384), u32 0, u64 n_bits, u64 bits_off,
 *     u64 nib_off, u64 container_bytes, u8 codelen[32] (at 64), zero to 128;
 *   at 128: n_blocks records of 136 bytes {u64 start_bit, u16 lane_bits[64]}
 *     (lane chunks past the last value count 0); zero pad to 256;
 *   bitstream at bits_off: n_bits code bits, MSB first, zero padded to a
 *     multiple of 16 bytes, then to 256;
 *   nibble plane at nib_off: ceil(n / 2) bytes, zero padded to 256; that
 *     offset plus the padded plane is container_bytes. *
 * Widening (section 2.2: the page's decoder hands its output over as 16-bit
 * floating-point values rather than FP8 bytes). Reading: output value i is the
 * FP8 value of decoded byte i (section 1.2's format: sign, exponent field with
 * bias 2^(e-1) - 1, mantissa with an implicit one unless the exponent field is
 * zero; E4M3 has no infinities and S.1111.111 is NaN, E5M2 keeps IEEE's
 * all-ones exponent for infinities and NaNs) times a per-tensor scale, the
 * product taken in single precision, then rounded to the nearest value of the
 * 16-bit output format (bfloat16: 8 exponent and 7 mantissa bits; IEEE half:
 * 5 and 10), ties to an even mantissa, overflow to infinity; a NaN stays a NaN.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define E8_MAXLEN 16
#define E8_BLOCK 16384u
#define E8_LANE 256u
#define E8_LANES (E8_BLOCK / E8_LANE)
#define E8_HDR 128u
#define E8_REC (8u + 2u * E8_LANES)

enum {
    E8_OK = 0,
    E8_E_ARG = -1,
    E8_E_EMPTY = -2,
    E8_E_OVERSUB = -3,
    E8_E_BADLEN = -4,
    E8_E_FORMAT = -6,
    E8_E_CORRUPT = -7,
    E8_E_INDEX = -9,
};

/* Huffman leaf depths over 256 counts (k3huf_oracle.c; the same tie rule). */
int oh_huffman_depths(const uint64_t count[256], uint8_t depth[256]);

static uint64_t rd_le(const uint8_t *p, int n) {
    uint64_t v = 0;
    for (int i = n - 1; i >= 0; i--) v = (v << 8) | p[i];
    return v;
}
static void wr_le(uint8_t *p, uint64_t v, int n) {
    for (int i = 0; i < n; i++) { p[i] = (uint8_t)(v & 0xff); v >>= 8; }
}
static uint64_t up16(uint64_t x) { return (x + 15) & ~(uint64_t)15; }
static uint64_t up256(uint64_t x) { return (x + 255) & ~(uint64_t)255; }

static int n_symbols(int exp_bits) { return 1 << exp_bits; }

/* Kraft sum in units of 2^-16: sum over coded symbols of 2^(16 - len);
 * -1 if a length exceeds 16. */
int64_t e8_kraft(const uint8_t len[32]) {
    int64_t k = 0;
    for (int s = 0; s < 32; s++) {
        if (!len[s]) continue;
        if (len[s] > E8_MAXLEN) return -1;
        k += (int64_t)1 << (E8_MAXLEN - len[s]);
    }
    return k;
}

/* Code lengths (ECF8 page, section 2.1): Huffman depths of the exponent
 * histogram; while the deepest is above 16 bits, smooth the counts
 * (c -> c / 2 + 1 for every live count) and rebuild. A lone symbol gets
 * length 1. Returns the number of smoothing rounds, or E8_E_EMPTY. */
int e8_code_lengths(const uint64_t count[32], uint8_t len[32]) {
    uint64_t c[256] = {0};
    uint8_t d[256];
    int live = 0;
    for (int s = 0; s < 32; s++) {
        c[s] = count[s];
        live += count[s] != 0;
        len[s] = 0;
    }
    if (live == 0) return E8_E_EMPTY;
    if (live == 1) {
        for (int s = 0; s < 32; s++) len[s] = count[s] ? 1 : 0;
        return 0;
    }
    int rounds = 0;
    for (;;) {
        int maxd = oh_huffman_depths(c, d);
        if (maxd <= E8_MAXLEN) break;
        for (int s = 0; s < 32; s++)
            if (c[s]) c[s] = c[s] / 2 + 1;
        rounds++;
    }
    for (int s = 0; s < 32; s++) len[s] = d[s];
    return rounds;
}

/* Canonical codes, shortest length first: first[1] = 0, first[l] =
 * (first[l-1] + count[l-1]) << 1; ascending symbols within a length take
 * consecutive codes. */
void e8_canonical(const uint8_t len[32], uint32_t code[32]) {
    uint32_t cnt[E8_MAXLEN + 1] = {0}, next[E8_MAXLEN + 1] = {0};
    for (int s = 0; s < 32; s++)
        if (len[s] && len[s] <= E8_MAXLEN) cnt[len[s]]++;
    uint32_t c = 0;   /* cnt[0] = 0: lengths start at 1, code 0 */
    for (int l = 1; l <= E8_MAXLEN; l++) {
        c = (c + cnt[l - 1]) << 1;
        next[l] = c;
    }
    for (int s = 0; s < 32; s++) {
        code[s] = 0;
        if (len[s] && len[s] <= E8_MAXLEN) code[s] = next[len[s]]++;
    }
}

/* Table validity: not empty, no length above 16, Kraft sum at most 2^16; and
 * every canonical code fits its length and no code prefixes another (checked
 * pair by pair). */
int e8_check_table(const uint8_t len[32]) {
    int any = 0;
    for (int s = 0; s < 32; s++) {
        if (len[s] > E8_MAXLEN) return E8_E_BADLEN;
        any |= len[s] != 0;
    }
    if (!any) return E8_E_EMPTY;
    if (e8_kraft(len) > ((int64_t)1 << E8_MAXLEN)) return E8_E_OVERSUB;
    uint32_t code[32];
    e8_canonical(len, code);
    for (int a = 0; a < 32; a++) {
        if (!len[a]) continue;
        if (code[a] >= (1u << len[a])) return E8_E_OVERSUB;
        for (int b = 0; b < 32; b++) {
            if (b == a || !len[b] || len[b] < len[a]) continue;
            if ((code[b] >> (len[b] - len[a])) == code[a]) return E8_E_OVERSUB;
        }
    }
    return E8_OK;
}

/* Bit-by-bit decoder state: codes of length l are the cnt[l] values from
 * first[l]; sym[l][k] is the k-th smallest symbol of length l. */
typedef struct {
    uint32_t cnt[E8_MAXLEN + 1], first[E8_MAXLEN + 1];
    uint8_t sym[E8_MAXLEN + 1][32];
} e8_dec_t;

static void dec_init(const uint8_t len[32], e8_dec_t *d) {
    memset(d, 0, sizeof *d);
    for (int s = 0; s < 32; s++)
        if (len[s]) d->sym[len[s]][d->cnt[len[s]]++] = (uint8_t)s;
    uint32_t code[32];
    e8_canonical(len, code);
    for (int l = 1; l <= E8_MAXLEN; l++)
        if (d->cnt[l]) d->first[l] = code[d->sym[l][0]];
}

static int dec_one(const e8_dec_t *d, const uint8_t *bits, uint64_t nbits, uint64_t *pos) {
    uint32_t code = 0;
    for (int l = 1; l <= E8_MAXLEN; l++) {
        if (*pos >= nbits) return -1;
        uint32_t b = (bits[*pos >> 3] >> (7 - (*pos & 7))) & 1;
        (*pos)++;
        code = (code << 1) | b;
        if (d->cnt[l] && code >= d->first[l] && code - d->first[l] < d->cnt[l])
            return d->sym[l][code - d->first[l]];
    }
    return -1;
}

/* Bit-by-bit decode of the 16-bit string bits16 (first bit = bit 15): the
 * symbol and length of the code that prefixes it, or -1. */
int e8_decode_prefix(const uint8_t len[32], uint32_t bits16, int *sym, int *clen) {
    e8_dec_t d;
    dec_init(len, &d);
    uint8_t b[2] = {(uint8_t)(bits16 >> 8), (uint8_t)bits16};
    uint64_t pos = 0;
    int s = dec_one(&d, b, 16, &pos);
    if (s < 0) return -1;
    *sym = s;
    *clen = (int)pos;
    return 0;
}

/* --------------------------------------------------------------------------
 * container */

static uint64_t n_blocks_of(uint64_t n) { return (n + E8_BLOCK - 1) / E8_BLOCK; }

int64_t e8_encode_bound(uint64_t n) {
    if (n == 0) return E8_E_ARG;
    uint64_t nb = n_blocks_of(n);
    return (int64_t)(up256(E8_HDR + E8_REC * nb) + up256(up16((n * E8_MAXLEN + 7) / 8)) + up256((n + 1) / 2));
}

static void put_bits(uint8_t *buf, uint64_t *pos, uint32_t code, int l) {
    for (int b = l - 1; b >= 0; b--) {
        if ((code >> b) & 1) buf[*pos >> 3] |= (uint8_t)(0x80u >> (*pos & 7));
        (*pos)++;
    }
}

/* Encoder: exponent histogram of the whole tensor, code lengths, canonical
 * codes; the exponent codes MSB first with the per-block records; the
 * sign/mantissa nibbles raw. Returns the container size or an error. */
int64_t e8_encode(const uint8_t *x, uint64_t n, int exp_bits, uint8_t *out, uint64_t cap) {
    if (!x || !out || n == 0 || (exp_bits != 4 && exp_bits != 5)) return E8_E_ARG;
    if ((uint64_t)e8_encode_bound(n) > cap) return E8_E_ARG;
    const int m = 7 - exp_bits;
    const uint32_t emask = (uint32_t)n_symbols(exp_bits) - 1;
    uint64_t count[32] = {0};
    for (uint64_t i = 0; i < n; i++) count[(x[i] >> m) & emask]++;
    uint8_t len[32];
    if (e8_code_lengths(count, len) < 0) return E8_E_EMPTY;
    if (e8_check_table(len) != E8_OK) return E8_E_CORRUPT;
    uint32_t code[32];
    e8_canonical(len, code);

    memset(out, 0, cap);
    uint64_t nb = n_blocks_of(n);
    uint64_t bits_off = up256(E8_HDR + E8_REC * nb);
    uint8_t *bits = out + bits_off;
    uint64_t pos = 0, lane_start = 0;
    for (uint64_t i = 0; i < n; i++) {
        if (i % E8_LANE == 0) {
            if (i > 0) {
                uint64_t pl = (i - 1) / E8_LANE;
                wr_le(out + E8_HDR + E8_REC * (pl / E8_LANES) + 8 + 2 * (pl % E8_LANES), pos - lane_start, 2);
            }
            lane_start = pos;
        }
        if (i % E8_BLOCK == 0) wr_le(out + E8_HDR + E8_REC * (i / E8_BLOCK), pos, 8);
        uint32_t e = (x[i] >> m) & emask;
        put_bits(bits, &pos, code[e], len[e]);
    }
    {
        uint64_t pl = (n - 1) / E8_LANE;
        wr_le(out + E8_HDR + E8_REC * (pl / E8_LANES) + 8 + 2 * (pl % E8_LANES), pos - lane_start, 2);
    }
    uint64_t nib_off = up256(bits_off + up16((pos + 7) / 8));
    for (uint64_t i = 0; i < n; i++) {
        uint32_t v = ((uint32_t)(x[i] >> 7) << m) | (x[i] & ((1u << m) - 1));
        out[nib_off + i / 2] |= (uint8_t)(v << (4 * (i & 1)));
    }
    uint64_t total = up256(nib_off + (n + 1) / 2);
    memcpy(out, "E8HF", 4);
    wr_le(out + 4, 1, 2);
    out[6] = (uint8_t)exp_bits;
    out[7] = E8_MAXLEN;
    wr_le(out + 8, n, 8);
    wr_le(out + 16, E8_BLOCK, 4);
    wr_le(out + 20, E8_LANE, 4);
    wr_le(out + 24, nb, 4);
    wr_le(out + 28, 0, 4);
    wr_le(out + 32, pos, 8);
    wr_le(out + 40, bits_off, 8);
    wr_le(out + 48, nib_off, 8);
    wr_le(out + 56, total, 8);
    memcpy(out + 64, len, 32);
    return (int64_t)total;
}

typedef struct {
    uint64_t n, n_bits, bits_off, nib_off, nb;
    int exp_bits;
    const uint8_t *len;
} e8_hdr_t;

static int parse(const uint8_t *blob, uint64_t size, e8_hdr_t *H) {
    if (!blob || size < E8_HDR || memcmp(blob, "E8HF", 4) != 0) return E8_E_FORMAT;
    if (rd_le(blob + 4, 2) != 1 || (blob[6] != 4 && blob[6] != 5) || blob[7] != E8_MAXLEN) return E8_E_FORMAT;
    if (rd_le(blob + 16, 4) != E8_BLOCK || rd_le(blob + 20, 4) != E8_LANE) return E8_E_FORMAT;
    H->exp_bits = blob[6];
    H->n = rd_le(blob + 8, 8);
    H->nb = rd_le(blob + 24, 4);
    H->n_bits = rd_le(blob + 32, 8);
    H->bits_off = rd_le(blob + 40, 8);
    H->nib_off = rd_le(blob + 48, 8);
    H->len = blob + 64;
    if (H->n == 0 || H->nb != n_blocks_of(H->n)) return E8_E_FORMAT;
    if (rd_le(blob + 56, 8) > size) return E8_E_FORMAT;
    if (H->bits_off < E8_HDR + E8_REC * H->nb || H->bits_off + (H->n_bits + 7) / 8 > H->nib_off)
        return E8_E_FORMAT;
    if (H->nib_off + (H->n + 1) / 2 > size) return E8_E_FORMAT;
    for (int s = n_symbols(H->exp_bits); s < 32; s++)
        if (H->len[s]) return E8_E_FORMAT;
    return E8_OK;
}

/* Bit-by-bit decode of the whole tensor, ignoring the block records. */
int e8_decode(const uint8_t *blob, uint64_t size, uint8_t *out, uint64_t n) {
    e8_hdr_t H;
    int rc = parse(blob, size, &H);
    if (rc) return rc;
    if (n != H.n) return E8_E_ARG;
    rc = e8_check_table(H.len);
    if (rc) return rc;
    e8_dec_t d;
    dec_init(H.len, &d);
    const int m = 7 - H.exp_bits;
    const uint8_t *bits = blob + H.bits_off, *nib = blob + H.nib_off;
    uint64_t pos = 0;
    for (uint64_t i = 0; i < n; i++) {
        int e = dec_one(&d, bits, H.n_bits, &pos);
        if (e < 0) return E8_E_CORRUPT;
        uint32_t v = (nib[i / 2] >> (4 * (i & 1))) & 15;
        out[i] = (uint8_t)(((v >> m) << 7) | ((uint32_t)e << m) | (v & ((1u << m) - 1)));
    }
    return pos == H.n_bits ? E8_OK : E8_E_CORRUPT;
}

/* Index checker: replays the decode and compares every block's start bit and
 * every lane chunk's code-bit count with the records. */
int e8_check_index(const uint8_t *blob, uint64_t size) {
    e8_hdr_t H;
    int rc = parse(blob, size, &H);
    if (rc) return rc;
    rc = e8_check_table(H.len);
    if (rc) return rc;
    e8_dec_t d;
    dec_init(H.len, &d);
    const uint8_t *bits = blob + H.bits_off;
    uint64_t pos = 0;
    for (uint64_t b = 0; b < H.nb; b++) {
        const uint8_t *rec = blob + E8_HDR + E8_REC * b;
        if (rd_le(rec, 8) != pos) return E8_E_INDEX;
        for (uint32_t t = 0; t < E8_LANES; t++) {
            uint64_t p0 = pos;
            for (uint32_t k = 0; k < E8_LANE; k++) {
                uint64_t i = b * E8_BLOCK + (uint64_t)t * E8_LANE + k;
                if (i >= H.n) break;
                if (dec_one(&d, bits, H.n_bits, &pos) < 0) return E8_E_CORRUPT;
            }
            if (rd_le(rec + 8 + 2 * t, 2) != pos - p0) return E8_E_INDEX;
        }
    }
    return pos == H.n_bits ? E8_OK : E8_E_INDEX;
}

/* Value count recorded in a container header, or a negative error. */
int64_t e8_n_values(const uint8_t *blob, uint64_t size) {
    e8_hdr_t H;
    int rc = parse(blob, size, &H);
    return rc ? rc : (int64_t)H.n;
}

/* The value an FP8 byte stands for (section 1.2's format), exactly, as a
 * double. */
static double fp8_value(uint8_t b, int exp_bits) {
    const int mb = 7 - exp_bits;                       /* mantissa bits */
    const int bias = (1 << (exp_bits - 1)) - 1;        /* 7 (E4M3), 15 (E5M2) */
    const int e = (b >> mb) & ((1 << exp_bits) - 1);
    const int f = b & ((1 << mb) - 1);
    double v;
    if (exp_bits == 4 && e == 15 && f == 7)
        v = NAN;                                       /* E4M3: the one NaN pattern */
    else if (exp_bits == 5 && e == 31)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, 1 - bias - mb);           /* subnormal: f * 2^(1 - bias - mb) */
    else
        v = ldexp(1.0 + ldexp((double)f, -mb), e - bias);
    return (b & 0x80) ? -v : v;
}

/* x rounded to the nearest value of a 16-bit binary format with eb exponent
 * and mb mantissa bits (bias 2^(eb-1) - 1), ties to the even significand,
 * magnitudes past the largest finite value's rounding range to infinity. */
static uint16_t round16(float x, int eb, int mb) {
    const int bias = (1 << (eb - 1)) - 1, eall = (1 << eb) - 1;
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | (eall << mb) | (1u << (mb - 1)));
    if (isinf(x)) return (uint16_t)(sign | (eall << mb));
    const double a = fabs((double)x);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);                                     /* a = f * 2^e2, f in [0.5, 1) */
    int ue = e2 - 1;                                   /* a in [2^ue, 2^(ue+1)) */
    if (ue < 1 - bias) ue = 1 - bias;                  /* below the normal range: subnormal quantum */
    double q = rint(ldexp(a, mb - ue));                /* significand in quanta of 2^(ue - mb), ties to even */
    if (q < ldexp(1.0, mb)) return (uint16_t)(sign | (uint32_t)q);   /* subnormal or zero */
    if (q == ldexp(1.0, mb + 1)) {                     /* rounded up to the next power of two */
        q = ldexp(1.0, mb);
        ue += 1;
    }
    const int field = ue + bias;
    if (field >= eall) return (uint16_t)(sign | (eall << mb));
    return (uint16_t)(sign | ((uint32_t)field << mb) | ((uint32_t)q - (1u << mb)));
}

/* out[i] = round16(float(value(x[i])) * scale) for the output kind (1:
 * bfloat16, 2: IEEE half). Returns 0, or E8_E_ARG. */
int e8_widen(const uint8_t *x, uint64_t n, int exp_bits, float scale, int out_kind, uint16_t *out) {
    if ((exp_bits != 4 && exp_bits != 5) || (out_kind != 1 && out_kind != 2) || (n && (!x || !out)))
        return E8_E_ARG;
    const int eb = out_kind == 1 ? 8 : 5, mb = out_kind == 1 ? 7 : 10;
    for (uint64_t i = 0; i < n; i++) {
        const float v = (float)fp8_value(x[i], exp_bits);   /* exact: every FP8 value is a float */
        const float p = v * scale;                           /* single-precision product */
        out[i] = round16(p, eb, mb);
    }
    return E8_OK;
}
