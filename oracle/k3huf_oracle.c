/*
 * k3huf_oracle.c -- plain, slow CPU oracle for the bf16 high-byte Huffman codec.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library. The product's
 * decode path must never call it, and this file shares no source, header,
 * table or constant with the product library: it restates the container
 * layout from its written specification.
 *
 * Sources ("K3 page" = the page "Kimi K3 纯 CPU 推理中的无损 Trunk 压缩：一次被
 * 解码速度判死刑的 Huffman 压缩实验", yfxerp.com/news/153994):
 *   - K3 page, "core idea" section: only the high (sign+exponent) byte of each
 *     bf16 value is entropy coded; the mantissa byte is stored raw; lossless.
 *   - K3 page, "what was implemented" section: a layer header holding
 *     codelen[256], then per stripe [stripe header][odd-plane Huffman
 *     bitstream][even plane raw].
 *   - K3 page, "key design points" section: 64 MiB stripes decoded
 *     independently; odd offsets (little-endian high byte) coded, even offsets
 *     copied; code length limited to 12 bits.
 *   - K3 page, "canonical code assignment and Kraft check" section: the Kraft
 *     sum must fill the 12-bit code space exactly or under-fill it, an
 *     over-full or empty table is corrupt; canonical codes are assigned
 *     longest length first, in symbol order within a length; code lengths come
 *     from the depths of a standard Huffman tree, with a repair that lengthens
 *     the least frequent code while the Kraft sum is over-full.
 *   - K3 page, "decode loop" section: the head of the stream sits at the top
 *     of the bit window, i.e. codes are read most-significant bit first.
 *
 * Readings where the page is silent or garbled (each also listed in the design
 * notes): the garbled recurrence is read as first[l] = code; code = (code +
 * count[l]) >> 1; a single live symbol gets length 1; the repair loop may leave
 * the table under-full, and an under-full table with the floor recurrence can
 * give one code as a prefix of another, so this encoder adds a "repay" pass
 * that shortens codes until the table is exactly full, and the decoder rejects
 * any table whose codes are not prefix-free. The per-subblock index (start bit
 * per 65,536-byte subblock, code bits per 256-symbol lane chunk) is an addition
 * for parallel decoding, counted in the container size.
 *
 * The length limit and the repay pass are a procedure, fixed up to their
 * tie rules: the tests pin their exact output on hand-derived cases (clamp
 * only, lengthen then repay, a tie in each loop, a repay that shortens one
 * code twice), besides invariants (no length above 12, an exactly full table
 * for two or more symbols, a cost at least the optimal limited cost). Every
 * decode reads the lengths from the container.
 *
 * The decoder here ignores the index entirely: it reads the stripe bitstream
 * one bit at a time and matches the growing code against the canonical ranges.
 *
 * Container layout (all little-endian), restated from the format description:
 *   layer header, 304 bytes: magic "K3HF", u16 version 1, u16 maxlen 12,
 *     u32 stripe_bytes 2^26, u32 subblock_bytes = 256 * lane_syms,
 *     u32 lane_syms (256, or 64 for the short-chunk layout of small layers),
 *     u32 n_stripes, u64 raw_bytes, u32 n_subblocks, u32 0, u64 container_bytes,
 *     u8 codelen[256]; then u64 stripe_off[n_stripes]; zero pad to 256.
 *   stripe record at stripe_off[s] (256-aligned): u32 raw_bytes, u32 n_syms,
 *     u32 n_bits, u32 bit_bytes, u32 first_subblock, u32 n_subblocks,
 *     u32 bits_off, u32 even_off; then n_subblocks records of 264 bytes
 *     {u32 start_bit, u32 n_syms, u16 lane_bits[128]} (a subblock holds 128
 *     lane chunks of lane_syms symbols); zero pad to 256; the
 *     bitstream (bit_bytes = ceil(n_bits/8) rounded up to 16, zero padded) at
 *     bits_off; zero pad to 256; the even plane (n_syms bytes, zero padded to
 *     256) at even_off. bits_off and even_off count from the stripe record's
 *     first byte and are multiples of 256. (Decoders need only 16-byte
 *     alignment; the 256-byte padding keeps the planes on cache-line
 *     boundaries.)
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OH_MAXLEN 12
#define OH_STRIPE (1u << 26)
#define OH_LANES 128u              /* lane chunks per subblock */
#define OH_HDR 304u
#define OH_STRIPE_HDR 32u
#define OH_REC (8u + 2u * OH_LANES)

enum {
    OH_OK = 0,
    OH_E_ARG = -1,
    OH_E_EMPTY = -2,
    OH_E_OVERSUB = -3,
    OH_E_BADLEN = -4,
    OH_E_OVERLAP = -5,
    OH_E_FORMAT = -6,
    OH_E_CORRUPT = -7,
    OH_E_INDEX = -9,
};

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

/* ---------------------------------------------------------------------------
 * Code lengths (K3 page, "canonical code assignment and Kraft check": lengths
 * are the leaf depths of a standard Huffman tree).
 * Plain O(n^2) construction: repeatedly merge the two lightest live nodes.
 * Ties are broken by node id (leaves get ids 0.. in ascending symbol order,
 * internal nodes get the next ids as they are made), which makes the result
 * reproducible. A lone symbol has depth 0 here. Returns the maximum depth.
 * ------------------------------------------------------------------------- */
int oh_huffman_depths(const uint64_t count[256], uint8_t depth[256]) {
    uint64_t w[511];
    int parent[511], alive[511], leaf_of[256];
    int n = 0;
    for (int s = 0; s < 256; s++) {
        depth[s] = 0;
        leaf_of[s] = -1;
        if (count[s]) { leaf_of[s] = n; w[n] = count[s]; parent[n] = -1; alive[n] = 1; n++; }
    }
    int live = n, total = n;
    while (live > 1) {
        int a = -1, b = -1;
        for (int i = 0; i < total; i++) {
            if (!alive[i]) continue;
            if (a < 0 || w[i] < w[a]) { b = a; a = i; }
            else if (b < 0 || w[i] < w[b]) { b = i; }
        }
        int p = total++;
        w[p] = w[a] + w[b];
        parent[p] = -1;
        alive[p] = 1;
        parent[a] = p; parent[b] = p;
        alive[a] = 0; alive[b] = 0;
        live--;
    }
    int maxd = 0;
    for (int s = 0; s < 256; s++) {
        if (leaf_of[s] < 0) continue;
        int d = 0;
        for (int x = leaf_of[s]; parent[x] >= 0; x = parent[x]) d++;
        if (d > 255) d = 255;
        depth[s] = (uint8_t)d;
        if (d > maxd) maxd = d;
    }
    return maxd;
}

/* Kraft sum in units of 2^-12: sum over coded symbols of 2^(12 - len).
 * Returns -1 if any length exceeds 12 (K3 page, "key design points": the
 * code length is capped at 12 bits). */
int oh_kraft(const uint8_t len[256]) {
    int k = 0;
    for (int s = 0; s < 256; s++) {
        if (!len[s]) continue;
        if (len[s] > OH_MAXLEN) return -1;
        k += 1 << (OH_MAXLEN - len[s]);
    }
    return k;
}

/* Encoder code lengths: Huffman depths, then the length limit.
 * K3 page, "canonical code assignment and Kraft check": the limit repair
 * repeatedly lengthens the least frequent code while the Kraft sum is over-full
 * ("key design points": deeper trees are flattened to 12 bits).
 * Steps: (1) clamp depths above 12 to 12; (2) while over-full, lengthen the
 * lowest-count symbol among those shorter than 12 (ties: larger symbol);
 * (3) repay, not on the page: while under-full and at least two symbols are
 * coded, shorten by one the highest-count symbol whose shortening still fits
 * (ties: smaller symbol), which ends exactly full; (4) a lone symbol gets
 * length 1. Returns the final Kraft sum, or OH_E_EMPTY when nothing is coded. */
int oh_code_lengths(const uint64_t count[256], uint8_t len[256]) {
    int live = 0;
    for (int s = 0; s < 256; s++) live += count[s] != 0;
    oh_huffman_depths(count, len);
    if (live == 0) return OH_E_EMPTY;
    if (live == 1) {
        for (int s = 0; s < 256; s++) len[s] = count[s] ? 1 : 0;
        return oh_kraft(len);
    }
    for (int s = 0; s < 256; s++)
        if (count[s] && len[s] > OH_MAXLEN) len[s] = OH_MAXLEN;
    int k = oh_kraft(len);
    while (k > (1 << OH_MAXLEN)) {
        int pick = -1;
        for (int s = 0; s < 256; s++) {
            if (!count[s] || len[s] >= OH_MAXLEN) continue;
            if (pick < 0 || count[s] <= count[pick]) pick = s; /* '<=': later (larger) symbol wins ties */
        }
        len[pick]++;
        k = oh_kraft(len);
    }
    while (k < (1 << OH_MAXLEN)) {
        int pick = -1;
        for (int s = 0; s < 256; s++) {
            if (!count[s] || len[s] <= 1) continue;
            if ((1 << (OH_MAXLEN - len[s])) > (1 << OH_MAXLEN) - k) continue;
            if (pick < 0 || count[s] > count[pick]) pick = s; /* '>': earlier (smaller) symbol wins ties */
        }
        if (pick < 0) break; /* cannot happen for >= 2 symbols; kept for safety */
        len[pick]--;
        k = oh_kraft(len);
    }
    return k;
}

/* Canonical codes, longest length first (K3 page, "canonical code assignment
 * and Kraft check"): code = 0; for l = 12 down to 1 { first[l] = code;
 * code = (code + count[l]) >> 1 }; then symbols in ascending value take the
 * consecutive codes first[l], first[l] + 1, ... of their length. */
void oh_canonical(const uint8_t len[256], uint32_t code[256]) {
    uint32_t cnt[OH_MAXLEN + 1] = {0}, first[OH_MAXLEN + 1] = {0}, next[OH_MAXLEN + 1];
    for (int s = 0; s < 256; s++)
        if (len[s] && len[s] <= OH_MAXLEN) cnt[len[s]]++;
    uint32_t c = 0;
    for (int l = OH_MAXLEN; l >= 1; l--) {
        first[l] = c;
        c = (c + cnt[l]) >> 1;
    }
    memcpy(next, first, sizeof next);
    for (int s = 0; s < 256; s++) {
        code[s] = 0;
        if (len[s] && len[s] <= OH_MAXLEN) code[s] = next[len[s]]++;
    }
}

/* Table validity (K3 page, "canonical code assignment and Kraft check": reject
 * over-full or empty tables; plus the reading that any table whose canonical
 * codes are not prefix-free is rejected, checked pair by pair). */
int oh_check_table(const uint8_t len[256]) {
    int any = 0;
    for (int s = 0; s < 256; s++) {
        if (len[s] > OH_MAXLEN) return OH_E_BADLEN;
        any |= len[s] != 0;
    }
    if (!any) return OH_E_EMPTY;
    if (oh_kraft(len) > (1 << OH_MAXLEN)) return OH_E_OVERSUB;
    uint32_t code[256];
    oh_canonical(len, code);
    for (int a = 0; a < 256; a++) {
        if (!len[a]) continue;
        if (code[a] >= (1u << len[a])) return OH_E_OVERLAP;
        for (int b = 0; b < 256; b++) {
            if (b == a || !len[b] || len[b] < len[a]) continue;
            if ((code[b] >> (len[b] - len[a])) == code[a]) return OH_E_OVERLAP;
        }
    }
    return OH_OK;
}

/* The decoder's canonical ranges: codes of length l are first[l] ..
 * first[l] + cnt[l] - 1, and sym[l][k] is the k-th smallest symbol of length l. */
typedef struct {
    uint32_t cnt[OH_MAXLEN + 1], first[OH_MAXLEN + 1];
    uint8_t sym[OH_MAXLEN + 1][256];
} oh_dec_t;

static void dec_init(const uint8_t len[256], oh_dec_t *d) {
    memset(d, 0, sizeof *d);
    for (int s = 0; s < 256; s++)
        if (len[s]) d->sym[len[s]][d->cnt[len[s]]++] = (uint8_t)s;
    uint32_t c = 0;
    for (int l = OH_MAXLEN; l >= 1; l--) {
        d->first[l] = c;
        c = (c + d->cnt[l]) >> 1;
    }
}

/* Bit-by-bit decode of one symbol whose code starts at bit *pos of an MSB-first
 * bitstream of nbits bits. Returns the symbol, or -1 on an invalid code or
 * when the stream ends first. */
static int dec_one(const oh_dec_t *d, const uint8_t *bits, uint64_t nbits, uint64_t *pos) {
    uint32_t code = 0;
    for (int l = 1; l <= OH_MAXLEN; l++) {
        if (*pos >= nbits) return -1;
        uint32_t bit = (bits[*pos >> 3] >> (7 - (*pos & 7))) & 1;
        (*pos)++;
        code = (code << 1) | bit;
        if (d->cnt[l] && code >= d->first[l] && code - d->first[l] < d->cnt[l])
            return d->sym[l][code - d->first[l]];
    }
    return -1;
}

/* Decode the 12-bit string `bits12` (first bit = bit 11) bit by bit under the
 * table `len`: writes the symbol and its code length, or returns -1 when no
 * code is a prefix of the string. Used to check a 4096-entry lookup table
 * slot by slot. */
int oh_decode_prefix(const uint8_t len[256], uint32_t bits12, int *sym, int *clen) {
    oh_dec_t d;
    dec_init(len, &d);
    uint8_t b[2] = {(uint8_t)(bits12 >> 4), (uint8_t)((bits12 & 15) << 4)};
    uint64_t pos = 0;
    int s = dec_one(&d, b, 12, &pos);
    if (s < 0) return -1;
    *sym = s;
    *clen = (int)pos;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* container geometry                                                          */

static uint32_t n_stripes_of(uint64_t raw) { return (uint32_t)((raw + OH_STRIPE - 1) / OH_STRIPE); }

/* the two lane-chunk lengths the format allows, and the subblock they make */
static int lane_syms_ok(uint32_t lane) { return lane == 256u || lane == 64u; }
static uint32_t sb_syms_of(uint32_t lane) { return OH_LANES * lane; }

/* Upper bound on the container size for raw_bytes of layer data (worst case:
 * every code 12 bits long), for lane chunks of `lane` symbols. */
int64_t oh_encode_bound_lanes(uint64_t raw, uint32_t lane) {
    if (!lane_syms_ok(lane)) return OH_E_ARG;
    uint64_t ns = n_stripes_of(raw);
    uint64_t b = up256(OH_HDR + 8 * ns);
    for (uint64_t s = 0; s < ns; s++) {
        uint64_t rb = raw - s * OH_STRIPE;
        if (rb > OH_STRIPE) rb = OH_STRIPE;
        uint64_t n = rb / 2, nsb = (n + sb_syms_of(lane) - 1) / sb_syms_of(lane);
        b += up256(OH_STRIPE_HDR + OH_REC * nsb) + up256(up16((n * OH_MAXLEN + 7) / 8)) + up256(n);
    }
    return (int64_t)b;
}
int64_t oh_encode_bound(uint64_t raw) { return oh_encode_bound_lanes(raw, 256u); }

static void put_bits(uint8_t *buf, uint64_t *pos, uint32_t code, int l) {
    for (int b = l - 1; b >= 0; b--) {
        if ((code >> b) & 1) buf[*pos >> 3] |= (uint8_t)(0x80u >> (*pos & 7));
        (*pos)++;
    }
}

/* Encoder (K3 page, "what was implemented" and "key design points"): one
 * histogram and one codelen[256] over the whole layer's odd bytes; per 64 MiB
 * stripe the odd-byte codes MSB-first, then the even bytes raw; plus the
 * subblock/lane index with lane chunks of `lane` symbols (256, or 64).
 * Returns the container size, or a negative error. */
int64_t oh_encode_layer_lanes(const uint8_t *raw, uint64_t n_raw, uint32_t lane, uint8_t *out, uint64_t cap) {
    if (!raw || !out || n_raw == 0 || (n_raw & 1) || !lane_syms_ok(lane)) return OH_E_ARG;
    if ((uint64_t)oh_encode_bound_lanes(n_raw, lane) > cap) return OH_E_ARG;
    const uint32_t sb_syms = sb_syms_of(lane);
    uint64_t count[256] = {0};
    for (uint64_t i = 1; i < n_raw; i += 2) count[raw[i]]++;
    uint8_t len[256];
    if (oh_code_lengths(count, len) < 0) return OH_E_EMPTY;
    if (oh_check_table(len) != OH_OK) return OH_E_CORRUPT;
    uint32_t code[256];
    oh_canonical(len, code);

    uint32_t ns = n_stripes_of(n_raw);
    memset(out, 0, cap);
    uint64_t o = up256(OH_HDR + 8ull * ns);
    uint32_t sb_total = 0;
    for (uint32_t s = 0; s < ns; s++) {
        uint64_t base = (uint64_t)s * OH_STRIPE;
        uint64_t rb = n_raw - base;
        if (rb > OH_STRIPE) rb = OH_STRIPE;
        uint32_t n = (uint32_t)(rb / 2);
        uint32_t nsb = (n + sb_syms - 1) / sb_syms;
        uint8_t *st = out + o;
        wr_le(out + OH_HDR + 8ull * s, o, 8);
        uint64_t bits_off = up256(OH_STRIPE_HDR + (uint64_t)OH_REC * nsb);
        uint8_t *bits = st + bits_off;
        uint64_t pos = 0;
        uint64_t lane_start = 0;
        for (uint32_t i = 0; i < n; i++) {
            if (i % lane == 0) {
                if (i > 0) {
                    uint32_t pl = (i - 1) / lane; /* previous lane, global in stripe */
                    uint8_t *rec = st + OH_STRIPE_HDR + (uint64_t)OH_REC * (pl / OH_LANES);
                    wr_le(rec + 8 + 2 * (pl % OH_LANES), pos - lane_start, 2);
                }
                lane_start = pos;
            }
            if (i % sb_syms == 0) {
                uint8_t *rec = st + OH_STRIPE_HDR + (uint64_t)OH_REC * (i / sb_syms);
                uint32_t left = n - i;
                wr_le(rec, pos, 4);
                wr_le(rec + 4, left < sb_syms ? left : sb_syms, 4);
            }
            uint8_t sym = raw[base + 2ull * i + 1];
            put_bits(bits, &pos, code[sym], len[sym]);
        }
        {
            uint32_t pl = (n - 1) / lane;
            uint8_t *rec = st + OH_STRIPE_HDR + (uint64_t)OH_REC * (pl / OH_LANES);
            wr_le(rec + 8 + 2 * (pl % OH_LANES), pos - lane_start, 2);
        }
        uint64_t bit_bytes = up16((pos + 7) / 8);
        uint64_t even_off = up256(bits_off + bit_bytes);
        for (uint32_t i = 0; i < n; i++) st[even_off + i] = raw[base + 2ull * i];
        wr_le(st + 0, rb, 4);
        wr_le(st + 4, n, 4);
        wr_le(st + 8, pos, 4);
        wr_le(st + 12, bit_bytes, 4);
        wr_le(st + 16, sb_total, 4);
        wr_le(st + 20, nsb, 4);
        wr_le(st + 24, bits_off, 4);
        wr_le(st + 28, even_off, 4);
        sb_total += nsb;
        o += up256(even_off + n);
    }
    memcpy(out, "K3HF", 4);
    wr_le(out + 4, 1, 2);
    wr_le(out + 6, OH_MAXLEN, 2);
    wr_le(out + 8, OH_STRIPE, 4);
    wr_le(out + 12, 2ull * sb_syms, 4);
    wr_le(out + 16, lane, 4);
    wr_le(out + 20, ns, 4);
    wr_le(out + 24, n_raw, 8);
    wr_le(out + 32, sb_total, 4);
    wr_le(out + 36, 0, 4);
    wr_le(out + 40, o, 8);
    memcpy(out + 48, len, 256);
    return (int64_t)o;
}
int64_t oh_encode_layer(const uint8_t *raw, uint64_t n_raw, uint8_t *out, uint64_t cap) {
    return oh_encode_layer_lanes(raw, n_raw, 256u, out, cap);
}

/* ------------------------------------------------------------------------- */
/* decoder                                                                     */

typedef struct {
    uint64_t raw;
    uint32_t ns, nsb, lane;
    const uint8_t *len;
} oh_layer_t;

static int parse_layer(const uint8_t *blob, uint64_t nb, oh_layer_t *L) {
    if (!blob || nb < OH_HDR) return OH_E_FORMAT;
    if (memcmp(blob, "K3HF", 4) != 0) return OH_E_FORMAT;
    if (rd_le(blob + 4, 2) != 1 || rd_le(blob + 6, 2) != OH_MAXLEN) return OH_E_FORMAT;
    L->lane = (uint32_t)rd_le(blob + 16, 4);
    if (rd_le(blob + 8, 4) != OH_STRIPE || !lane_syms_ok(L->lane) ||
        rd_le(blob + 12, 4) != 2ull * sb_syms_of(L->lane)) return OH_E_FORMAT;
    L->ns = (uint32_t)rd_le(blob + 20, 4);
    L->raw = rd_le(blob + 24, 8);
    L->nsb = (uint32_t)rd_le(blob + 32, 4);
    if (L->raw == 0 || (L->raw & 1) || L->ns != n_stripes_of(L->raw)) return OH_E_FORMAT;
    if (rd_le(blob + 40, 8) > nb) return OH_E_FORMAT;
    if (OH_HDR + 8ull * L->ns > nb) return OH_E_FORMAT;
    L->len = blob + 48;
    return OH_OK;
}

typedef struct {
    const uint8_t *st, *recs, *bits, *even;
    uint32_t n, n_bits, bit_bytes, nsb, first_sb;
} oh_stripe_t;

static int parse_stripe(const uint8_t *blob, uint64_t nb, const oh_layer_t *L, uint32_t s,
                        oh_stripe_t *S) {
    uint64_t off = rd_le(blob + OH_HDR + 8ull * s, 8);
    if (off % 16 || off + OH_STRIPE_HDR > nb) return OH_E_FORMAT;
    const uint8_t *st = blob + off;
    uint64_t rb = L->raw - (uint64_t)s * OH_STRIPE;
    if (rb > OH_STRIPE) rb = OH_STRIPE;
    if (rd_le(st, 4) != rb || rd_le(st + 4, 4) != rb / 2) return OH_E_FORMAT;
    S->n = (uint32_t)(rb / 2);
    S->n_bits = (uint32_t)rd_le(st + 8, 4);
    S->bit_bytes = (uint32_t)rd_le(st + 12, 4);
    S->first_sb = (uint32_t)rd_le(st + 16, 4);
    S->nsb = (uint32_t)rd_le(st + 20, 4);
    uint64_t bits_off = rd_le(st + 24, 4), even_off = rd_le(st + 28, 4);
    if (S->nsb != (S->n + sb_syms_of(L->lane) - 1) / sb_syms_of(L->lane)) return OH_E_FORMAT;
    if (bits_off < OH_STRIPE_HDR + (uint64_t)OH_REC * S->nsb) return OH_E_FORMAT;
    if ((uint64_t)S->n_bits > 8ull * S->bit_bytes) return OH_E_FORMAT;
    if (even_off < bits_off + S->bit_bytes) return OH_E_FORMAT;
    if (off + even_off + S->n > nb) return OH_E_FORMAT;
    S->st = st;
    S->recs = st + OH_STRIPE_HDR;
    S->bits = st + bits_off;
    S->even = st + even_off;
    return OH_OK;
}

/* Decode stripes [first, first + count) of a layer into out (the raw bytes of
 * those stripes, contiguous). Bit-by-bit, ignoring the subblock index; the
 * stripe's stored code-bit count must match what the decode consumed. */
int oh_decode_stripes(const uint8_t *blob, uint64_t nb, uint32_t first, uint32_t count,
                      uint8_t *out, uint64_t out_cap) {
    oh_layer_t L;
    int rc = parse_layer(blob, nb, &L);
    if (rc) return rc;
    if (first > L.ns || count > L.ns - first) return OH_E_ARG;
    rc = oh_check_table(L.len);
    if (rc) return rc;
    oh_dec_t d;
    dec_init(L.len, &d);
    uint64_t o = 0;
    for (uint32_t s = first; s < first + count; s++) {
        oh_stripe_t S;
        rc = parse_stripe(blob, nb, &L, s, &S);
        if (rc) return rc;
        if (o + 2ull * S.n > out_cap) return OH_E_ARG;
        uint64_t pos = 0;
        for (uint32_t i = 0; i < S.n; i++) {
            int sym = dec_one(&d, S.bits, S.n_bits, &pos);
            if (sym < 0) return OH_E_CORRUPT;
            out[o + 2ull * i] = S.even[i];
            out[o + 2ull * i + 1] = (uint8_t)sym;
        }
        if (pos != S.n_bits) return OH_E_CORRUPT;
        o += 2ull * S.n;
    }
    return OH_OK;
}

int oh_decode_layer(const uint8_t *blob, uint64_t nb, uint8_t *out, uint64_t out_bytes) {
    oh_layer_t L;
    int rc = parse_layer(blob, nb, &L);
    if (rc) return rc;
    if (out_bytes != L.raw) return OH_E_ARG;
    return oh_decode_stripes(blob, nb, 0, L.ns, out, out_bytes);
}

/* Index checker: replays the bit-by-bit decode of every stripe and compares
 * each subblock's recorded start bit and symbol count, and each lane chunk's
 * recorded code-bit count, with what the replay finds. */
int oh_check_index(const uint8_t *blob, uint64_t nb) {
    oh_layer_t L;
    int rc = parse_layer(blob, nb, &L);
    if (rc) return rc;
    rc = oh_check_table(L.len);
    if (rc) return rc;
    oh_dec_t d;
    dec_init(L.len, &d);
    uint32_t sb_total = 0;
    for (uint32_t s = 0; s < L.ns; s++) {
        oh_stripe_t S;
        rc = parse_stripe(blob, nb, &L, s, &S);
        if (rc) return rc;
        if (S.first_sb != sb_total) return OH_E_INDEX;
        uint64_t pos = 0;
        for (uint32_t b = 0; b < S.nsb; b++) {
            const uint8_t *rec = S.recs + (uint64_t)OH_REC * b;
            const uint32_t sb_syms = sb_syms_of(L.lane);
            uint32_t i0 = b * sb_syms;
            uint32_t m = S.n - i0 < sb_syms ? S.n - i0 : sb_syms;
            if (rd_le(rec, 4) != pos || rd_le(rec + 4, 4) != m) return OH_E_INDEX;
            for (uint32_t t = 0; t < OH_LANES; t++) {
                uint64_t p0 = pos;
                for (uint32_t k = 0; k < L.lane && t * L.lane + k < m; k++)
                    if (dec_one(&d, S.bits, S.n_bits, &pos) < 0) return OH_E_CORRUPT;
                if (rd_le(rec + 8 + 2 * t, 2) != pos - p0) return OH_E_INDEX;
            }
        }
        if (pos != S.n_bits) return OH_E_INDEX;
        sb_total += S.nsb;
    }
    if (sb_total != L.nsb) return OH_E_INDEX;
    return OH_OK;
}

/* Raw size recorded in a container header, or a negative error. */
int64_t oh_raw_bytes(const uint8_t *blob, uint64_t nb) {
    oh_layer_t L;
    int rc = parse_layer(blob, nb, &L);
    return rc ? rc : (int64_t)L.raw;
}
