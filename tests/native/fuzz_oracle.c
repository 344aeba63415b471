/* Container-parsing fuzz of the CPU oracle, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py (test-only).
 * Seeded random layers are encoded and decoded (round trip), then truncated
 * copies and copies with random byte flips in the header, the records and
 * the bitstream are fed to the oracle's parsers and decoders: each call must
 * return (an error or a decode) without any invalid memory access, which the
 * sanitizers would report. Both codecs: bf16 high bytes (k3huf_oracle.c) and
 * FP8 exponents (e8huf_oracle.c). Prints "ok <cases>". */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oh_encode_bound(uint64_t raw);
int64_t oh_encode_layer(const uint8_t *raw, uint64_t n_raw, uint8_t *out, uint64_t cap);
int oh_decode_layer(const uint8_t *blob, uint64_t nb, uint8_t *out, uint64_t out_bytes);
int oh_check_index(const uint8_t *blob, uint64_t nb);
int64_t oh_raw_bytes(const uint8_t *blob, uint64_t nb);
int64_t e8_encode_bound(uint64_t n);
int64_t e8_encode(const uint8_t *x, uint64_t n, int exp_bits, uint8_t *out, uint64_t cap);
int e8_decode(const uint8_t *blob, uint64_t size, uint8_t *out, uint64_t n);
int e8_check_index(const uint8_t *blob, uint64_t size);
int64_t e8_n_values(const uint8_t *blob, uint64_t size);

static uint64_t st = 0x243F6A8885A308D3ull;
static uint64_t rnd(void) {   /* xorshift64* */
    st ^= st >> 12; st ^= st << 25; st ^= st >> 27;
    return st * 0x2545F4914F6CDD1Dull;
}

/* decode a (possibly damaged) copy of exactly `len` bytes: the copy lives in
 * its own heap block, so a read past its end is caught */
static void k3_try(const uint8_t *blob, uint64_t len) {
    uint8_t *c = malloc(len ? len : 1);
    memcpy(c, blob, len);
    int64_t raw = oh_raw_bytes(c, len);
    (void)oh_check_index(c, len);
    if (raw > 0 && raw < (1 << 24)) {
        uint8_t *out = malloc((size_t)raw);
        (void)oh_decode_layer(c, len, out, (uint64_t)raw);
        free(out);
    }
    free(c);
}

static void e8_try(const uint8_t *blob, uint64_t len) {
    uint8_t *c = malloc(len ? len : 1);
    memcpy(c, blob, len);
    int64_t n = e8_n_values(c, len);
    (void)e8_check_index(c, len);
    if (n > 0 && n < (1 << 24)) {
        uint8_t *out = malloc((size_t)n);
        (void)e8_decode(c, len, out, (uint64_t)n);
        free(out);
    }
    free(c);
}

int main(void) {
    long cases = 0;
    for (int trial = 0; trial < 60; trial++) {
        /* a layer of random size; high bytes from a small random alphabet */
        uint64_t n = 2 * (1 + rnd() % (trial < 40 ? 40000 : 300000));
        uint8_t *x = malloc(n);
        int k = 1 + (int)(rnd() % 40);
        for (uint64_t i = 0; i < n; i++)
            x[i] = (i & 1) ? (uint8_t)(0x38 + (rnd() % (uint64_t)k) * (rnd() % 3 ? 1 : 7)) : (uint8_t)rnd();
        int64_t cap = oh_encode_bound(n);
        uint8_t *blob = malloc((size_t)cap);
        int64_t len = oh_encode_layer(x, n, blob, (uint64_t)cap);
        if (len <= 0) { printf("k3 encode failed %lld\n", (long long)len); return 1; }
        uint8_t *y = malloc(n);
        if (oh_decode_layer(blob, (uint64_t)len, y, n) != 0 || memcmp(x, y, n) != 0) { printf("k3 round trip\n"); return 1; }
        for (int t = 0; t < 24; t++, cases++) k3_try(blob, rnd() % (uint64_t)len);
        for (int t = 0; t < 40; t++, cases++) {
            uint8_t *c = malloc((size_t)len);
            memcpy(c, blob, (size_t)len);
            int flips = 1 + (int)(rnd() % 4);
            for (int f = 0; f < flips; f++) {
                uint64_t at = (rnd() % 3 == 0) ? rnd() % 640 : rnd() % (uint64_t)len;   /* header/records often */
                c[at] ^= (uint8_t)(1u << (rnd() % 8));
            }
            k3_try(c, (uint64_t)len);
            free(c);
        }
        free(blob);

        /* the same bytes as an FP8 tensor, both formats */
        for (int eb = 4; eb <= 5; eb++) {
            int64_t cap8 = e8_encode_bound(n);
            uint8_t *b8 = malloc((size_t)cap8);
            int64_t len8 = e8_encode(x, n, eb, b8, (uint64_t)cap8);
            if (len8 <= 0) { printf("e8 encode failed\n"); return 1; }
            if (e8_decode(b8, (uint64_t)len8, y, n) != 0 || memcmp(x, y, n) != 0) { printf("e8 round trip\n"); return 1; }
            for (int t = 0; t < 16; t++, cases++) e8_try(b8, rnd() % (uint64_t)len8);
            for (int t = 0; t < 30; t++, cases++) {
                uint8_t *c = malloc((size_t)len8);
                memcpy(c, b8, (size_t)len8);
                int flips = 1 + (int)(rnd() % 4);
                for (int f = 0; f < flips; f++) {
                    uint64_t at = (rnd() % 3 == 0) ? rnd() % 400 : rnd() % (uint64_t)len8;
                    c[at] ^= (uint8_t)(1u << (rnd() % 8));
                }
                e8_try(c, (uint64_t)len8);
                free(c);
            }
            free(b8);
        }
        free(y);
        free(x);
    }
    printf("ok %ld\n", cases);
    return 0;
}
