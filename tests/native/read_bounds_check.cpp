// CPU check of the decode kernel's read bounds (k3huf_bounds.h), compiled
// with g++ by tests/test_read_bounds.py: the same functions the kernel calls,
// with the device qualifiers defined away.
//
// For stripe records the kernel accepts (in both lane-chunk layouts: 128
// chunks of 256 or of 64 symbols per subblock), over blob sizes up to
// 2^36 - 1 and record offsets anywhere in the blob:
//   1. every clamped 16-byte bitstream read (fill path, dword index j >= -4)
//      and 8-byte read (gather path, j >= -2) lies inside the stripe's record
//      and planes, so inside [0, blob_bytes);
//   2. every dword that holds one of the stripe's n_bits code bits is read
//      unclamped, so a valid stripe decodes from its true bytes;
//   3. dmax is in [0, 2^31);
//   4. every subblock record j < nsb, read with or without the next record's
//      start_bit (as the kernel does when j + 1 < nsb), passes
//      subblock_rec_in_blob, so a record read before the stripe's values are
//      known is the right one whenever the stripe is accepted; and a record
//      that passes ends inside the blob.
// Prints "ok <records checked>" or the first failing record and exits 1.
#define __host__
#define __device__
#include <cstdio>
#include <cstdlib>

#include "k3huf_bounds.h"

using namespace k3huf_bounds;

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {   // xorshift64*
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}
static uint64_t below(uint64_t n) { return n ? next_u64() % n : 0; }
static uint64_t pad16(uint64_t x) { return (x + 15) & ~15ull; }
static uint64_t pad256(uint64_t x) { return (x + 255) & ~255ull; }

static int fail(const char* what, uint64_t blob, uint64_t soff, uint32_t n, uint32_t n_bits, uint32_t bit_bytes,
                uint32_t bits_off, uint32_t even_off, int64_t j) {
    std::printf("FAIL %s blob=%llu soff=%llu n=%u n_bits=%u bit_bytes=%u bits_off=%u even_off=%u j=%lld\n", what,
                (unsigned long long)blob, (unsigned long long)soff, n, n_bits, bit_bytes, bits_off, even_off,
                (long long)j);
    return 1;
}

// symbols per subblock of the two lane-chunk layouts (128 chunks of 256 or
// of 64 symbols)
static const uint32_t kSubSyms[2] = {K3HUF_LANES * K3HUF_LANE_SYMS, K3HUF_LANES * K3HUF_LANE_SYMS_SHORT};

static int check(uint64_t blob, uint64_t soff, uint32_t n, uint32_t n_bits, uint32_t bit_bytes, uint32_t bits_off,
                 uint32_t even_off, uint32_t sub_syms, long* accepted) {
    const uint32_t nsb = (n + sub_syms - 1) / sub_syms;
    if (!stripe_planes_ok(blob, soff, n, nsb, n_bits, bit_bytes, bits_off, even_off)) return 0;
    ++*accepted;
    const int32_t dmax = stripe_read_dmax(bits_off, even_off, n);
    if (dmax < 0 || (dmax & 3)) return fail("dmax range", blob, soff, n, n_bits, bit_bytes, bits_off, even_off, dmax);
    const uint64_t bits = soff + bits_off;
    // 1: indices near both ends and spread over the whole int range
    int32_t js[64];
    int m = 0;
    for (int32_t d = -4; d <= 8; ++d) js[m++] = d;
    for (int32_t d = -8; d <= 8; ++d) js[m++] = dmax + d;
    js[m++] = 0x7FFFFFF0;
    js[m++] = int32_t(below(0x7FFFFFFFull));
    js[m++] = int32_t(bit_bytes / 4);
    for (int i = 0; i < m; ++i) {
        const int32_t j = js[i];
        if (j < -4) continue;
        const int64_t off = clamped_read_off(j & ~3, dmax);          // fill path: 16 bytes
        if (int64_t(bits) + off < int64_t(soff + K3HUF_STRIPE_HDR_BYTES) || bits + off + 16 > blob)
            return fail("16-byte read", blob, soff, n, n_bits, bit_bytes, bits_off, even_off, j);
        if (j >= -2) {
            const int64_t o8 = clamped_read_off(j & ~1, dmax);        // gather path: 8 bytes
            if (int64_t(bits) + o8 < int64_t(soff + K3HUF_STRIPE_HDR_BYTES) || bits + o8 + 8 > blob)
                return fail("8-byte read", blob, soff, n, n_bits, bit_bytes, bits_off, even_off, j);
        }
    }
    // 4: the stripe's subblock records (first, last and a few between)
    const uint32_t jr[] = {0u, nsb - 1, nsb / 2, uint32_t(below(nsb))};
    for (uint32_t j : jr) {
        const bool nx = j + 1 < nsb;
        if (!subblock_rec_in_blob(blob, soff, j, nx))
            return fail("record outside", blob, soff, n, n_bits, bit_bytes, bits_off, even_off, j);
        if (soff + K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * (j + 1) + (nx ? 4 : 0) > blob)
            return fail("record end", blob, soff, n, n_bits, bit_bytes, bits_off, even_off, j);
    }
    // 2: the dwords holding code bits are read where they are
    if (n_bits) {
        const int32_t last = int32_t((uint64_t(n_bits) - 1) >> 5);
        if (clamped_read_off(last & ~3, dmax) != 4 * int64_t(last & ~3) ||
            clamped_read_off(last & ~1, dmax) != 4 * int64_t(last & ~1))
            return fail("code bits clamped", blob, soff, n, n_bits, bit_bytes, bits_off, even_off, last);
    }
    return 0;
}

int main() {
    long accepted = 0;
    const uint64_t kMaxBlob = (1ull << 36) - 1;
    // packer-shaped stripes (tight planes) at the start, the middle and the
    // end of blobs of every size class, including the 2^33+ sizes where a
    // blob-relative bound no longer fits 32 bits
    const uint64_t blobs[] = {4096, 1ull << 20, 1ull << 30, (1ull << 33) - 16, 1ull << 33, 9ull << 30,
                              (1ull << 35) + 4096, kMaxBlob};
    const uint32_t ns[] = {1, 2, 7, 8, 9, 255, 256, 4096, 16383, 16384, 16385, 32768, 32769, 1u << 24,
                           (1u << 25) - 1, 1u << 25};
    for (uint64_t blob : blobs)
        for (uint32_t n : ns)
            for (int k = 0; k < 64; ++k) {
                const uint32_t sub_syms = kSubSyms[k & 1];
                const uint32_t nsb = (n + sub_syms - 1) / sub_syms;
                const uint64_t n_bits = n + below(uint64_t(K3HUF_MAXLEN - 1) * n + 1);
                const uint64_t bit_bytes = pad16((n_bits + 7) / 8);
                const uint64_t bits_off = pad256(K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * nsb);
                const uint64_t even_off = pad256(bits_off + bit_bytes);
                const uint64_t span = pad256(even_off + n);
                if (span > blob) continue;
                const uint64_t where[] = {0, ((blob - span) / 2) & ~255ull, (blob - span) & ~15ull,
                                          below(blob - span + 1) & ~15ull};
                for (uint64_t soff : where)
                    if (check(blob, soff, n, uint32_t(n_bits), uint32_t(bit_bytes), uint32_t(bits_off),
                              uint32_t(even_off), sub_syms, &accepted))
                        return 1;
            }
    // arbitrary records (any field values the checks let through)
    for (long t = 0; t < 4000000; ++t) {
        const uint64_t blob = 304 + below(kMaxBlob - 303);
        const uint32_t n = 1 + uint32_t(below(1u << 25));
        const uint32_t sub_syms = kSubSyms[(t >> 3) & 1];
        const uint32_t nsb = (n + sub_syms - 1) / sub_syms;
        const uint32_t bit_bytes = uint32_t(below(1ull << 32)) & ~15u;
        const uint32_t n_bits = uint32_t(below(uint64_t(8) * bit_bytes + 1 < (1ull << 32) ? uint64_t(8) * bit_bytes + 1
                                                                                         : (1ull << 32)));
        const uint64_t min_bits = pad16(K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * nsb);
        const uint32_t bits_off = uint32_t((t & 1) ? min_bits + (below(1ull << 20) & ~15ull)
                                                   : below(1ull << 32) & ~15ull);
        const uint32_t even_off = uint32_t((t & 2) ? uint64_t(bits_off) + bit_bytes + (below(1ull << 12) & ~15ull)
                                                   : below(1ull << 32) & ~15ull);
        const uint64_t soff = (t & 4) ? below(blob) & ~15ull : (blob - (blob >> (1 + t % 30))) & ~15ull;
        if (check(blob, soff, n, n_bits, bit_bytes, bits_off, even_off, sub_syms, &accepted)) return 1;
    }
    // a record that passes subblock_rec_in_blob ends inside the blob, for
    // any offset and index the kernel can form (offsets below 2^36, j < 4096)
    for (long t = 0; t < 4000000; ++t) {
        const uint64_t blob = 304 + below(kMaxBlob - 303);
        const uint64_t back = below(blob < (1ull << 20) ? blob : (1ull << 20));
        const uint64_t soff = (t & 1) ? below(blob) & ~15ull : (blob - back) & ~15ull;
        const uint32_t j = uint32_t(below(4096));
        const bool nx = (t & 2) != 0;
        const uint64_t end = soff + K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * j +
                             K3HUF_SUBBLOCK_REC_BYTES + (nx ? 4 : 0);
        if (subblock_rec_in_blob(blob, soff, j, nx) != (end <= blob))
            return fail("record test", blob, soff, 0, 0, 0, 0, 0, j);
    }
    std::printf("ok %ld\n", accepted);
    return accepted > 100000 ? 0 : 1;
}
