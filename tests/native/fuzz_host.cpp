// Fuzz of the library's host code (k3huf_host.cpp, e8huf_host.cpp), built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py (test-only; no GPU code is built). The packers run
// on seeded random layers; the header parsers run on truncated and bit-flipped
// containers, each in a heap block of its exact length; the table builders
// run on random and invalid code-length vectors. Every call must return
// without an invalid memory access or undefined behaviour. Prints "ok <n>".
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "e8huf.h"
#include "k3huf.h"

static uint64_t st = 0x13198A2E03707344ull;
static uint64_t rnd() {
    st ^= st >> 12;
    st ^= st << 25;
    st ^= st >> 27;
    return st * 0x2545F4914F6CDD1Dull;
}

int main() {
    long cases = 0;
    for (int trial = 0; trial < 40; ++trial) {
        const uint64_t n = 2 * (1 + rnd() % 200000);
        std::vector<uint8_t> x(n);
        const int k = 1 + int(rnd() % 64);
        for (uint64_t i = 0; i < n; ++i) x[i] = (i & 1) ? uint8_t(0x30 + rnd() % uint64_t(k)) : uint8_t(rnd());
        // bf16 packer and header parse
        std::vector<uint8_t> blob(size_t(k3huf_encode_bound(n)));
        const int64_t len = k3huf_encode_layer(x.data(), n, blob.data(), blob.size(), 1 + int(rnd() % 4));
        if (len <= 0) { std::printf("k3 encode %lld\n", (long long)len); return 1; }
        for (int t = 0; t < 64; ++t, ++cases) {
            const size_t cut = (t < 16) ? size_t(rnd() % 400) : size_t(len);
            uint8_t* c = static_cast<uint8_t*>(std::malloc(cut ? cut : 1));
            std::memcpy(c, blob.data(), cut);
            if (t >= 16 && cut) c[rnd() % std::min<size_t>(cut, 400)] ^= uint8_t(1u << (rnd() % 8));
            k3huf_info info;
            (void)k3huf_layer_info(c, cut, &info);
            std::free(c);
        }
        // FP8 packer and header parse, both formats
        for (int eb = 4; eb <= 5; ++eb) {
            std::vector<uint8_t> b8(size_t(e8huf_encode_bound(n)));
            const int64_t l8 = e8huf_encode(x.data(), n, eb, b8.data(), b8.size(), 1 + int(rnd() % 4));
            if (l8 <= 0) { std::printf("e8 encode %lld\n", (long long)l8); return 1; }
            for (int t = 0; t < 48; ++t, ++cases) {
                const size_t cut = (t < 16) ? size_t(rnd() % 200) : size_t(l8);
                uint8_t* c = static_cast<uint8_t*>(std::malloc(cut ? cut : 1));
                std::memcpy(c, b8.data(), cut);
                if (t >= 16 && cut) c[rnd() % std::min<size_t>(cut, 128)] ^= uint8_t(1u << (rnd() % 8));
                e8huf_info info;
                (void)e8huf_layer_info(c, cut, &info);
                std::free(c);
            }
        }
    }
    // table builders on random length vectors (valid, over-full, too long)
    std::vector<uint16_t> lut(4096), l8(E8HUF_LUT_MAX);
    for (int t = 0; t < 20000; ++t, ++cases) {
        uint8_t len[256] = {};
        const int live = 1 + int(rnd() % 256);
        for (int i = 0; i < live; ++i) len[rnd() % 256] = uint8_t(rnd() % 15);
        (void)k3huf_build_table(len, lut.data());
        uint8_t l32[32] = {};
        const int eb = 4 + int(rnd() % 2);
        for (int i = 0; i < 32; ++i) l32[i] = (rnd() % 3) ? uint8_t(rnd() % 19) : 0;
        if (rnd() % 2)
            for (int i = 1 << eb; i < 32; ++i) l32[i] = 0;
        int entries = 0;
        (void)e8huf_build_table(l32, eb, l8.data(), &entries);
        if (entries > E8HUF_LUT_MAX) { std::printf("entries %d\n", entries); return 1; }
    }
    std::printf("ok %ld\n", cases);
    return 0;
}
