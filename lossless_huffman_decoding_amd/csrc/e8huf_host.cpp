// Host side of the FP8 exponent codec (include/e8huf.h): the two-level decode
// table, header parsing and the native packer.
//
// ECF8 page ("指数集中现象：GenAI模型权重压缩的理论基础", pwwt.cn/news/2030120),
// section 2.1: per-layer exponent histogram, smoothing so that no code is
// longer than 16 bits, Huffman code, a two-level 8 + 8-bit lookup table, and
// per-block metadata (bit offset, start in the symbol stream).
#include "e8huf.h"
#include "k3huf_internal.h"

#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

namespace {

inline uint64_t rd(const uint8_t* p, int n) {
    uint64_t v = 0;
    for (int i = n - 1; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}
inline void wr(uint8_t* p, uint64_t v, int n) {
    for (int i = 0; i < n; ++i, v >>= 8) p[i] = uint8_t(v);
}
using k3huf_detail::pad16;
using k3huf_detail::pad256;

constexpr int kMaxSyms = 32;
constexpr uint16_t kLink = 0x20;

uint64_t blocks_for(uint64_t n) { return (n + E8HUF_BLOCK_VALUES - 1) / E8HUF_BLOCK_VALUES; }

// Code lengths (format: Huffman depths; while a code is longer than 16 bits
// every live count c becomes c / 2 + 1 and the tree is rebuilt; a lone
// symbol gets length 1). False when no symbol occurs.
bool code_lengths(const uint64_t* count, uint8_t* len) {
    uint64_t c[256] = {};
    uint8_t d[256];
    int live = 0;
    for (int s = 0; s < kMaxSyms; ++s) {
        c[s] = count[s];
        live += count[s] != 0;
        len[s] = 0;
    }
    if (!live) return false;
    if (live == 1) {
        for (int s = 0; s < kMaxSyms; ++s) len[s] = count[s] ? 1 : 0;
        return true;
    }
    for (;;) {
        k3huf_detail::huffman_depths(c, d);
        int deepest = 0;
        for (int s = 0; s < kMaxSyms; ++s) deepest = std::max(deepest, int(d[s]));
        if (deepest <= E8HUF_MAXLEN) break;
        for (int s = 0; s < kMaxSyms; ++s)
            if (c[s]) c[s] = c[s] / 2 + 1;
    }
    for (int s = 0; s < kMaxSyms; ++s) len[s] = d[s];
    return true;
}

// Canonical codes, shortest length first.
void canonical(const uint8_t* len, uint32_t* code) {
    uint32_t cnt[E8HUF_MAXLEN + 1] = {}, next[E8HUF_MAXLEN + 1] = {};
    for (int s = 0; s < kMaxSyms; ++s)
        if (len[s]) ++cnt[len[s]];
    uint32_t c = 0;
    for (int l = 1; l <= E8HUF_MAXLEN; ++l) {
        c = (c + cnt[l - 1]) << 1;
        next[l] = c;
    }
    for (int s = 0; s < kMaxSyms; ++s) code[s] = len[s] ? next[len[s]]++ : 0;
}

int pick_threads(int n) {
    if (n > 0) return n;
    unsigned h = std::thread::hardware_concurrency();
    return int(std::max(1u, std::min(h, 64u)));
}

template <class F>
void parallel_for(int n, int threads, F f) {
    threads = std::max(1, std::min(threads, n));
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t)
        pool.emplace_back([=] {
            for (int i = t; i < n; i += threads) f(i);
        });
    for (auto& th : pool) th.join();
}

// MSB-first bit writer over bytes [first, last] of out: the first byte and a
// last partial byte may be shared with a neighbouring range, so they are
// returned in edge words for the caller to OR in; every byte strictly inside
// is stored.
struct BitWriter {
    uint8_t* out;
    uint64_t pos;        // next bit index
    uint64_t acc = 0;    // pending bits, MSB-aligned in the low `n` bits
    int n = 0;
    uint64_t first_byte;
    bool first_shared;
    uint8_t head = 0;    // first byte, when shared
    BitWriter(uint8_t* o, uint64_t p) : out(o), pos(p), first_byte(p >> 3), first_shared((p & 7) != 0) {
        n = int(p & 7);   // the bits before p in its byte are the neighbour's: zeros here
    }
    void put(uint32_t code, int len) {
        acc = (acc << len) | code;
        n += len;
        pos += uint64_t(len);
        while (n >= 8) {
            const uint64_t at = (pos - uint64_t(n)) >> 3;   // the oldest pending byte
            n -= 8;
            const uint8_t b = uint8_t(acc >> n);
            if (first_shared && at == first_byte) head = b;
            else out[at] = b;
        }
    }
    // the last partial byte (bits after it are the neighbour's): returned
    uint8_t tail() const { return n ? uint8_t(acc << (8 - n)) : 0; }
};

}  // namespace

extern "C" {

int e8huf_build_table(const uint8_t codelen[32], int exp_bits, uint16_t* lut, int* n_entries) {
    if (!codelen || !lut || !n_entries || (exp_bits != 4 && exp_bits != 5)) return K3HUF_E_ARG;
    std::memset(lut, 0, sizeof(uint16_t) * E8HUF_LUT_MAX);
    *n_entries = 0;
    const int nsym = 1 << exp_bits;
    bool any = false;
    uint64_t kraft = 0;
    for (int s = 0; s < kMaxSyms; ++s) {
        if (!codelen[s]) continue;
        if (s >= nsym) return K3HUF_E_ARG;
        if (codelen[s] > E8HUF_MAXLEN) return K3HUF_E_BADLEN;
        any = true;
        kraft += uint64_t(1) << (E8HUF_MAXLEN - codelen[s]);
    }
    if (!any) return K3HUF_E_EMPTY;
    if (kraft > (uint64_t(1) << E8HUF_MAXLEN)) return K3HUF_E_OVERSUB;
    uint32_t code[kMaxSyms];
    canonical(codelen, code);
    // level 1: codes of up to 8 bits cover 2^(8 - len) indices each; every
    // 8-bit prefix of a longer code gets a level-2 table, numbered in prefix
    // order
    int tables = 0;
    int table_of[256];
    for (int i = 0; i < 256; ++i) table_of[i] = -1;
    for (int p = 0; p < 256; ++p)
        for (int s = 0; s < kMaxSyms; ++s)
            if (codelen[s] > 8 && (code[s] >> (codelen[s] - 8)) == uint32_t(p)) {
                table_of[p] = tables++;
                break;
            }
    // at most 17 for any table accepted above (include/e8huf.h); kept as a
    // check so that no table can write past E8HUF_LUT_MAX entries
    if (256 * (1 + tables) > E8HUF_LUT_MAX) return K3HUF_E_ARG;
    for (int s = 0; s < kMaxSyms; ++s) {
        const int l = codelen[s];
        if (!l) continue;
        if (l <= 8) {
            const uint32_t lo = code[s] << (8 - l), hi = lo + (1u << (8 - l));
            for (uint32_t i = lo; i < hi; ++i) lut[i] = uint16_t((s << 8) | l);
        } else {
            const uint32_t p = code[s] >> (l - 8);
            const int t = table_of[p];
            lut[p] = uint16_t((t << 8) | kLink);
            const uint32_t rest = code[s] & ((1u << (l - 8)) - 1);
            const uint32_t lo = rest << (16 - l), hi = lo + (1u << (16 - l));
            uint16_t* l2 = lut + 256 * (1 + t);
            for (uint32_t j = lo; j < hi; ++j) l2[j] = uint16_t((s << 8) | l);
        }
    }
    *n_entries = 256 * (1 + tables);
    return K3HUF_OK;
}

int e8huf_layer_info(const void* h_blob, size_t h_bytes, e8huf_info* out) {
    if (!h_blob || !out || h_bytes < E8HUF_HDR_BYTES) return K3HUF_E_ARG;
    const uint8_t* b = static_cast<const uint8_t*>(h_blob);
    if (std::memcmp(b, "E8HF", 4) != 0 || rd(b + 4, 2) != 1 || (b[6] != 4 && b[6] != 5) ||
        b[7] != E8HUF_MAXLEN || rd(b + 16, 4) != E8HUF_BLOCK_VALUES || rd(b + 20, 4) != E8HUF_LANE_VALUES)
        return K3HUF_E_FORMAT;
    e8huf_info I;
    I.exp_bits = b[6];
    I.n_values = rd(b + 8, 8);
    I.n_blocks = uint32_t(rd(b + 24, 4));
    I.n_bits = rd(b + 32, 8);
    I.container_bytes = rd(b + 56, 8);
    if (!I.n_values || I.n_blocks != blocks_for(I.n_values) || I.n_bits > uint64_t(E8HUF_MAXLEN) * I.n_values)
        return K3HUF_E_FORMAT;
    std::memcpy(I.codelen, b + 64, 32);
    for (int s = 1 << I.exp_bits; s < kMaxSyms; ++s)
        if (I.codelen[s]) return K3HUF_E_FORMAT;
    *out = I;
    return K3HUF_OK;
}

int64_t e8huf_encode_bound(uint64_t n) {
    if (!n) return K3HUF_E_ARG;
    return int64_t(pad256(E8HUF_HDR_BYTES + E8HUF_BLOCK_REC_BYTES * blocks_for(n)) +
                   pad256(pad16((n * E8HUF_MAXLEN + 7) / 8)) + pad256((n + 1) / 2));
}

int64_t e8huf_encode(const void* h_x, uint64_t n, int exp_bits, void* h_out, uint64_t cap, int n_threads) {
    if (!h_x || !h_out || !n || (exp_bits != 4 && exp_bits != 5)) return K3HUF_E_ARG;
    if (uint64_t(e8huf_encode_bound(n)) > cap) return K3HUF_E_ARG;
    const uint8_t* x = static_cast<const uint8_t*>(h_x);
    uint8_t* out = static_cast<uint8_t*>(h_out);
    const int threads = pick_threads(n_threads);
    const int m = 7 - exp_bits;
    const uint32_t emask = (1u << exp_bits) - 1;
    const uint64_t nb = blocks_for(n);

    // exponent histogram, per block (the block bit counts come from it)
    std::vector<uint32_t> bhist(nb * kMaxSyms, 0);
    parallel_for(int(std::min<uint64_t>(nb, 4096)), threads, [&](int w) {
        for (uint64_t b = uint64_t(w); b < nb; b += 4096) {
            const uint64_t v0 = b * E8HUF_BLOCK_VALUES, v1 = std::min(n, v0 + E8HUF_BLOCK_VALUES);
            uint32_t* h = &bhist[b * kMaxSyms];
            for (uint64_t i = v0; i < v1; ++i) ++h[(x[i] >> m) & emask];
        }
    });
    uint64_t count[kMaxSyms] = {};
    for (uint64_t b = 0; b < nb; ++b)
        for (int s = 0; s < kMaxSyms; ++s) count[s] += bhist[b * kMaxSyms + s];
    uint8_t len[kMaxSyms];
    if (!code_lengths(count, len)) return K3HUF_E_ARG;
    uint32_t code[kMaxSyms];
    canonical(len, code);

    // block start bits (a prefix sum of the blocks' code bits) and layout
    std::vector<uint64_t> start(nb + 1, 0);
    for (uint64_t b = 0; b < nb; ++b) {
        uint64_t bits = 0;
        for (int s = 0; s < kMaxSyms; ++s) bits += uint64_t(bhist[b * kMaxSyms + s]) * len[s];
        start[b + 1] = start[b] + bits;
    }
    const uint64_t n_bits = start[nb];
    const uint64_t bits_off = pad256(E8HUF_HDR_BYTES + E8HUF_BLOCK_REC_BYTES * nb);
    const uint64_t nib_off = pad256(bits_off + pad16((n_bits + 7) / 8));
    const uint64_t total = pad256(nib_off + (n + 1) / 2);
    std::memset(out, 0, total);
    std::memcpy(out, "E8HF", 4);
    wr(out + 4, 1, 2);
    out[6] = uint8_t(exp_bits);
    out[7] = E8HUF_MAXLEN;
    wr(out + 8, n, 8);
    wr(out + 16, E8HUF_BLOCK_VALUES, 4);
    wr(out + 20, E8HUF_LANE_VALUES, 4);
    wr(out + 24, nb, 4);
    wr(out + 32, n_bits, 8);
    wr(out + 40, bits_off, 8);
    wr(out + 48, nib_off, 8);
    wr(out + 56, total, 8);
    std::memcpy(out + 64, len, kMaxSyms);

    // records, codes and nibbles, over contiguous ranges of blocks; the bytes
    // two ranges share are OR-ed in afterwards
    const int ranges = int(std::min<uint64_t>(nb, uint64_t(threads) * 4));
    std::vector<uint8_t> heads(ranges, 0), tails(ranges, 0);
    std::vector<uint64_t> head_at(ranges, 0), tail_at(ranges, 0);
    std::vector<char> has_head(ranges, 0), has_tail(ranges, 0);
    uint8_t* bits = out + bits_off;
    uint8_t* nib = out + nib_off;
    parallel_for(ranges, threads, [&](int r) {
        const uint64_t b0 = nb * uint64_t(r) / uint64_t(ranges), b1 = nb * uint64_t(r + 1) / uint64_t(ranges);
        if (b0 == b1) return;
        BitWriter w(bits, start[b0]);
        for (uint64_t b = b0; b < b1; ++b) {
            uint8_t* rec = out + E8HUF_HDR_BYTES + E8HUF_BLOCK_REC_BYTES * b;
            wr(rec, start[b], 8);
            const uint64_t v0 = b * E8HUF_BLOCK_VALUES, v1 = std::min(n, v0 + E8HUF_BLOCK_VALUES);
            for (uint64_t c0 = v0; c0 < v1; c0 += E8HUF_LANE_VALUES) {
                const uint64_t p0 = w.pos, c1 = std::min(v1, c0 + E8HUF_LANE_VALUES);
                for (uint64_t i = c0; i < c1; ++i) {
                    const uint32_t e = (x[i] >> m) & emask;
                    w.put(code[e], len[e]);
                }
                wr(rec + 8 + 2 * ((c0 - v0) / E8HUF_LANE_VALUES), w.pos - p0, 2);
            }
            // nibbles: blocks start at even values, so each block owns whole bytes
            for (uint64_t i = v0; i < v1; i += 2) {
                uint32_t lo = (uint32_t(x[i] >> 7) << m) | (x[i] & ((1u << m) - 1)), hi = 0;
                if (i + 1 < v1) hi = (uint32_t(x[i + 1] >> 7) << m) | (x[i + 1] & ((1u << m) - 1));
                nib[i / 2] = uint8_t(lo | (hi << 4));
            }
        }
        has_head[r] = w.first_shared;
        heads[r] = w.head;
        head_at[r] = w.first_byte;
        if (w.n) {
            has_tail[r] = 1;
            tails[r] = w.tail();
            tail_at[r] = (w.pos - uint64_t(w.n)) >> 3;
        }
    });
    for (int r = 0; r < ranges; ++r) {
        if (has_head[r]) bits[head_at[r]] |= heads[r];
        if (has_tail[r]) bits[tail_at[r]] |= tails[r];
    }
    return int64_t(total);
}

}  // extern "C"
