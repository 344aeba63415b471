// Host side of the k3huf library: decode-table build, header parsing and the
// native packer. Container layout and sources: include/k3huf.h.
#include "k3huf.h"
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
using k3huf_detail::stripes_for;
using k3huf_detail::StripeGeom;

int kraft_units(const uint8_t* len) {
    int k = 0;
    for (int s = 0; s < 256; ++s)
        if (len[s]) k += 1 << (K3HUF_MAXLEN - len[s]);
    return k;
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

}  // namespace

namespace k3huf_detail {

// Huffman leaf depths with a binary heap keyed (weight, node id); leaves get
// ids 0.. in ascending symbol order and merged nodes the following ids, so the
// tree -- and the container -- is reproducible. Fixed-size arrays: at most 256
// leaves and 255 merged nodes, no heap allocation.
void huffman_depths(const uint64_t* count, uint8_t* depth) {
    struct Node { uint64_t w; int id; };
    auto before = [](const Node& a, const Node& b) { return a.w != b.w ? a.w < b.w : a.id < b.id; };
    Node heap[256];
    int size = 0, nodes = 0;
    int parent[511];
    int leaf[256];
    auto push = [&](Node x) {
        int i = size++;
        while (i > 0 && before(x, heap[(i - 1) / 2])) {
            heap[i] = heap[(i - 1) / 2];
            i = (i - 1) / 2;
        }
        heap[i] = x;
    };
    auto pop = [&]() {
        const Node top = heap[0];
        const Node x = heap[--size];
        int i = 0;
        for (;;) {
            int c = 2 * i + 1;
            if (c >= size) break;
            if (c + 1 < size && before(heap[c + 1], heap[c])) ++c;
            if (!before(heap[c], x)) break;
            heap[i] = heap[c];
            i = c;
        }
        if (size > 0) heap[i] = x;
        return top;
    };
    for (int s = 0; s < 256; ++s) {
        depth[s] = 0;
        leaf[s] = -1;
        if (count[s]) {
            leaf[s] = nodes;
            parent[nodes] = -1;
            push({count[s], nodes++});
        }
    }
    while (size > 1) {
        const Node a = pop();
        const Node b = pop();
        const int p = nodes++;
        parent[p] = -1;
        parent[a.id] = p;
        parent[b.id] = p;
        push({a.w + b.w, p});
    }
    for (int s = 0; s < 256; ++s) {
        if (leaf[s] < 0) continue;
        int d = 0;
        for (int x = leaf[s]; parent[x] >= 0; x = parent[x]) ++d;
        depth[s] = uint8_t(std::min(d, 255));
    }
}

// Code lengths for the layer: Huffman depths, then the 12-bit limit (K3
// page, "canonical code assignment and Kraft check": while the Kraft sum is
// over-full, lengthen the least frequent code), then shorten the most
// frequent codes that still fit until the table is exactly full, so the
// longest-first canonical codes are prefix-free. Ties: lengthen the larger
// symbol, shorten the smaller one. A lone symbol gets length 1.
bool limited_lengths(const uint64_t* count, uint8_t* len) {
    int live = 0;
    for (int s = 0; s < 256; ++s) live += count[s] != 0;
    if (!live) return false;
    huffman_depths(count, len);
    if (live == 1) {
        for (int s = 0; s < 256; ++s) len[s] = count[s] ? 1 : 0;
        return true;
    }
    for (int s = 0; s < 256; ++s)
        if (len[s] > K3HUF_MAXLEN) len[s] = K3HUF_MAXLEN;
    const int full = 1 << K3HUF_MAXLEN;
    int k = kraft_units(len);
    while (k > full) {
        int pick = -1;
        for (int s = 255; s >= 0; --s)
            if (count[s] && len[s] < K3HUF_MAXLEN && (pick < 0 || count[s] < count[pick])) pick = s;
        k -= 1 << (K3HUF_MAXLEN - 1 - len[pick]);
        ++len[pick];
    }
    while (k < full) {
        int pick = -1;
        for (int s = 0; s < 256; ++s) {
            if (!count[s] || len[s] <= 1 || (1 << (K3HUF_MAXLEN - len[s])) > full - k) continue;
            if (pick < 0 || count[s] > count[pick]) pick = s;
        }
        if (pick < 0) break;
        k += 1 << (K3HUF_MAXLEN - len[pick]);
        --len[pick];
    }
    return true;
}

void canonical_codes(const uint8_t* len, uint32_t* code) {
    uint32_t cnt[K3HUF_MAXLEN + 1] = {}, next[K3HUF_MAXLEN + 1] = {};
    for (int s = 0; s < 256; ++s)
        if (len[s]) ++cnt[len[s]];
    uint32_t c = 0;
    for (int l = K3HUF_MAXLEN; l >= 1; --l) {
        next[l] = c;
        c = (c + cnt[l]) >> 1;
    }
    for (int s = 0; s < 256; ++s) code[s] = len[s] ? next[len[s]]++ : 0;
}

uint64_t layout(uint64_t raw_bytes, const uint64_t* hist, const uint8_t* len, StripeGeom* g,
                uint32_t* nsb_total, uint32_t lane_syms) {
    const uint32_t ns = stripes_for(raw_bytes);
    const uint32_t sub_syms = K3HUF_LANES * lane_syms;
    for (uint32_t s = 0; s < ns; ++s) g[s] = StripeGeom{};
    uint64_t o = pad256(K3HUF_HDR_BYTES + 8ull * ns);
    uint32_t nsb = 0;
    for (uint32_t s = 0; s < ns; ++s) {
        StripeGeom& G = g[s];
        G.raw0 = uint64_t(s) * K3HUF_STRIPE_BYTES;
        G.raw = uint32_t(std::min<uint64_t>(K3HUF_STRIPE_BYTES, raw_bytes - G.raw0));
        G.n = G.raw / 2;
        G.nsb = (G.n + sub_syms - 1) / sub_syms;
        uint64_t nbits = 0;
        for (int v = 0; v < 256; ++v) nbits += hist[size_t(s) * 256 + v] * len[v];
        G.nbits = uint32_t(nbits);
        G.bit_bytes = uint32_t(pad16((nbits + 7) / 8));
        G.bits_off = uint32_t(pad256(K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * G.nsb));
        G.even_off = uint32_t(pad256(uint64_t(G.bits_off) + G.bit_bytes));
        G.off = o;
        o += pad256(uint64_t(G.even_off) + G.n);
        nsb += G.nsb;
    }
    *nsb_total = nsb;
    return o;
}

void write_layer_header(uint8_t* out, uint64_t raw_bytes, const uint8_t* len, const StripeGeom* g,
                        uint32_t nsb_total, uint64_t total, uint32_t lane_syms) {
    const uint32_t ns = stripes_for(raw_bytes);
    std::memset(out, 0, pad256(K3HUF_HDR_BYTES + 8ull * ns));
    std::memcpy(out, "K3HF", 4);
    wr(out + 4, 1, 2);
    wr(out + 6, K3HUF_MAXLEN, 2);
    wr(out + 8, K3HUF_STRIPE_BYTES, 4);
    wr(out + 12, 2ull * K3HUF_LANES * lane_syms, 4);
    wr(out + 16, lane_syms, 4);
    wr(out + 20, ns, 4);
    wr(out + 24, raw_bytes, 8);
    wr(out + 32, nsb_total, 4);
    wr(out + 36, 0, 4);
    wr(out + 40, total, 8);
    std::memcpy(out + 48, len, 256);
    for (uint32_t s = 0; s < ns; ++s) wr(out + K3HUF_HDR_BYTES + 8ull * s, g[s].off, 8);
}

}  // namespace k3huf_detail

using k3huf_detail::canonical_codes;
using k3huf_detail::lane_syms_ok;
using k3huf_detail::limited_lengths;

extern "C" {

const char* k3huf_strerror(int code) {
    switch (code) {
        case K3HUF_OK: return "ok";
        case K3HUF_E_ARG: return "bad argument";
        case K3HUF_E_EMPTY: return "code table is empty";
        case K3HUF_E_OVERSUB: return "code table over-fills the 12-bit code space";
        case K3HUF_E_BADLEN: return "code length above 12";
        case K3HUF_E_OVERLAP: return "canonical codes are not prefix-free";
        case K3HUF_E_FORMAT: return "malformed container";
        case K3HUF_E_CORRUPT: return "container data inconsistent";
        case K3HUF_E_HIP: return "HIP runtime error";
        default: return "unknown error";
    }
}

int k3huf_build_table(const uint8_t codelen[256], uint16_t lut[4096]) {
    if (!codelen || !lut) return K3HUF_E_ARG;
    std::memset(lut, 0, K3HUF_LUT_ENTRIES * sizeof(uint16_t));
    uint32_t cnt[K3HUF_MAXLEN + 1] = {};
    bool any = false;
    for (int s = 0; s < 256; ++s) {
        if (codelen[s] > K3HUF_MAXLEN) return K3HUF_E_BADLEN;
        if (codelen[s]) { ++cnt[codelen[s]]; any = true; }
    }
    if (!any) return K3HUF_E_EMPTY;
    if (kraft_units(codelen) > (1 << K3HUF_MAXLEN)) return K3HUF_E_OVERSUB;
    uint32_t code[256];
    canonical_codes(codelen, code);
    for (int s = 0; s < 256; ++s) {
        const int l = codelen[s];
        if (!l) continue;
        if (code[s] >= (1u << l)) {
            std::memset(lut, 0, K3HUF_LUT_ENTRIES * sizeof(uint16_t));
            return K3HUF_E_OVERLAP;
        }
        const uint32_t lo = code[s] << (K3HUF_MAXLEN - l), n = 1u << (K3HUF_MAXLEN - l);
        for (uint32_t i = lo; i < lo + n; ++i) {
            if (lut[i]) {
                std::memset(lut, 0, K3HUF_LUT_ENTRIES * sizeof(uint16_t));
                return K3HUF_E_OVERLAP;
            }
            lut[i] = uint16_t((s << 4) | l);
        }
    }
    return K3HUF_OK;
}

int k3huf_layer_info(const void* h_blob, size_t h_bytes, k3huf_info* out) {
    if (!h_blob || !out || h_bytes < K3HUF_HDR_BYTES) return K3HUF_E_ARG;
    const uint8_t* b = static_cast<const uint8_t*>(h_blob);
    const uint32_t lane_syms = uint32_t(rd(b + 16, 4));
    const uint64_t sub_bytes = 2ull * K3HUF_LANES * lane_syms;
    if (std::memcmp(b, "K3HF", 4) != 0 || rd(b + 4, 2) != 1 || rd(b + 6, 2) != K3HUF_MAXLEN ||
        rd(b + 8, 4) != K3HUF_STRIPE_BYTES || !lane_syms_ok(lane_syms) || rd(b + 12, 4) != sub_bytes)
        return K3HUF_E_FORMAT;
    k3huf_info I;
    I.lane_syms = lane_syms;
    I.n_stripes = uint32_t(rd(b + 20, 4));
    I.raw_bytes = rd(b + 24, 8);
    I.n_subblocks = uint32_t(rd(b + 32, 4));
    I.container_bytes = rd(b + 40, 8);
    if (!I.raw_bytes || (I.raw_bytes & 1) || I.n_stripes != stripes_for(I.raw_bytes) ||
        I.n_subblocks != (I.raw_bytes + sub_bytes - 1) / sub_bytes ||
        I.container_bytes < K3HUF_HDR_BYTES + 8ull * I.n_stripes)
        return K3HUF_E_FORMAT;
    std::memcpy(I.codelen, b + 48, 256);
    *out = I;
    return K3HUF_OK;
}

int64_t k3huf_encode_bound_lanes(uint64_t raw, uint32_t lane_syms) {
    if (!raw || (raw & 1) || !lane_syms_ok(lane_syms)) return K3HUF_E_ARG;
    const uint64_t sub_syms = uint64_t(K3HUF_LANES) * lane_syms;
    const uint64_t ns = stripes_for(raw);
    uint64_t b = pad256(K3HUF_HDR_BYTES + 8 * ns);
    for (uint64_t s = 0; s < ns; ++s) {
        const uint64_t rb = std::min<uint64_t>(K3HUF_STRIPE_BYTES, raw - s * K3HUF_STRIPE_BYTES);
        const uint64_t n = rb / 2, nsb = (n + sub_syms - 1) / sub_syms;
        b += pad256(K3HUF_STRIPE_HDR_BYTES + K3HUF_SUBBLOCK_REC_BYTES * nsb) +
             pad256(pad16((n * K3HUF_MAXLEN + 7) / 8)) + pad256(n);
    }
    return int64_t(b);
}

int64_t k3huf_encode_bound(uint64_t raw) { return k3huf_encode_bound_lanes(raw, K3HUF_LANE_SYMS); }

uint32_t k3huf_lane_syms_for(uint64_t raw_bytes) {
    return raw_bytes <= K3HUF_SHORT_LANES_MAX_RAW ? K3HUF_LANE_SYMS_SHORT : K3HUF_LANE_SYMS;
}

int64_t k3huf_encode_layer_lanes(const void* h_raw, uint64_t raw_bytes, uint32_t lane_syms, void* h_out,
                                 uint64_t cap, int n_threads) {
    if (!h_raw || !h_out || !raw_bytes || (raw_bytes & 1) || !lane_syms_ok(lane_syms)) return K3HUF_E_ARG;
    if (uint64_t(k3huf_encode_bound_lanes(raw_bytes, lane_syms)) > cap) return K3HUF_E_ARG;
    const uint32_t sub_syms = K3HUF_LANES * lane_syms;
    const uint8_t* raw = static_cast<const uint8_t*>(h_raw);
    uint8_t* out = static_cast<uint8_t*>(h_out);
    const int threads = pick_threads(n_threads);
    const uint32_t ns = stripes_for(raw_bytes);

    // per-stripe histograms of the odd (high) bytes
    std::vector<uint64_t> hist(size_t(ns) * 256, 0);
    std::vector<StripeGeom> g(ns);
    for (uint32_t s = 0; s < ns; ++s) {
        g[s].raw0 = uint64_t(s) * K3HUF_STRIPE_BYTES;
        g[s].raw = uint32_t(std::min<uint64_t>(K3HUF_STRIPE_BYTES, raw_bytes - g[s].raw0));
        g[s].n = g[s].raw / 2;
    }
    parallel_for(int(ns), threads, [&](int s) {
        uint64_t h[4][256] = {};
        const uint8_t* p = raw + g[s].raw0;
        uint32_t i = 0;
        for (; i + 4 <= g[s].n; i += 4) {
            ++h[0][p[2 * i + 1]]; ++h[1][p[2 * i + 3]];
            ++h[2][p[2 * i + 5]]; ++h[3][p[2 * i + 7]];
        }
        for (; i < g[s].n; ++i) ++h[0][p[2 * i + 1]];
        for (int v = 0; v < 256; ++v) hist[size_t(s) * 256 + v] = h[0][v] + h[1][v] + h[2][v] + h[3][v];
    });
    uint64_t count[256] = {};
    for (uint32_t s = 0; s < ns; ++s)
        for (int v = 0; v < 256; ++v) count[v] += hist[size_t(s) * 256 + v];
    uint8_t len[256];
    if (!limited_lengths(count, len)) return K3HUF_E_ARG;
    uint32_t code[256];
    canonical_codes(len, code);

    // layout: every stripe's size is known from its histogram
    uint32_t nsb_total = 0;
    const uint64_t total = k3huf_detail::layout(raw_bytes, hist.data(), len, g.data(), &nsb_total, lane_syms);
    k3huf_detail::write_layer_header(out, raw_bytes, len, g.data(), nsb_total, total, lane_syms);

    // stripes are independent (K3 page, "key design points"): pack in parallel
    parallel_for(int(ns), threads, [&](int s) {
        const StripeGeom& G = g[s];
        uint8_t* st = out + G.off;
        const uint64_t span = pad256(uint64_t(G.even_off) + G.n);
        std::memset(st, 0, span);
        wr(st + 0, G.raw, 4);
        wr(st + 4, G.n, 4);
        wr(st + 8, G.nbits, 4);
        wr(st + 12, G.bit_bytes, 4);
        wr(st + 16, uint64_t(s) * (K3HUF_STRIPE_BYTES / (2ull * sub_syms)), 4);
        wr(st + 20, G.nsb, 4);
        wr(st + 24, G.bits_off, 4);
        wr(st + 28, G.even_off, 4);
        const uint8_t* p = raw + G.raw0;
        uint8_t* bits = st + G.bits_off;
        uint8_t* even = st + G.even_off;
        uint64_t acc = 0;   // pending bits, left-aligned at bit 63
        int nacc = 0;
        uint64_t pos = 0;   // bits emitted so far
        size_t wbyte = 0;
        for (uint32_t b = 0; b < G.nsb; ++b) {
            uint8_t* rec = st + K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * b;
            const uint32_t i0 = b * sub_syms;
            const uint32_t m = std::min<uint32_t>(sub_syms, G.n - i0);
            wr(rec, pos, 4);
            wr(rec + 4, m, 4);
            for (uint32_t t = 0; t < K3HUF_LANES; ++t) {
                const uint32_t j0 = i0 + t * lane_syms;
                const uint32_t j1 = std::min<uint32_t>(j0 + lane_syms, i0 + m);
                const uint64_t p0 = pos;
                for (uint32_t i = j0; i < j1; ++i) {
                    const uint8_t v = p[2ull * i + 1];
                    even[i] = p[2ull * i];
                    const int l = len[v];
                    acc |= uint64_t(code[v]) << (64 - nacc - l);
                    nacc += l;
                    pos += l;
                    while (nacc >= 8) {
                        bits[wbyte++] = uint8_t(acc >> 56);
                        acc <<= 8;
                        nacc -= 8;
                    }
                }
                wr(rec + 8 + 2 * t, pos - p0, 2);
            }
        }
        if (nacc > 0) bits[wbyte++] = uint8_t(acc >> 56);
    });
    return int64_t(total);
}

int64_t k3huf_encode_layer(const void* h_raw, uint64_t raw_bytes, void* h_out, uint64_t cap, int n_threads) {
    return k3huf_encode_layer_lanes(h_raw, raw_bytes, K3HUF_LANE_SYMS, h_out, cap, n_threads);
}

}  // extern "C"
