// Host helpers shared by the native packer (k3huf_host.cpp) and the GPU
// encoder's host driver (k3huf_encode.hip): code lengths, canonical codes and
// the container geometry. Not part of the C ABI.
#ifndef K3HUF_INTERNAL_H
#define K3HUF_INTERNAL_H

#include <stdint.h>

#include "k3huf.h"

namespace k3huf_detail {

inline uint64_t pad16(uint64_t x) { return (x + 15) & ~uint64_t(15); }
// planes and stripe records start on 256-byte boundaries (whole cache lines)
inline uint64_t pad256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
inline uint32_t stripes_for(uint64_t raw) {
    return uint32_t((raw + K3HUF_STRIPE_BYTES - 1) / K3HUF_STRIPE_BYTES);
}

// Huffman leaf depths over 256 counts (0 for absent symbols); ties in weight
// go to the lower node id (leaves 0.. by symbol, merged nodes the following
// ids). No allocation.
void huffman_depths(const uint64_t* count, uint8_t* depth);

// Code lengths from the layer's odd-byte histogram (false if it is empty).
// No allocation.
bool limited_lengths(const uint64_t* count, uint8_t* len);
// Longest-first canonical codes for the lengths.
void canonical_codes(const uint8_t* len, uint32_t* code);

struct StripeGeom {
    uint64_t raw0, off;       // first raw byte, record offset in the blob
    uint32_t raw, n, nsb, nbits, bit_bytes, bits_off, even_off;
};

// the lane-chunk lengths the format allows (K3HUF_LANE_SYMS and
// K3HUF_LANE_SYMS_SHORT); a subblock holds K3HUF_LANES chunks
inline bool lane_syms_ok(uint32_t lane_syms) {
    return lane_syms == K3HUF_LANE_SYMS || lane_syms == K3HUF_LANE_SYMS_SHORT;
}

// Geometry of every stripe from the per-stripe histograms (hist[s * 256 + v])
// and the code lengths, for lane chunks of lane_syms symbols; returns the
// container size. Fills g (caller storage of stripes_for(raw_bytes) entries)
// and the subblock total. No allocation.
uint64_t layout(uint64_t raw_bytes, const uint64_t* hist, const uint8_t* len, StripeGeom* g,
                uint32_t* nsb_total, uint32_t lane_syms = K3HUF_LANE_SYMS);

// The layer header and stripe offset table (pad256(K3HUF_HDR_BYTES + 8 ns)
// bytes, zero padded) into out, from the stripes_for(raw_bytes) entries of g.
void write_layer_header(uint8_t* out, uint64_t raw_bytes, const uint8_t* len, const StripeGeom* g,
                        uint32_t nsb_total, uint64_t total, uint32_t lane_syms = K3HUF_LANE_SYMS);

}  // namespace k3huf_detail

#endif
