// Read bounds of the decode kernel, as host-and-device functions so that the
// same arithmetic the kernel runs can be checked exhaustively on the CPU.
// Container layout: include/k3huf.h.
//
// A stripe record is accepted only when everything the kernel reads for the
// stripe lies inside the blob: the record itself, its subblock records, and
// its two planes, the bitstream at bits_off and the even plane at even_off,
// which runs to even_off + pad16(n_syms). Reads of the bitstream are then
// clamped to that stripe's own planes, with offsets taken relative to the
// stripe's bitstream start, so their range does not depend on where the
// stripe sits in the blob or on how large the blob is.
#ifndef K3HUF_BOUNDS_H
#define K3HUF_BOUNDS_H

#include <stdint.h>

#include "k3huf.h"

namespace k3huf_bounds {

// The record checks that bound the kernel's reads of stripe s, whose record
// starts at blob offset soff and which holds n_syms symbols in nsb subblocks
// (the other fields come from the record): the record is 16-byte aligned and
// inside the blob, the subblock records end before the bitstream, the
// bitstream ends before the even plane, and the padded even plane ends
// inside the blob. All in 64-bit arithmetic.
__host__ __device__ inline bool stripe_planes_ok(uint64_t blob_bytes, uint64_t soff, uint32_t n_syms,
                                                 uint32_t nsb, uint32_t n_bits, uint32_t bit_bytes,
                                                 uint32_t bits_off, uint32_t even_off) {
    return (soff & 15) == 0 && soff + K3HUF_STRIPE_HDR_BYTES <= blob_bytes && (bits_off & 15) == 0 &&
           (even_off & 15) == 0 &&
           uint64_t(bits_off) >= K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * nsb &&
           uint64_t(n_bits) <= 8ull * bit_bytes && uint64_t(even_off) >= uint64_t(bits_off) + bit_bytes &&
           soff + even_off + ((uint64_t(n_syms) + 15) & ~15ull) <= blob_bytes;
}

// Whether subblock record j of the stripe record at soff lies inside the
// blob, together with the next record's start_bit when has_next (the bytes a
// decoder reads for the record: [rec, rec + 264), or [rec, rec + 268)). For a
// stripe that stripe_planes_ok accepts, every record j < nsb passes: the
// records end at or before bits_off, inside the blob. So a decoder may read
// a record before it has the stripe's other values, sending a read this
// test fails to the blob's first bytes instead.
__host__ __device__ inline bool subblock_rec_in_blob(uint64_t blob_bytes, uint64_t soff, uint32_t j,
                                                     bool has_next) {
    return soff + K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * j + K3HUF_SUBBLOCK_REC_BYTES +
               (has_next ? 4u : 0u) <=
           blob_bytes;
}

// Largest dword index, counted from the stripe's bitstream start and a
// multiple of 4, at which a 16-byte read still ends inside the stripe's
// padded even plane. For an accepted record with n_syms >= 1 it lies in
// [0, 2^31): even_off < 2^32 and the padded even plane holds at most 2^25
// bytes.
__host__ __device__ inline int32_t stripe_read_dmax(uint32_t bits_off, uint32_t even_off, uint32_t n_syms) {
    const uint64_t end = uint64_t(even_off) + ((uint64_t(n_syms) + 15) & ~15ull);
    return int32_t(((end - bits_off - 16) >> 2) & ~3ull);
}

// Byte offset from the bitstream start of the read the kernel makes for
// dword index j (j >= -4: a window starts at most one 16-byte unit before
// the stripe's first code, inside the stripe's subblock records), clamped to
// dmax. 64-bit, so no product of a clamped index overflows.
__host__ __device__ inline int64_t clamped_read_off(int32_t j, int32_t dmax) {
    return 4 * int64_t(j < dmax ? j : dmax);
}

}  // namespace k3huf_bounds

#endif
