/*
 * e8huf.h -- C ABI of the MI355X (gfx950) decoder for FP8 tensors whose
 * exponent field is coded with a canonical Huffman code of at most 16 bits
 * (the ECF8-style variant of the k3huf library).
 *
 * Source: the ECF8 page ("指数集中现象：GenAI模型权重压缩的理论基础",
 * pwwt.cn/news/2030120). Section 1.2: the base format is FP8 (E4M3 or E5M2).
 * Section 2.1: per layer, the exponent values' frequencies are counted and
 * smoothed so that no code gets extremely long (at most 16 bits), a Huffman
 * code is built, a two-level lookup table is generated (the first level on an
 * 8-bit prefix decodes directly or points to a second-level table on the next
 * 8 bits), and metadata per thread block records its bit offset and its start
 * in the symbol stream. Section 2.2: the GPU decoder gives each thread its
 * start bit from that metadata, decodes into on-chip memory and writes out
 * coalesced; its output is 16-bit floats (e8huf_decode_widen), or here also
 * the FP8 bytes themselves (e8huf_decode).
 *
 * All functions are plain C: pointers and sizes only. A "stream" is a
 * hipStream_t passed as void* (NULL = the null stream). Return codes are the
 * K3HUF_* codes of k3huf.h (0 or negative); functions never throw.
 *
 * ---------------------------------------------------------------------------
 * Container ("E8HF"), all integers little-endian.
 *   header, E8HUF_HDR_BYTES = 128:
 *     0  char[4] "E8HF"        4  u16 version = 1
 *     6  u8 exp_bits (4: E4M3 s eeee mmm, 5: E5M2 s eeeee mm)
 *     7  u8 maxlen = 16         8  u64 n_values (> 0)
 *     16 u32 block_values = 16384   20 u32 lane_values = 256
 *     24 u32 n_blocks = ceil(n_values / 16384)   28 u32 reserved = 0
 *     32 u64 n_bits (code bits of the whole tensor)
 *     40 u64 bits_off    48 u64 nib_off    (from the blob start, multiples of 256)
 *     56 u64 container_bytes
 *     64 u8 codelen[32] (exponent field -> code length, 0 = absent; entries
 *        at and past 2^exp_bits are 0)     96..127 zero
 *   128: n_blocks block records, E8HUF_BLOCK_REC_BYTES = 136 each:
 *     u64 start_bit (bit index of the block's first code),
 *     u16 lane_bits[64] (code bits of each 256-value lane chunk; 0 past the
 *     last value); zero pad to 256
 *   bits_off: the exponent codes, most-significant bit first, zero padded to
 *     a multiple of 16 bytes, then to 256
 *   nib_off: ceil(n_values / 2) bytes of sign/mantissa nibbles (sign << m |
 *     mantissa, m = 7 - exp_bits), value 2i in the low nibble of byte i, the
 *     odd one in the high nibble; zero padded to 256; container_bytes =
 *     nib_off + that padded plane.
 * Codes are canonical, shortest first: first[1] = 0, first[l] =
 * (first[l-1] + count[l-1]) << 1, ascending exponent values take consecutive
 * codes within a length.
 */
#ifndef E8HUF_H
#define E8HUF_H

#include <stddef.h>
#include <stdint.h>

#include "k3huf.h"

#ifdef __cplusplus
extern "C" {
#endif

#define E8HUF_MAXLEN 16
#define E8HUF_BLOCK_VALUES 16384u
#define E8HUF_LANE_VALUES 256u
#define E8HUF_LANES (E8HUF_BLOCK_VALUES / E8HUF_LANE_VALUES)
#define E8HUF_HDR_BYTES 128u
#define E8HUF_BLOCK_REC_BYTES (8u + 2u * E8HUF_LANES)
/* two-level table: level 1 (256 entries), then at most 17 level-2 tables:
 * with codes assigned shortest first, the codes longer than 8 bits are the
 * numerically last ones, so they cover one contiguous range of the 16-bit
 * code space of at most 32 * 2^7 values, which spans at most 17 8-bit
 * prefixes */
#define E8HUF_LUT_MAX (256 * 18)

/* device status bits, OR-ed into *d_status by the decode kernel */
#define E8HUF_DEV_HEADER 1u    /* header does not match the call or the blob */
#define E8HUF_DEV_INDEX 4u     /* a block record is inconsistent */
#define E8HUF_DEV_CODE 8u      /* the decode met bits no code covers */
#define E8HUF_DEV_LANE_END 16u /* a lane chunk's codes did not end where its index says */

/*
 * e8huf_build_table -- the two-level decode table of ECF8 page section 2.1
 * from codelen[32] (entries at and past 2^exp_bits must be 0).
 * lut[0..255] is level 1, indexed by the first 8 bits of the bit window:
 *   (symbol << 8) | length for a code of length 1..8 that prefixes the index;
 *   (t << 8) | 0x20 when every code under the index is longer than 8 bits
 *   (a link to level-2 table t); 0 when no code covers the index.
 * lut[256 (1 + t) ..] is level-2 table t, indexed by the next 8 bits:
 *   (symbol << 8) | length (9..16), or 0. Tables are numbered in the order of
 *   their 8-bit prefixes.
 * The table is checked like the page's "reject corrupt tables" rule of the K3
 * codec: all-zero (K3HUF_E_EMPTY), a length above 16 (K3HUF_E_BADLEN),
 * Kraft sum above 2^16 (K3HUF_E_OVERSUB). exp_bits must be 4 or 5, and nonzero
 * lengths past 2^exp_bits are K3HUF_E_ARG.
 * lut: host array of E8HUF_LUT_MAX entries; *n_entries receives the entries
 * used (256 * (1 + tables)). Host only, no allocation, thread-safe. On error
 * lut[] is left zeroed.
 */
int e8huf_build_table(const uint8_t codelen[32], int exp_bits, uint16_t* lut, int* n_entries);

typedef struct e8huf_info {
    uint64_t n_values;
    uint64_t n_bits;
    uint64_t container_bytes;
    uint32_t n_blocks;
    uint32_t exp_bits;
    uint8_t codelen[32];
} e8huf_info;

/*
 * e8huf_layer_info -- parse and check an E8HF header held in host memory
 * (ECF8 page, section 2.1: the layer's table is carried as its code lengths,
 * from which e8huf_build_table makes the decode table).
 * h_blob/h_bytes: at least E8HUF_HDR_BYTES bytes, host, caller-owned.
 * Errors: K3HUF_E_ARG (null, short), K3HUF_E_FORMAT (a field off the format;
 * *out is left unchanged).
 */
int e8huf_layer_info(const void* h_blob, size_t h_bytes, e8huf_info* out);

/*
 * e8huf_encode_bound / e8huf_encode -- host packer: the container for n FP8
 * bytes h_x (E4M3 when exp_bits is 4, E5M2 when 5), byte for byte what the
 * format above prescribes: exponent histogram of the whole tensor, Huffman
 * depths, the smoothing c -> c / 2 + 1 while a code is longer than 16 bits (a
 * lone exponent value gets length 1), shortest-first canonical codes, the
 * block records, the bitstream and the nibble plane (ECF8 page, section 2.1).
 * h_out: host buffer of cap >= e8huf_encode_bound(n). n_threads <= 0 picks
 * the core count. Returns the container size, or K3HUF_E_ARG.
 */
int64_t e8huf_encode_bound(uint64_t n);
int64_t e8huf_encode(const void* h_x, uint64_t n, int exp_bits, void* h_out, uint64_t cap, int n_threads);

/*
 * e8huf_decode -- decode an E8HF container on the GPU (ECF8 page, section
 * 2.2: each lane starts at the bit offset its block record gives it, decodes
 * into LDS, and the wave writes the output out coalesced).
 * d_blob: device, 16-byte aligned, blob_bytes (the whole container).
 * d_lut, lut_entries: the table from e8huf_build_table for this blob's
 *   codelen, in device memory (lut_entries u16 values, 2-byte aligned).
 * d_out: device, 16-byte aligned, n_values bytes: receives the FP8 bytes.
 * stream: queued there; returns without synchronizing or allocating.
 * d_status: device u32 (nullable): E8HUF_DEV_* bits for a header that does
 *   not match the call or the blob, inconsistent block records, bits no code
 *   covers, or lane chunks whose codes end off their index; blocks with bad
 *   records are left unwritten; no read leaves [d_blob, d_blob + blob_bytes).
 * Any number of decodes may run at once on any streams (the kernel keeps no
 * state between launches).
 * Returns K3HUF_OK once queued, K3HUF_E_ARG (null or misaligned pointers,
 * n_values 0 or above 2^40, blob_bytes below a header or at least 2^44,
 * lut_entries not 256 * (1 + t) for t in 0..17), K3HUF_E_HIP (launch failed).
 */
int e8huf_decode(const void* d_blob, size_t blob_bytes, const uint16_t* d_lut, int lut_entries,
                 void* d_out, uint64_t n_values, void* stream, uint32_t* d_status);

/* output kinds of e8huf_decode_widen */
#define E8HUF_OUT_BF16 1   /* bfloat16: 8 exponent, 7 mantissa bits */
#define E8HUF_OUT_F16 2    /* IEEE half: 5 exponent, 10 mantissa bits */

/*
 * e8huf_decode_widen -- e8huf_decode whose output is 16-bit floats instead of
 * FP8 bytes (ECF8 page, section 2.2: the page's decoder writes its values out
 * as 16-bit floats). Element i of d_out is the FP8 value of the tensor's byte
 * i (E4M3 or E5M2 as the header's exp_bits says; section 1.2), multiplied by
 * scale in single precision and rounded to the nearest out_kind value, ties
 * to even, overflow to infinity; a NaN (an E4M3 S.1111.111 byte, an E5M2 NaN,
 * or a product such as 0 * infinity) gives a NaN whose payload is not
 * specified. scale = 1 widens exactly: every E4M3 and E5M2 value is a
 * bfloat16 value, and every E5M2 value a half value.
 * d_out: device, 16-byte aligned, 2 * n_values bytes. out_kind:
 * E8HUF_OUT_BF16 or E8HUF_OUT_F16 (anything else is K3HUF_E_ARG). Every other
 * argument, the status bits, the errors and the concurrency rules are
 * e8huf_decode's.
 */
int e8huf_decode_widen(const void* d_blob, size_t blob_bytes, const uint16_t* d_lut, int lut_entries,
                       void* d_out, uint64_t n_values, int out_kind, float scale, void* stream,
                       uint32_t* d_status);

#ifdef __cplusplus
}
#endif

#endif /* E8HUF_H */
