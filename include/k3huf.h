/*
 * k3huf.h -- C ABI of the MI355X (gfx950) decoder for bf16 layers whose high
 * (sign + exponent) byte plane is coded with a 12-bit length-limited canonical
 * Huffman code.
 *
 * Sources. "K3 page" is the page "Kimi K3 纯 CPU 推理中的无损 Trunk 压缩：一次被解码
 * 速度判死刑的 Huffman 压缩实验" (yfxerp.com/news/153994). "ECF8 page" is the
 * pwwt.cn page on exponent-concentration FP8 (pwwt.cn/news/2030120). "K3
 * TUNING page" is zwxr.cn/news/188695.
 *
 * All functions are plain C: pointers and sizes only. A "stream" argument is
 * a hipStream_t passed as void* (NULL = the null stream). Functions return
 * K3HUF_OK (0) or a negative K3HUF_E_* code and never throw.
 *
 * ---------------------------------------------------------------------------
 * Container ("layer blob") layout, all integers little-endian.
 * K3 page, "what was implemented": [layer header holding codelen[256]], then
 * per stripe [stripe header][odd-plane Huffman bitstream][even plane raw].
 * K3 page, "key design points": 64 MiB of raw layer bytes per stripe; the odd
 * offsets of a little-endian bf16 layer (high bytes) are coded, the even
 * offsets (mantissa bytes) are copied raw; code length at most 12.
 * The subblock/lane index is an addition for parallel decoding (after the
 * per-thread bit offsets of the ECF8 page, section 2.1), counted in the size.
 *
 *   layer header (K3HUF_HDR_BYTES = 304):
 *     0   char[4] magic "K3HF"         4  u16 version = 1
 *     6   u16 maxlen = 12               8  u32 stripe_bytes = 2^26
 *     12  u32 subblock_bytes = 256 * lane_syms (2^16, or 2^14)
 *     16  u32 lane_syms = 256, or 64 (K3HUF_LANE_SYMS_SHORT: the layout for
 *         small layers, whose decode time is one lane chunk's chain of
 *         dependent table lookups; a subblock always holds 128 lane chunks)
 *     20  u32 n_stripes = ceil(raw_bytes / 2^26)
 *     24  u64 raw_bytes (even, > 0)     32 u32 n_subblocks (total)
 *     36  u32 reserved = 0              40 u64 container_bytes
 *     48  u8  codelen[256]
 *   304   u64 stripe_off[n_stripes]: byte offset of each stripe record from
 *         the blob start, a multiple of 256; zero pad to 256.
 *   stripe record (at stripe_off[s]):
 *     0 u32 raw_bytes   4 u32 n_syms = raw_bytes / 2   8 u32 n_bits
 *     12 u32 bit_bytes = ceil(n_bits / 8) rounded up to 16
 *     16 u32 first_subblock = s * 2^26 / subblock_bytes
 *     20 u32 n_subblocks = ceil(n_syms / (128 * lane_syms))
 *     24 u32 bits_off   28 u32 even_off  (both from the record start,
 *          multiples of 256; decoders require only 16-byte alignment)
 *     32 subblock records, K3HUF_SUBBLOCK_REC_BYTES = 264 each:
 *          u32 start_bit (stripe-relative bit index of the subblock's first code)
 *          u32 n_syms    (128 * lane_syms, or fewer in the stripe's last subblock)
 *          u16 lane_bits[128] (code bits of each lane chunk of lane_syms
 *                             symbols; 0 if empty)
 *        zero pad to 256
 *     bits_off: the stripe's codes, most-significant bit first (K3 page,
 *        "decode loop": the stream head sits at the top of the bit window),
 *        zero padded to bit_bytes, then to a multiple of 256
 *     even_off: the even-offset bytes of the stripe (n_syms), zero padded to 256
 *   The 256-byte boundaries keep each plane on whole cache lines, so the
 *   GPU's line-sized reads of a lane chunk's even bytes touch one line each.
 *   Stripe s covers raw bytes [s * 2^26, min((s + 1) * 2^26, raw_bytes)).
 *   Global subblock k covers raw bytes [k * subblock_bytes, min((k + 1) *
 *   subblock_bytes, raw_bytes)).
 */
#ifndef K3HUF_H
#define K3HUF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define K3HUF_MAXLEN 12
#define K3HUF_LUT_ENTRIES 4096
#define K3HUF_STRIPE_BYTES (1u << 26)
#define K3HUF_SUBBLOCK_BYTES (1u << 16)
#define K3HUF_SUBBLOCK_SYMS (K3HUF_SUBBLOCK_BYTES / 2)
#define K3HUF_LANE_SYMS 256u
#define K3HUF_LANE_SYMS_SHORT 64u
#define K3HUF_LANES (K3HUF_SUBBLOCK_SYMS / K3HUF_LANE_SYMS)
#define K3HUF_HDR_BYTES 304u
#define K3HUF_STRIPE_HDR_BYTES 32u
#define K3HUF_SUBBLOCK_REC_BYTES (8u + 2u * K3HUF_LANES)

/* return codes */
#define K3HUF_OK 0
#define K3HUF_E_ARG (-1)      /* bad argument (null, size, alignment) */
#define K3HUF_E_EMPTY (-2)    /* code table codes no symbol */
#define K3HUF_E_OVERSUB (-3)  /* Kraft sum over-fills the 12-bit code space */
#define K3HUF_E_BADLEN (-4)   /* a code length above 12 */
#define K3HUF_E_OVERLAP (-5)  /* canonical codes are not prefix-free */
#define K3HUF_E_FORMAT (-6)   /* container header or stripe record malformed */
#define K3HUF_E_CORRUPT (-7)  /* data inconsistent with its index or table */
#define K3HUF_E_HIP (-8)      /* a HIP runtime call failed */

/* device status bits, OR-ed into *d_status by the decode kernel */
#define K3HUF_DEV_HEADER 1u   /* layer header does not match the call */
#define K3HUF_DEV_STRIPE 2u   /* a stripe record is out of bounds or inconsistent */
#define K3HUF_DEV_INDEX 4u    /* a subblock record or lane bit count is inconsistent */
#define K3HUF_DEV_CODE 8u     /* the decode hit an unused lookup-table slot */
#define K3HUF_DEV_LANE_END 16u /* a lane chunk's codes did not end where its index says */

/*
 * k3huf_build_table -- 4096-entry decode table from codelen[256].
 * K3 page, "key design points": a table of 1 << 12 entries, each entry packs
 * (symbol << 4) | code_length, so one lookup yields both. K3 page, "canonical
 * code assignment and Kraft check": the Kraft sum sum_l count[l] << (12 - l)
 * must fill the 12-bit space exactly or under-fill it (over-full or empty =
 * corrupt); codes are assigned longest length first with first[l] = code;
 * code = (code + count[l]) >> 1, symbols in ascending order within a length,
 * and each code is expanded over all 12-bit indices it prefixes.
 * Entry 0 marks an index no code covers (possible only for under-full tables).
 * Host memory in, host memory out; pure, no allocation, thread-safe.
 * Errors: K3HUF_E_ARG (null), K3HUF_E_BADLEN, K3HUF_E_EMPTY, K3HUF_E_OVERSUB,
 * K3HUF_E_OVERLAP (a slot would be written twice: an under-full table whose
 * canonical codes are not prefix-free). On error lut[] is left zeroed.
 */
int k3huf_build_table(const uint8_t codelen[256], uint16_t lut[4096]);

typedef struct k3huf_info {
    uint64_t raw_bytes;       /* decoded size */
    uint64_t container_bytes; /* blob size recorded in the header */
    uint32_t n_stripes;
    uint32_t n_subblocks;
    uint8_t codelen[256];
    uint32_t lane_syms;       /* 256 or 64 */
} k3huf_info;

/*
 * k3huf_layer_info -- parse and check a layer header held in host memory.
 * K3 page, "what was implemented": a layer starts with a header that holds
 * its codelen[256] (one code table per layer), followed by its stripes; this
 * reads that header (plus the geometry fields the container adds) so the
 * caller can build the layer's table and size its output.
 * h_blob/h_bytes: at least the first K3HUF_HDR_BYTES bytes of a blob (host
 *   memory, caller-owned, only read). out: caller-owned, filled on success.
 * Checks magic, version, geometry constants, raw size and stripe count; the
 * stripe records are not read.
 * Errors: K3HUF_E_ARG (null pointer, h_bytes < K3HUF_HDR_BYTES),
 * K3HUF_E_FORMAT (a field off the format; *out is left unchanged).
 */
int k3huf_layer_info(const void* h_blob, size_t h_bytes, k3huf_info* out);

/*
 * k3huf_decode_layer -- decode one layer blob on the GPU.
 * d_blob: device pointer, 16-byte aligned, blob_bytes long (the whole blob).
 * d_lut: device pointer to the 4096 u16 entries k3huf_build_table made from
 *   this blob's codelen[256] (the caller uploads it once per layer).
 * d_out: device pointer, 16-byte aligned, out_bytes = the blob's raw_bytes;
 *   receives the bf16 layer bytes.
 * stream: hipStream_t (as void*) the work is queued on; the call returns
 *   after queuing, without synchronizing and without allocating.
 * d_status: device u32 (nullable). The kernel ORs K3HUF_DEV_* bits into it
 *   when it meets a malformed header, stripe or index, an unused table slot,
 *   or a lane whose codes end off its index; the caller clears it beforehand
 *   and reads it after the stream synchronizes. Subblocks with bad records
 *   are left unwritten; no read ever leaves [d_blob, d_blob + blob_bytes).
 * Both lane-chunk layouts are decoded (the kernel reads lane_syms from the
 * header).
 * Returns K3HUF_OK once queued, K3HUF_E_ARG for bad sizes or alignment (also
 * for blob_bytes >= 2^36: the kernel keeps stripe offsets in 16-byte units;
 * and for out_bytes > 2 * blob_bytes, which no blob of this format allows:
 * its even plane alone is out_bytes / 2),
 * K3HUF_E_HIP if the launch fails. Decoding follows the K3 page's "decode
 * loop" (MSB-first bit window, one table lookup per symbol) and "key design
 * points" (even plane interleaved back at even offsets).
 * Concurrency: any number of decodes may be queued and may run at the same
 * time, on any streams and from graph replays. A layer of more than five
 * rounds of work units (above about 290 MB of output on MI355X) launched on
 * one of the first 256 distinct streams of a device hands out its later
 * units through counters of its stream's own (per-device, process-lifetime)
 * slot. Every other launch hands each workgroup's share of units to its
 * waves from a counter in the workgroup's own LDS, which shares nothing: for
 * smaller layers it is as fast or faster, for larger ones slower (about
 * 1.05 times the time on the trunk layer). That covers launches on later
 * streams, launches on hipStreamPerThread (one handle for a different stream
 * in each host thread) and launches made while the stream is being captured
 * into a graph (and so all of a graph's replays). A slot belongs to a stream
 * handle's value: a stream must not be destroyed while a decode on it is
 * still pending if a new stream could then be created at the same address
 * and decode at the same time.
 */
int k3huf_decode_layer(const void* d_blob, size_t blob_bytes, const uint16_t* d_lut,
                       void* d_out, size_t out_bytes, void* stream, uint32_t* d_status);

/*
 * k3huf_decode_ring -- decode layers 0..n_layers-1 in order into a ring of
 * device slots (K3 TUNING page, section 2: a trunk ring whose default of two
 * slots lets one layer be consumed while the next one is produced; K3 page,
 * "background": layers are visited in the fixed order 0..92).
 * Layer k goes to slot k % n_slots on stream k % n_streams, after the previous
 * user of that slot has released it (event wait); then cb (nullable) is called
 * to queue the consumer's work on that stream, and the slot is released behind
 * it. All queued asynchronously; the call returns without synchronizing.
 * layers[k]: device blob, its size, its device LUT, its raw size (<= slot_bytes).
 * d_slots[n_slots], streams[n_streams] (hipStream_t as void*): caller-owned.
 * d_status: as for k3huf_decode_layer (shared by all layers).
 * Errors: K3HUF_E_ARG, K3HUF_E_HIP.
 */
typedef struct k3huf_ring_layer {
    const void* d_blob;
    size_t blob_bytes;
    const uint16_t* d_lut;
    size_t raw_bytes;
} k3huf_ring_layer;

typedef void (*k3huf_ring_cb)(int layer, void* d_slot, size_t raw_bytes, void* stream, void* user);

int k3huf_decode_ring(const k3huf_ring_layer* layers, int n_layers, void* const* d_slots,
                      int n_slots, size_t slot_bytes, void* const* streams, int n_streams,
                      k3huf_ring_cb cb, void* user, uint32_t* d_status);

/*
 * k3huf_decode_ring_host -- the layer ring fed from host memory: each layer's
 * container is copied over PCIe into a device stage buffer on copy_stream,
 * then decoded from there into the slot ring as k3huf_decode_ring does.
 * K3 page, "background" and "the measurement that shelved it": every token
 * streams the trunk from storage in the fixed layer order, and the decoder
 * must keep up with the feed; K3 TUNING page, section 5 ("--trunk-ring N"):
 * of the ring's slots one holds the layer in use and the others are reads in
 * flight, so extra stage buffers let copies run ahead of decoding.
 * Layer k is copied into stage k % n_stage once the decode that last read
 * that stage is done (event wait on copy_stream), and decoded on stream
 * k % n_streams into slot k % n_slots once the copy is done and the slot's
 * previous consumer released it; cb (nullable) then queues the consumer, and
 * the slot is released behind it. Everything is queued asynchronously; the
 * call returns without synchronizing.
 * layers[k]: h_blob, the container in host memory (pinned memory, e.g. from
 *   hipHostMalloc, for copies that overlap decoding; pageable memory works
 *   but its copies do not overlap), its size (<= stage_bytes), its device LUT
 *   (from k3huf_build_table), its raw size (<= slot_bytes). The host blob
 *   must stay unchanged until its copy has run.
 * d_stage[n_stage]: device buffers, 16-byte aligned, stage_bytes each.
 * d_slots[n_slots], streams[n_streams], copy_stream (hipStream_t as void*):
 *   caller-owned; copy_stream should differ from the decode streams so
 *   copies overlap decoding.
 * d_status: as for k3huf_decode_layer (shared by all layers).
 * Errors: K3HUF_E_ARG (nulls, counts < 1, a layer larger than a stage or
 * slot, a misaligned stage), K3HUF_E_HIP (work queued before the failing call
 * still runs).
 */
typedef struct k3huf_host_layer {
    const void* h_blob;
    size_t blob_bytes;
    const uint16_t* d_lut;
    size_t raw_bytes;
} k3huf_host_layer;

int k3huf_decode_ring_host(const k3huf_host_layer* layers, int n_layers, void* const* d_stage,
                           int n_stage, size_t stage_bytes, void* const* d_slots, int n_slots,
                           size_t slot_bytes, void* copy_stream, void* const* streams,
                           int n_streams, k3huf_ring_cb cb, void* user, uint32_t* d_status);

/*
 * k3huf_encode_bound -- container size upper bound for raw_bytes of layer data.
 * k3huf_encode_layer -- host packer: one histogram and codelen[256] over the
 * whole layer's odd bytes (K3 page, "what was implemented"), Huffman depths
 * limited to 12 bits (K3 page, "canonical code assignment and Kraft check"),
 * longest-first canonical codes, stripes and the subblock/lane index.
 * h_raw: host bf16 layer bytes (raw_bytes even, > 0). h_out: host buffer of
 * cap >= k3huf_encode_bound(raw_bytes). n_threads <= 0 picks the core count.
 * Returns the container size, or K3HUF_E_ARG. Lane chunks of 256 symbols.
 * k3huf_encode_bound_lanes / k3huf_encode_layer_lanes -- the same for lane
 * chunks of lane_syms symbols, 256 or K3HUF_LANE_SYMS_SHORT (64); any other
 * value is K3HUF_E_ARG. The code, bitstream and even plane do not depend on
 * it, only the index does (its records cover 128 * lane_syms symbols each).
 */
int64_t k3huf_encode_bound(uint64_t raw_bytes);
int64_t k3huf_encode_layer(const void* h_raw, uint64_t raw_bytes, void* h_out, uint64_t cap,
                           int n_threads);
int64_t k3huf_encode_bound_lanes(uint64_t raw_bytes, uint32_t lane_syms);
/* The lane-chunk length that decodes faster on MI355X for a layer of
 * raw_bytes: 64 up to K3HUF_SHORT_LANES_MAX_RAW (16 MiB), where a decode is
 * one round of work units and its time one lane's chain of dependent table
 * lookups (measured on trunk-recipe layers: 8.0 against 14.5 us at 64 KiB,
 * 8.9 against 15.3 us at 4 MiB, 13.6 against 16.1 us at 16 MiB), else 256
 * (19.5 against 17.7 us at 32 MiB, 98 against 83 us at 256 MiB). */
#define K3HUF_SHORT_LANES_MAX_RAW (16ull << 20)
uint32_t k3huf_lane_syms_for(uint64_t raw_bytes);
int64_t k3huf_encode_layer_lanes(const void* h_raw, uint64_t raw_bytes, uint32_t lane_syms, void* h_out,
                                 uint64_t cap, int n_threads);

/*
 * k3huf_encode_work_bytes -- device work-buffer size k3huf_encode_layer_dev
 *   needs for raw_bytes of layer data (or K3HUF_E_ARG for an odd or zero size).
 * k3huf_encode_layer_dev -- the packer on the GPU: the bf16 layer in device
 * memory becomes, in device memory, the container k3huf_encode_layer writes
 * for the same bytes (byte for byte). K3 page, "what was implemented": one
 * histogram and codelen[256] for the whole layer's odd bytes, MSB-first
 * Huffman bitstream per stripe, even plane raw; "canonical code assignment
 * and Kraft check": depths limited to 12 bits, longest-first canonical codes.
 * The histogram, the lane-chunk bit counts, the subblock index (each unit's
 * start bit from the units before it in its stripe), the bit packing and the
 * even-plane copy run on the GPU; the code lengths and the layout are
 * computed on the host from the GPU's 256-bin histograms.
 * d_raw: device, 16-byte aligned, raw_bytes (even, > 0). d_out: device,
 *   16-byte aligned, cap >= k3huf_encode_bound(raw_bytes). d_work: device,
 *   16-byte aligned, work_bytes >= k3huf_encode_work_bytes(raw_bytes); its
 *   contents are scratch. All buffers are caller-owned.
 * stream: hipStream_t as void*. The call is synchronous: it waits for the
 *   histograms, then queues the rest and waits for it, so the container is
 *   complete on return. It allocates no device memory. Its host round trips
 *   go through pinned host buffers (about 2.1 KB per stripe) leased from a
 *   process-wide pool that keeps them until the process ends.
 * Returns the container size, K3HUF_E_ARG (bad sizes, alignment or
 * capacity), K3HUF_E_HIP (a HIP call failed, or a packing wave waited too
 * long for the start bit of its unit), or K3HUF_E_CORRUPT if d_raw changed
 * during the call (the GPU's bit counts disagree with its histograms; no
 * bitstream word is then written past a stripe's bits).
 */
int64_t k3huf_encode_work_bytes(uint64_t raw_bytes);
int64_t k3huf_encode_layer_dev(const void* d_raw, uint64_t raw_bytes, void* d_out, uint64_t cap,
                               void* d_work, uint64_t work_bytes, void* stream);
/* The same for lane chunks of lane_syms symbols (256, or K3HUF_LANE_SYMS_SHORT
 * = 64; any other value is K3HUF_E_ARG): the container
 * k3huf_encode_layer_lanes writes, with cap >=
 * k3huf_encode_bound_lanes(raw_bytes, lane_syms) and work_bytes >=
 * k3huf_encode_work_bytes_lanes(raw_bytes, lane_syms) (the 64-symbol layout
 * has four times as many packing units, so its work buffer is larger). */
int64_t k3huf_encode_work_bytes_lanes(uint64_t raw_bytes, uint32_t lane_syms);
int64_t k3huf_encode_layer_dev_lanes(const void* d_raw, uint64_t raw_bytes, uint32_t lane_syms, void* d_out,
                                     uint64_t cap, void* d_work, uint64_t work_bytes, void* stream);

/*
 * k3huf_encode_layer_dev_static -- k3huf_encode_layer_dev without any
 * allocation, for callers that cannot allocate device or pinned memory (code
 * that must not call hipMalloc or hipHostMalloc, harnesses that forbid it).
 * Same result, byte for byte, as k3huf_encode_layer_dev on the same layer.
 * Its work buffer is a library-owned device array of about 3.3 MB (one copy
 * per GPU, held until the process ends) and its host staging is a
 * library-owned host array (about 132 KB); so layers are limited to
 * raw_bytes <= K3HUF_STATIC_MAX_RAW (4 GiB), and the host round trips are
 * copies from pageable memory. The arrays keep the last call's contents; each
 * call clears what must start at zero with a kernel. Calls are serialized
 * inside the library (a second caller waits for the first to return), and
 * each call is synchronous, so calls never overlap on a GPU.
 * d_raw, raw_bytes, d_out, cap, stream: as for k3huf_encode_layer_dev.
 * Returns the container size, K3HUF_E_ARG (as for k3huf_encode_layer_dev,
 * and for raw_bytes above K3HUF_STATIC_MAX_RAW), K3HUF_E_HIP, or
 * K3HUF_E_CORRUPT (d_raw changed during the call).
 */
#define K3HUF_STATIC_MAX_RAW (1ull << 32)
int64_t k3huf_encode_layer_dev_static(const void* d_raw, uint64_t raw_bytes, void* d_out, uint64_t cap,
                                      void* stream);

/*
 * k3huf_stream_ref -- measurement reference, not a decode step: a plain
 * streaming kernel that reads in_bytes from d_in and writes out_bytes to
 * d_out in 16-byte units (output unit u = input unit u while the input
 * lasts, then {u mod 2^32, 0, 0, 0}; input units past the output are only
 * read). Given a decode launch's container and output sizes it moves the same
 * HBM bytes with nothing in between, so a benchmark can report the rate a
 * simple kernel reaches for that traffic beside the decode's own.
 * d_in (nullable when in_bytes is 0), d_out: device, 16-byte aligned; both
 * sizes multiples of 16, out_bytes > 0. grid: workgroups of 256 threads,
 * 1..2^20. nontemporal != 0 streams the stores past the caches. Queued on
 * `stream`; returns K3HUF_OK, K3HUF_E_ARG or K3HUF_E_HIP.
 */
int k3huf_stream_ref(const void* d_in, uint64_t in_bytes, void* d_out, uint64_t out_bytes, int grid,
                     int nontemporal, void* stream);

/* Static text for a return code. */
const char* k3huf_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* K3HUF_H */
