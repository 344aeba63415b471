// gfx950 encoder of the k3huf library: packs a bf16 layer held in device
// memory into the container of include/k3huf.h, byte for byte what the host
// packer writes.
//
// What is computed (K3 page = "Kimi K3 纯 CPU 推理中的无损 Trunk 压缩…",
// yfxerp.com/news/153994): one histogram and codelen[256] for the whole
// layer's odd (high) bytes ("what was implemented"), Huffman depths limited to
// 12 bits and longest-first canonical codes ("canonical code assignment and
// Kraft check"), 64 MiB stripes whose odd bytes become an MSB-first bitstream
// and whose even bytes are copied raw ("key design points"), plus the
// subblock/lane index. The code lengths and the layout are computed on the
// host from the GPU's histograms (they are 256-entry problems); the byte work
// runs in five kernels:
//   enc_hist   per-stripe histograms of the odd bytes;
//   enc_count  code bits of every 256-symbol lane chunk, and of every
//              subblock (128 chunks);
//   enc_scan   per stripe: subblock start bits (the subblock records) and
//              the stripe record;
//   enc_pack   one wave per half subblock (64 lane chunks, one per lane): the
//              lanes' start bits (a wave prefix sum), their lane bit counts,
//              their codes packed into a per-wave LDS buffer (words two lanes
//              share are OR-ed), then copied out with whole-wave stores, and
//              the even bytes; a unit's first and last words, which a
//              neighbouring unit may share, are set aside;
//   enc_edges  one thread per unit: the words units share, from both sides.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "k3huf.h"
#include "k3huf_internal.h"

namespace {

using k3huf_detail::pad256;
using k3huf_detail::StripeGeom;

constexpr uint32_t kChunksPerStripe = (K3HUF_STRIPE_BYTES / 2) / K3HUF_LANE_SYMS;   // 131072
constexpr int kHistThreads = 1024;
constexpr int kHistCopies = 32;        // sub-histograms per block (lane mod 32)
constexpr int kScanThreads = 1024;     // = subblocks per stripe
constexpr int kChunkThreads = 256;
constexpr int kPackWaves = 4;       // waves (units) per packing block
constexpr int kPackWords = 2048;       // per-wave LDS bit buffer (8 KiB)
constexpr uint32_t kUnitChunks = 64;   // lane chunks per packing unit
constexpr uint32_t kUnitsPerStripe = kChunksPerStripe / kUnitChunks;
static_assert(kScanThreads == K3HUF_STRIPE_BYTES / K3HUF_SUBBLOCK_BYTES, "one scan thread per subblock");

// stripe geometry as the kernels read it
struct StripeDev {
    uint64_t raw0, off;
    uint32_t raw, n, nsb, nbits, bit_bytes, bits_off, even_off, pad;
};

struct CodeTable {
    uint32_t e[256];   // (length << 16) | code, 0 for symbols without a code
};

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

struct WorkLayout {
    uint64_t hist, geom, chunks, subblocks, edges, status, total;
};

// Per packing unit: its first and last bitstream words when another unit
// shares them (0 otherwise), and its start and end bits.
struct UnitEdges {
    uint32_t first, last, b0, b1;
};

// work buffer: per-stripe histograms (u64), stripe geometry, lane-chunk bit
// counts (u32), subblock bit counts then start bits (u32), unit edges, a
// status word
WorkLayout work_layout(uint64_t raw_bytes) {
    const uint64_t ns = k3huf_detail::stripes_for(raw_bytes);
    const uint64_t n_chunks = (raw_bytes / 2 + K3HUF_LANE_SYMS - 1) / K3HUF_LANE_SYMS;
    const uint64_t n_sub = (raw_bytes + K3HUF_SUBBLOCK_BYTES - 1) / K3HUF_SUBBLOCK_BYTES;
    const uint64_t n_units = (n_chunks + 63) / 64;
    WorkLayout w;
    w.hist = 0;
    w.geom = align256(w.hist + 256 * 8 * ns);
    w.chunks = align256(w.geom + sizeof(StripeDev) * ns);
    w.subblocks = align256(w.chunks + 4 * n_chunks);
    w.edges = align256(w.subblocks + 4 * n_sub);
    w.status = align256(w.edges + sizeof(UnitEdges) * n_units);
    w.total = w.status + 256;
    return w;
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

__device__ __forceinline__ uint32_t bswap32(uint32_t x) {
    return __builtin_amdgcn_perm(0u, x, 0x00010203u);
}

// Zero the words [0, n) of p (16-byte stores, grid-stride).
__global__ void enc_fill_zero(uint4* p, uint64_t n16) {
    for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
         i += uint64_t(gridDim.x) * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Zero what enc_scan and enc_pack do not overwrite whole: stripe s's record
// area and bitstream [off, off + even_off) (the stripe header, subblock
// records and codes are written later; codes are OR-ed into it), and the
// padding after its even plane. Grid (blocks, stripes).
__global__ void enc_zero_stripes(uint8_t* out, const StripeDev* g) {
    const StripeDev G = g[blockIdx.y];
    uint4* p = reinterpret_cast<uint4*>(out + G.off);
    const uint32_t n16 = G.even_off / 16;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
    if (blockIdx.x == 0) {
        const uint64_t e0 = G.off + G.even_off + G.n, e1 = G.off + ((uint64_t(G.even_off) + G.n + 255) & ~255ull);
        for (uint64_t i = e0 + threadIdx.x; i < e1; i += blockDim.x) out[i] = 0;
    }
}

// Per-stripe histograms of the odd bytes: grid (blocks per stripe, stripes),
// sized so that the whole grid is resident at once (a partial last round of
// blocks left most CUs idle: 64 blocks per stripe took 7% longer than 28). Each block counts a slice of its stripe into 32 interleaved LDS
// sub-histograms (bin v, copy c at v * 32 + c: lanes adding the same symbol
// hit different banks), then adds its counts into hist[s * 256 + v].
__global__ __launch_bounds__(kHistThreads) void enc_hist(const uint8_t* raw, uint64_t raw_bytes,
                                                         unsigned long long* hist) {
    __shared__ uint32_t h[256 * kHistCopies];
    for (int i = threadIdx.x; i < 256 * kHistCopies; i += kHistThreads) h[i] = 0;
    __syncthreads();
    const uint32_t s = blockIdx.y;
    const uint64_t base = uint64_t(s) * K3HUF_STRIPE_BYTES;
    const uint64_t len = min(uint64_t(K3HUF_STRIPE_BYTES), raw_bytes - base);
    const uint64_t n16 = len / 16;
    const uint32_t c = threadIdx.x & (kHistCopies - 1);
    const uint4* p = reinterpret_cast<const uint4*>(raw + base);
    for (uint64_t i = uint64_t(blockIdx.x) * kHistThreads + threadIdx.x; i < n16;
         i += uint64_t(gridDim.x) * kHistThreads) {
        const uint4 v = p[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            atomicAdd(&h[((w[k] >> 8) & 0xFFu) * kHistCopies + c], 1u);
            atomicAdd(&h[(w[k] >> 24) * kHistCopies + c], 1u);
        }
    }
    // the stripe's last (len mod 16) bytes: whole symbols, len is even
    if (blockIdx.x == 0) {
        const uint64_t r0 = n16 * 16;
        for (uint64_t i = r0 + 2 * threadIdx.x; i < len; i += 2 * kHistThreads)
            atomicAdd(&h[uint32_t(raw[base + i + 1]) * kHistCopies + c], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 256) {
        uint32_t t = 0;
        for (int k = 0; k < kHistCopies; ++k) t += h[threadIdx.x * kHistCopies + k];
        if (t) atomicAdd(&hist[uint64_t(s) * 256 + threadIdx.x], (unsigned long long)t);
    }
}

// Code bits of lane chunk c (symbols [256 c, min(256 c + 256, n))). A block's
// 256 chunks are two whole subblocks (stripes hold whole blocks); their sums
// go to sb_bits. Each wave counts 64 chunks (32 KiB of raw bytes) with
// whole-wave loads: load i covers chunks 2i (lanes 0-31) and 2i + 1 (lanes
// 32-63); each half's sum is reduced across its lanes and kept by the lane
// that owns the chunk. The layer's last wave, whose chunks may be partial or
// missing, reads its own chunk per lane instead.
__global__ __launch_bounds__(kChunkThreads) void enc_count(const uint8_t* raw, uint64_t raw_bytes,
                                                           uint64_t n_chunks, CodeTable ct,
                                                           uint32_t* chunk, uint32_t* sb_bits) {
    __shared__ uint8_t len[256];
    __shared__ uint32_t wsum[kChunkThreads / 64];
    if (threadIdx.x < 256) len[threadIdx.x] = uint8_t(ct.e[threadIdx.x] >> 16);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const uint64_t c0 = uint64_t(blockIdx.x) * kChunkThreads + (threadIdx.x & ~63u);   // wave's first chunk
    const uint64_t c = c0 + lane;
    uint32_t bits = 0;
    if ((c0 + 64) * 2 * K3HUF_LANE_SYMS <= raw_bytes) {
        const uint4* p = reinterpret_cast<const uint4*>(raw + c0 * 2 * K3HUF_LANE_SYMS);
#pragma unroll 4
        for (int i = 0; i < 32; ++i) {
            const uint4 v = p[i * 64 + lane];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            uint32_t b = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) b += len[(w[k] >> 8) & 0xFFu] + len[w[k] >> 24];
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) b += __shfl_xor(b, o);
            const uint32_t lo = __builtin_amdgcn_readlane(b, 0), hi = __builtin_amdgcn_readlane(b, 32);
            bits = lane == 2 * i ? lo : (lane == 2 * i + 1 ? hi : bits);
        }
        chunk[c] = bits;
    } else if (c < n_chunks) {
        const uint64_t b0 = c * 2 * K3HUF_LANE_SYMS;
        const uint64_t b1 = min(b0 + 2 * K3HUF_LANE_SYMS, raw_bytes);
        for (uint64_t i = b0; i < b1; i += 2) bits += len[raw[i + 1]];
        chunk[c] = bits;
    }
    const uint32_t ws = wave_sum(bits);
    if (lane == 0) wsum[threadIdx.x >> 6] = ws;
    __syncthreads();
    if (threadIdx.x < 2) {
        const uint64_t sb = uint64_t(blockIdx.x) * 2 + threadIdx.x;
        if (sb * K3HUF_LANES < n_chunks) sb_bits[sb] = wsum[2 * threadIdx.x] + wsum[2 * threadIdx.x + 1];
    }
}

// Per stripe (one block, thread j = subblock j): exclusive prefix of the
// subblock bit counts. Writes each subblock record's start bit and symbol
// count, the stripe record, and replaces sb_bits[] with the start bits. A
// total that differs from the host's count (the input changed during the
// call) sets *status.
__global__ __launch_bounds__(kScanThreads) void enc_scan(uint8_t* out, const StripeDev* g,
                                                         uint32_t* sb_bits, uint32_t* status) {
    __shared__ uint32_t part[kScanThreads];
    const uint32_t s = blockIdx.x, j = threadIdx.x;
    const StripeDev G = g[s];
    uint32_t* sb = sb_bits + uint64_t(s) * kScanThreads;
    const uint32_t v = j < G.nsb ? sb[j] : 0u;
    part[j] = v;
    __syncthreads();
    for (int d = 1; d < kScanThreads; d <<= 1) {
        const uint32_t t = j >= uint32_t(d) ? part[j - d] : 0u;
        __syncthreads();
        part[j] += t;
        __syncthreads();
    }
    const uint32_t start = part[j] - v;
    if (j < G.nsb) {
        uint8_t* rec = out + G.off + K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * j;
        reinterpret_cast<uint32_t*>(rec)[0] = start;
        reinterpret_cast<uint32_t*>(rec)[1] = min(uint32_t(K3HUF_SUBBLOCK_SYMS), G.n - j * K3HUF_SUBBLOCK_SYMS);
        sb[j] = start;
    }
    if (j == kScanThreads - 1) {
        if (part[j] != G.nbits) atomicOr(status, 1u);
        uint32_t* hd = reinterpret_cast<uint32_t*>(out + G.off);
        hd[0] = G.raw;
        hd[1] = G.n;
        hd[2] = G.nbits;
        hd[3] = G.bit_bytes;
        hd[4] = s * (K3HUF_STRIPE_BYTES / K3HUF_SUBBLOCK_BYTES);
        hd[5] = G.nsb;
        hd[6] = G.bits_off;
        hd[7] = G.even_off;
    }
}

// One wave per unit of 64 lane chunks (half a subblock), lane t packing
// chunk t, in four phases of 64 symbols per chunk (small LDS rows keep 12
// waves per CU):
//   A. whole-wave loads of the phase's raw bytes (8 lanes cover the 128
//      bytes of one chunk's phase); the odd bytes go to the chunk's LDS row,
//      the even bytes straight to the even plane (8 lanes write half a line);
//   B. each lane appends its row's codes, MSB first, to the unit's words in
//      the wave's LDS bit buffer (a lane's first and last words may be
//      shared with its neighbours and are OR-ed in; the words between are its
//      own).
// Then the buffer is written out with whole-wave stores, except the unit's
// first and last words when a neighbouring unit shares them: those go to the
// unit's edge record, and enc_edges writes each shared word once from both
// halves (atomics on words another CU is writing cost more than the rest of
// the copy). A unit whose codes exceed the buffer packs straight into memory,
// OR-ing every shared word (enc_zero_stripes cleared the bitstream), and
// leaves its edge record zero. The layer's last unit, which may end inside a
// chunk, stages its rows symbol by symbol.
constexpr int kPackPhases = 4;
constexpr int kPhSyms = K3HUF_LANE_SYMS / kPackPhases;   // 64 symbols per chunk per phase
constexpr int kRowBytes = kPhSyms + 4;    // 64 odd bytes + 4: rows start in distinct LDS banks

__global__ __launch_bounds__(kPackWaves * 64) void enc_pack(const uint8_t* raw, uint64_t raw_bytes,
                                                            uint64_t n_chunks, CodeTable ct,
                                                            const StripeDev* g, const uint32_t* chunk,
                                                            const uint32_t* sb_start, UnitEdges* edges,
                                                            uint8_t* out) {
    __shared__ uint32_t tab[256];
    __shared__ uint32_t stage[kPackWaves][kPackWords];
    __shared__ __attribute__((aligned(16))) uint8_t rows[kPackWaves][64 * kRowBytes];
    if (threadIdx.x < 256) tab[threadIdx.x] = ct.e[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t u = uint64_t(blockIdx.x) * kPackWaves + wave;   // unit
    const uint64_t n_units = (n_chunks + kUnitChunks - 1) / kUnitChunks;
    if (u >= n_units) return;
    const uint32_t s = uint32_t(u / kUnitsPerStripe);
    const StripeDev G = g[s];
    const uint64_t sbg = u / 2;                         // global subblock
    const uint32_t half = uint32_t(u & 1);
    const uint32_t sbl = uint32_t(sbg % kScanThreads);  // subblock within the stripe
    // bit counts of both halves of the subblock: this unit starts after the
    // first half when it is the second
    const uint64_t ca = sbg * K3HUF_LANES + lane, cb = ca + kUnitChunks;
    const uint32_t ba = ca < n_chunks ? chunk[ca] : 0u, bb = cb < n_chunks ? chunk[cb] : 0u;
    const uint32_t ia = wave_incl_scan(ba, lane), ib = wave_incl_scan(bb, lane);
    const uint32_t bits = half ? bb : ba, incl = half ? ib : ia;
    const uint32_t u0 = sb_start[sbg] + (half ? __shfl(ia, 63) : 0u);
    const uint32_t u1 = u0 + __shfl(incl, 63);
    const uint64_t c0 = u * kUnitChunks;                // first chunk of the unit
    const uint64_t c = c0 + lane;
    const bool has = c < n_chunks;
    uint8_t* rec = out + G.off + K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * sbl;
    if (has) reinterpret_cast<uint16_t*>(rec + 8)[half * kUnitChunks + lane] = uint16_t(bits);

    uint32_t* words = reinterpret_cast<uint32_t*>(out + G.off + G.bits_off);
    uint32_t* buf = stage[wave];
    uint8_t* row = rows[wave];
    const uint32_t w0 = u0 >> 5, nw = ((u1 + 31) >> 5) - w0;
    const bool staged = uint32_t(__builtin_amdgcn_readfirstlane(nw)) <= uint32_t(kPackWords);   // uniform
    if (staged)
        for (uint32_t i = lane; i < nw; i += 64) buf[i] = 0u;
    // the unit's raw bytes, symbols and even plane (stripe symbol index)
    const uint8_t* uraw = raw + c0 * 2 * K3HUF_LANE_SYMS;
    const uint64_t n_syms = raw_bytes / 2;
    const bool tail = (c0 + kUnitChunks) * K3HUF_LANE_SYMS > n_syms;   // layer's last unit, partial
    uint8_t* ueven = out + G.off + G.even_off + uint32_t(c0 % kChunksPerStripe) * K3HUF_LANE_SYMS;
    const int cnt = has ? int(min(uint64_t(K3HUF_LANE_SYMS), n_syms - c * K3HUF_LANE_SYMS)) : 0;

    const uint32_t b0 = u0 + incl - bits;
    uint32_t w = b0 >> 5;
    uint64_t acc = 0;            // pending bits, the earliest at bit 63
    uint32_t nacc = b0 & 31u;    // word w's bits before acc's top belong to the previous lane
    bool first = true;
    // word w of the stripe's bitstream (bit 31 = earliest); shared words are OR-ed
    auto emit = [&](uint32_t v, bool shared) {
        if (staged) {
            if (shared)
                atomicOr(&buf[w - w0], v);
            else
                buf[w - w0] = v;
        } else {
            if (shared)
                atomicOr(&words[w], bswap32(v));
            else
                words[w] = bswap32(v);
        }
    };
    // two symbols into the staged buffer without branches: their codes (at
    // most 24 bits) complete at most one word, which is OR-ed in; when none
    // completes, zero is OR-ed into the word being filled (a no-op)
    auto put2 = [&](uint32_t s0, uint32_t s1) {
        const uint32_t e0 = tab[s0], e1 = tab[s1];
        const uint32_t l1 = e1 >> 16, l = (e0 >> 16) + l1;
        const uint32_t code = ((e0 & 0xFFFFu) << l1) | (e1 & 0xFFFFu);
        acc |= uint64_t(code) << (64u - nacc - l);
        nacc += l;
        const bool full = nacc >= 32;
        atomicOr(&buf[w - w0], full ? uint32_t(acc >> 32) : 0u);
        w += full ? 1u : 0u;
        acc = full ? acc << 32 : acc;
        nacc -= full ? 32u : 0u;
    };
    auto put = [&](uint32_t sym) {
        const uint32_t e = tab[sym];
        const uint32_t l = e >> 16;
        acc |= uint64_t(e & 0xFFFFu) << (64u - nacc - l);
        nacc += l;
        if (nacc >= 32) {
            emit(uint32_t(acc >> 32), first);
            first = false;
            ++w;
            acc <<= 32;
            nacc -= 32;
        }
    };

    // phase ph's raw bytes: chunk i * 8 + sub, bytes [q * 16, q * 16 + 16) of
    // its phase (8 lanes per chunk phase of 128 raw bytes); the next phase's
    // are requested as soon as this phase's are staged
    const int q = lane & 7, sub = lane >> 3;
    uint4 rv[8];
    auto load_raw = [&](int ph) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            rv[i] = *reinterpret_cast<const uint4*>(uraw + uint64_t(i * 8 + sub) * 512 + ph * 2 * kPhSyms + q * 16);
    };
    // B. phase ph's codes, from the lane's row
    auto pack_phase = [&](int ph) {
        if (!has) return;
        const int m = min(max(cnt - ph * kPhSyms, 0), kPhSyms);
        const uint32_t* r = reinterpret_cast<const uint32_t*>(row + lane * kRowBytes);
        if (m == kPhSyms && staged) {
#pragma unroll 4
            for (int k = 0; k < kPhSyms / 4; ++k) {
                const uint32_t v = r[k];
                put2(v & 0xFFu, (v >> 8) & 0xFFu);
                put2((v >> 16) & 0xFFu, v >> 24);
            }
        } else if (m == kPhSyms) {
#pragma unroll 2
            for (int k = 0; k < kPhSyms / 4; ++k) {
                const uint32_t v = r[k];
                put(v & 0xFFu);
                put((v >> 8) & 0xFFu);
                put((v >> 16) & 0xFFu);
                put(v >> 24);
            }
        } else {
            const uint8_t* rb = row + lane * kRowBytes;
            for (int k = 0; k < m; ++k) put(rb[k]);
        }
    };
    if (!tail) {
        load_raw(0);
        // unrolled, so the raw registers need no copies between phases (a
        // copy waits for every outstanding load and store)
#pragma unroll
        for (int ph = 0; ph < kPackPhases; ++ph) {
            // A. stage this phase's odd bytes and keep its even bytes; the
            // next phase's raw bytes are requested before the even bytes are
            // written, so waiting for those loads never waits for these
            // stores (loads and stores retire in issue order)
            uint2 ev[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int ch = i * 8 + sub;
                const uint4 v = rv[i];
                uint32_t* r = reinterpret_cast<uint32_t*>(row + ch * kRowBytes + q * 8);
                r[0] = __builtin_amdgcn_perm(v.y, v.x, 0x07050301u);
                r[1] = __builtin_amdgcn_perm(v.w, v.z, 0x07050301u);
                ev[i] = make_uint2(__builtin_amdgcn_perm(v.y, v.x, 0x06040200u),
                                   __builtin_amdgcn_perm(v.w, v.z, 0x06040200u));
            }
            if (ph + 1 < kPackPhases) load_raw(ph + 1);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<uint2*>(ueven + (i * 8 + sub) * K3HUF_LANE_SYMS + ph * kPhSyms + q * 8) = ev[i];
            wave_sync();
            pack_phase(ph);
            wave_sync();
        }
    } else {
#pragma unroll 1
        for (int ph = 0; ph < kPackPhases; ++ph) {
            for (int j = ph * kPhSyms; j < min(cnt, (ph + 1) * kPhSyms); ++j) {
                const uint8_t* p = uraw + uint64_t(lane) * 512 + 2 * j;
                row[lane * kRowBytes + (j - ph * kPhSyms)] = p[1];
                ueven[lane * K3HUF_LANE_SYMS + j] = p[0];
            }
            wave_sync();
            pack_phase(ph);
            wave_sync();
        }
    }
    if (has && nacc > 0) emit(uint32_t(acc >> 32), true);
    wave_sync();
    // the unit's edge record: its shared first and last words (staged units)
    // and its bit range
    uint32_t* er = reinterpret_cast<uint32_t*>(edges + u);
    if (lane < 4) {
        const uint32_t f = staged && (u0 & 31u) ? bswap32(buf[0]) : 0u;
        const uint32_t l = staged && (u1 & 31u) ? bswap32(buf[min(nw, uint32_t(kPackWords)) - 1]) : 0u;
        er[lane] = lane == 0 ? f : lane == 1 ? l : lane == 2 ? u0 : u1;
    }
    if (staged) {
        const uint32_t i0 = (u0 & 31u) ? 1u : 0u, i1 = (u1 & 31u) ? nw - 1 : nw;
        for (uint32_t i = i0 + lane; i < i1; i += 64) words[w0 + i] = bswap32(buf[i]);
    }
}

// One thread per packing unit: the word holding the unit's first bit, when
// the unit before it (same stripe) ends inside it, is the OR of both units'
// parts, and the stripe's last unit also writes its own last word. Each such
// word is written by exactly one thread; a unit that packed straight into
// memory has already OR-ed its part in (its edge record is zero), so the
// parts are OR-ed onto what memory holds.
__global__ void enc_edges(const UnitEdges* edges, uint64_t n_units, const StripeDev* g, uint8_t* out) {
    const uint64_t u = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (u >= n_units) return;
    const UnitEdges e = edges[u];
    const StripeDev G = g[u / kUnitsPerStripe];
    uint32_t* words = reinterpret_cast<uint32_t*>(out + G.off + G.bits_off);
    const bool first_in_stripe = u % kUnitsPerStripe == 0;
    const bool last_in_stripe = u + 1 == n_units || (u + 1) % kUnitsPerStripe == 0;
    if ((e.b0 & 31u) && !first_in_stripe)
        words[e.b0 >> 5] |= e.first | edges[u - 1].last;
    if ((e.b1 & 31u) && last_in_stripe) words[e.b1 >> 5] |= e.last;
}

// a kernel launch's status as a return code
int launched() { return hipGetLastError() == hipSuccess ? K3HUF_OK : K3HUF_E_HIP; }

// blocks of `kernel` (block size `threads`, no dynamic LDS) resident on the
// current device at once, or 0 when the runtime cannot tell
template <class K>
int resident_blocks(K kernel, int threads) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess)
        return 0;
    return cus * per;
}

}  // namespace

extern "C" {

int64_t k3huf_encode_work_bytes(uint64_t raw_bytes) {
    if (!raw_bytes || (raw_bytes & 1)) return K3HUF_E_ARG;
    return int64_t(work_layout(raw_bytes).total);
}

int64_t k3huf_encode_layer_dev(const void* d_raw, uint64_t raw_bytes, void* d_out, uint64_t cap,
                               void* d_work, uint64_t work_bytes, void* stream) {
    if (!d_raw || !d_out || !d_work || !raw_bytes || (raw_bytes & 1)) return K3HUF_E_ARG;
    if ((reinterpret_cast<uintptr_t>(d_raw) & 15) || (reinterpret_cast<uintptr_t>(d_out) & 15) ||
        (reinterpret_cast<uintptr_t>(d_work) & 15))
        return K3HUF_E_ARG;
    const int64_t bound = k3huf_encode_bound(raw_bytes);
    if (bound < 0 || uint64_t(bound) > cap) return K3HUF_E_ARG;
    const WorkLayout wl = work_layout(raw_bytes);
    if (work_bytes < wl.total) return K3HUF_E_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint8_t* raw = static_cast<const uint8_t*>(d_raw);
    uint8_t* out = static_cast<uint8_t*>(d_out);
    uint8_t* work = static_cast<uint8_t*>(d_work);
    const uint32_t ns = k3huf_detail::stripes_for(raw_bytes);
    const uint64_t n_chunks = (raw_bytes / 2 + K3HUF_LANE_SYMS - 1) / K3HUF_LANE_SYMS;
    auto* hist = reinterpret_cast<unsigned long long*>(work + wl.hist);
    auto* geom = reinterpret_cast<StripeDev*>(work + wl.geom);
    auto* chunk = reinterpret_cast<uint32_t*>(work + wl.chunks);
    auto* sb_bits = reinterpret_cast<uint32_t*>(work + wl.subblocks);
    auto* status = reinterpret_cast<uint32_t*>(work + wl.status);
    auto* edges = reinterpret_cast<UnitEdges*>(work + wl.edges);

    // 1. per-stripe histograms (the status word is cleared with them)
    hipLaunchKernelGGL(enc_fill_zero, dim3(64), dim3(256), 0, st, reinterpret_cast<uint4*>(work),
                       wl.total / 16);
    const int hist_res = resident_blocks(enc_hist, kHistThreads);
    const unsigned hist_per_stripe = unsigned(std::max(1, (hist_res > 0 ? hist_res : 512) / int(ns)));
    hipLaunchKernelGGL(enc_hist, dim3(hist_per_stripe, ns), dim3(kHistThreads), 0, st, raw,
                       raw_bytes, hist);
    if (launched()) return K3HUF_E_HIP;
    std::vector<uint64_t> h(size_t(ns) * 256);
    if (hipMemcpyAsync(h.data(), hist, h.size() * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return K3HUF_E_HIP;

    // 2. code lengths, canonical codes and the layout, on the host
    uint64_t count[256] = {};
    for (uint32_t s = 0; s < ns; ++s)
        for (int v = 0; v < 256; ++v) count[v] += h[size_t(s) * 256 + v];
    uint8_t len[256];
    if (!k3huf_detail::limited_lengths(count, len)) return K3HUF_E_ARG;
    uint32_t code[256];
    k3huf_detail::canonical_codes(len, code);
    CodeTable ct;
    for (int v = 0; v < 256; ++v) ct.e[v] = (uint32_t(len[v]) << 16) | code[v];
    std::vector<StripeGeom> g;
    uint32_t nsb_total = 0;
    const uint64_t total = k3huf_detail::layout(raw_bytes, h.data(), len, g, &nsb_total);
    if (total > cap) return K3HUF_E_ARG;
    std::vector<uint8_t> hdr(pad256(K3HUF_HDR_BYTES + 8ull * ns));
    k3huf_detail::write_layer_header(hdr.data(), raw_bytes, len, g, nsb_total, total);
    std::vector<StripeDev> gd(ns);
    for (uint32_t s = 0; s < ns; ++s)
        gd[s] = StripeDev{g[s].raw0, g[s].off, g[s].raw, g[s].n, g[s].nsb, g[s].nbits,
                          g[s].bit_bytes, g[s].bits_off, g[s].even_off, 0u};

    // 3. headers, then the byte work
    if (hipMemcpyAsync(out, hdr.data(), hdr.size(), hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(geom, gd.data(), gd.size() * sizeof(StripeDev), hipMemcpyHostToDevice, st) !=
            hipSuccess)
        return K3HUF_E_HIP;
    hipLaunchKernelGGL(enc_zero_stripes, dim3(64, ns), dim3(256), 0, st, out, geom);
    const unsigned chunk_blocks = unsigned((n_chunks + kChunkThreads - 1) / kChunkThreads);
    hipLaunchKernelGGL(enc_count, dim3(chunk_blocks), dim3(kChunkThreads), 0, st, raw, raw_bytes,
                       n_chunks, ct, chunk, sb_bits);
    hipLaunchKernelGGL(enc_scan, dim3(ns), dim3(kScanThreads), 0, st, out, geom, sb_bits, status);
    const uint64_t n_units = (n_chunks + kUnitChunks - 1) / kUnitChunks;
    hipLaunchKernelGGL(enc_pack, dim3(unsigned((n_units + kPackWaves - 1) / kPackWaves)),
                       dim3(kPackWaves * 64), 0, st, raw, raw_bytes, n_chunks, ct, geom, chunk, sb_bits,
                       edges, out);
    hipLaunchKernelGGL(enc_edges, dim3(unsigned((n_units + 255) / 256)), dim3(256), 0, st, edges,
                       n_units, geom, out);
    if (launched()) return K3HUF_E_HIP;
    uint32_t bad = 0;
    if (hipMemcpyAsync(&bad, status, 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return K3HUF_E_HIP;
    return bad ? K3HUF_E_CORRUPT : int64_t(total);
}

}  // extern "C"
