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
// runs in three kernels:
//   enc_hist   per-stripe histograms of the odd bytes;
//   enc_pack   one wave per half subblock (64 lane chunks of 256, or of 64
//              symbols in the layout for small layers; one chunk per lane): the
//              chunks' code bits, the unit's start bit from the units before
//              it (a look-back), its codes packed in LDS and written out, its
//              records, its even bytes and the stripe's zero padding; a
//              unit's first and last words, which a neighbouring unit may
//              share, are set aside;
//   enc_edges  one thread per unit: the words units share, OR-ed from both
//              sides.
// Every byte of the container is written; nothing is cleared beforehand.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "k3huf.h"
#include "k3huf_internal.h"

namespace {

using k3huf_detail::pad256;
using k3huf_detail::StripeGeom;

constexpr int kHistThreads = 1024;
constexpr int kHistCopies = 32;        // sub-histograms per block (lane mod 32)
constexpr int kPackWaves = 4;          // waves (units) per packing block
constexpr int kPackWords = 2048;       // per-wave LDS bit buffer (8 KiB)
constexpr uint32_t kUnitChunks = 64;   // lane chunks per packing unit

// Geometry of a layer with lane chunks of L symbols (K3HUF_LANE_SYMS, or
// K3HUF_LANE_SYMS_SHORT): a subblock holds K3HUF_LANES chunks, a packing unit
// half of them, and a chunk is packed in L / 64 phases.
template <uint32_t L>
struct EGeo {
    static constexpr uint32_t kChunksPerStripe = (K3HUF_STRIPE_BYTES / 2) / L;      // 131072 or 524288
    static constexpr uint32_t kSubSyms = K3HUF_LANES * L;
    static constexpr uint32_t kSubPerStripe = K3HUF_STRIPE_BYTES / (2 * kSubSyms);  // 1024 or 4096
    static constexpr uint32_t kUnitsPerStripe = kChunksPerStripe / kUnitChunks;
    static constexpr int kPhases = int(L) / 64;
};

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
    uint64_t hist, geom, edges, look, status, total;
};

// Per packing unit: its first and last bitstream words when another unit
// shares them (0 otherwise), and its start and end bits.
struct UnitEdges {
    uint32_t first, last, b0, b1;
};

// work buffer: per-stripe histograms (u64), stripe geometry, unit edges,
// the units' look-back words (u64), then a status word and the packing
// kernel's block ticket
WorkLayout work_layout(uint64_t raw_bytes, uint32_t lane_syms = K3HUF_LANE_SYMS) {
    const uint64_t ns = k3huf_detail::stripes_for(raw_bytes);
    const uint64_t n_chunks = (raw_bytes / 2 + lane_syms - 1) / lane_syms;
    const uint64_t n_units = (n_chunks + 63) / 64;
    WorkLayout w;
    w.hist = 0;
    w.geom = align256(w.hist + 256 * 8 * ns);
    w.edges = align256(w.geom + sizeof(StripeDev) * ns);
    w.look = align256(w.edges + sizeof(UnitEdges) * n_units);
    w.status = align256(w.look + 8 * n_units);
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

// One wave per unit of 64 lane chunks (half a subblock), lane t packing
// chunk t:
//   A. the chunks' code bits: whole-wave loads of the unit's raw bytes (8
//      lanes cover the 128 raw bytes of one chunk's quarter), each lane adding
//      up the code lengths of the odd bytes it holds; the sums over each
//      chunk's 8 lanes and their prefix sum give every lane its start bit
//      within the unit and the unit's bit count;
//   B. the start bit, by a decoupled look-back (the single-pass prefix scan
//      of Merrill and Garland, 2016): the unit publishes its bit count in its
//      look-back word (state << 32 | bits; state 1: the unit's own count, 2:
//      the stripe's bits up to and including the unit) and reads the words
//      of the units before it back to the nearest one holding a stripe
//      prefix, adding the counts of those without one yet. A stripe's first
//      unit publishes its prefix at once;
//   C. in four phases of 64 symbols per chunk (small LDS rows keep 12 waves
//      per CU), the odd bytes go to the chunks' LDS rows and the even bytes
//      straight to the even plane; each lane appends its row's codes, MSB
//      first, to the unit's words in the wave's LDS bit buffer from bit 0 of
//      the buffer (a lane's first and last words may be shared with its
//      neighbours and are OR-ed in);
//   D. the buffer is shifted to the start bit's place in its word as it is
//      written out with whole-wave stores, except the unit's first and last
//      words when a neighbouring unit shares them: those go to the unit's
//      edge record, and enc_edges writes each shared word once from both
//      halves (atomics on words another CU is writing cost more than the rest
//      of the copy).
// The look-back is requested before the packing and resolved after it, so
// the wait is mostly covered. A unit whose codes exceed the buffer resolves
// its start bit first, clears its own words and packs straight into memory
// (the words its lanes share are OR-ed), setting aside the words it shares
// with neighbouring units as a buffered unit does. The layer's last unit, which may end inside a chunk, stages its rows
// symbol by symbol. Blocks take their units in ticket order, so a unit only
// waits for units of blocks that are already running, which publish their
// counts before they wait for anything; the wait is bounded all the same (a
// wave that gives up flags bit 2 of *status).
constexpr uint32_t kSpinLimit = 1u << 22;   // look-back re-reads before a wave gives up (~0.2 s)

// look-back words are read and written whole at device scope (every XCD
// sees them)
__device__ __forceinline__ uint64_t look_load(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void look_store(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kPhSyms = 64;               // symbols per chunk per phase
constexpr int kRowBytes = kPhSyms + 4;    // 64 odd bytes + 4: rows start in distinct LDS banks

template <uint32_t L>
__global__ __launch_bounds__(kPackWaves * 64) void enc_pack(const uint8_t* raw, uint64_t raw_bytes,
                                                            uint64_t n_chunks, CodeTable ct,
                                                            const StripeDev* g, UnitEdges* edges,
                                                            uint64_t* look, uint32_t* ticket,
                                                            uint32_t* status, uint8_t* out) {
    __shared__ uint32_t tab[256];
    __shared__ uint8_t lens[256];
    __shared__ uint32_t blk;
    __shared__ uint32_t stage[kPackWaves][kPackWords];
    __shared__ __attribute__((aligned(16))) uint8_t rows[kPackWaves][64 * kRowBytes];
    for (int i = threadIdx.x; i < 256; i += kPackWaves * 64) {
        tab[i] = ct.e[i];
        lens[i] = uint8_t(ct.e[i] >> 16);
    }
    if (threadIdx.x == 0) blk = atomicAdd(ticket, 1u);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t u = uint64_t(blk) * kPackWaves + wave;   // unit
    const uint64_t n_units = (n_chunks + kUnitChunks - 1) / kUnitChunks;
    if (u >= n_units) return;
    using EG = EGeo<L>;
    constexpr int kPackPhases = EG::kPhases;
    constexpr uint32_t kChunkRaw = 2 * L;   // raw bytes of a lane chunk
    const uint32_t s = uint32_t(u / EG::kUnitsPerStripe);
    const StripeDev G = g[s];
    const uint64_t sbg = u / 2;                         // global subblock
    const uint32_t half = uint32_t(u & 1);
    const uint32_t sbl = uint32_t(sbg % EG::kSubPerStripe);  // subblock within the stripe
    const uint64_t us0 = uint64_t(s) * EG::kUnitsPerStripe;  // the stripe's first unit
    const uint64_t c0 = u * kUnitChunks;                // first chunk of the unit
    const uint64_t c = c0 + lane;
    const bool has = c < n_chunks;
    const uint8_t* uraw = raw + c0 * kChunkRaw;
    const uint64_t n_syms = raw_bytes / 2;
    const bool tail = (c0 + kUnitChunks) * L > n_syms;   // layer's last unit, partial
    const int cnt = has ? int(min(uint64_t(L), n_syms - c * L)) : 0;

    // phase ph's raw bytes: chunk i * 8 + sub, bytes [q * 16, q * 16 + 16) of
    // its phase (8 lanes per chunk phase of 128 raw bytes)
    const int q = lane & 7, sub = lane >> 3;
    uint4 rv[8];
    uint4 ra[8], rb[8];   // after A: phases 1 and 2's raw bytes (rv holds phase 0's)
    auto load_into = [&](uint4* r, int ph) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r[i] = *reinterpret_cast<const uint4*>(uraw + uint64_t(i * 8 + sub) * kChunkRaw + ph * 2 * kPhSyms + q * 16);
    };
    auto load_raw = [&](int ph) { load_into(rv, ph); };

    // A. the lane chunks' code bits: every lane adds up the code lengths of
    // the odd bytes it loads (phases 3 and 2, then 1 and 0, two in flight at
    // a time; the bytes of phases 0-2 stay in registers for C, so only phase
    // 3 is read again: all four would take 180 VGPRs, two waves per SIMD),
    // then the 8 lanes of each chunk are summed and lane t takes chunk t's sum
    uint32_t bits = 0;
    if (!tail) {
        uint32_t part[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        auto count = [&](const uint4* r) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t o0 = __builtin_amdgcn_perm(r[i].y, r[i].x, 0x07050301u);
                const uint32_t o1 = __builtin_amdgcn_perm(r[i].w, r[i].z, 0x07050301u);
                part[i] += lens[o0 & 0xFFu] + lens[(o0 >> 8) & 0xFFu] + lens[(o0 >> 16) & 0xFFu] + lens[o0 >> 24] +
                           lens[o1 & 0xFFu] + lens[(o1 >> 8) & 0xFFu] + lens[(o1 >> 16) & 0xFFu] + lens[o1 >> 24];
            }
        };
        if (kPackPhases == 4) {
            load_into(ra, 3);
            load_into(rb, 2);
            count(ra);
            load_into(ra, 1);
            load_into(rv, 0);
            count(rb);
            count(ra);
            count(rv);
        } else {
            load_into(rv, 0);
            count(rv);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t p = part[i];
            p += __shfl_xor(p, 1);
            p += __shfl_xor(p, 2);
            p += __shfl_xor(p, 4);
            const uint32_t x = __shfl(p, (lane & 7) * 8);
            bits = (lane >> 3) == i ? x : bits;
        }
    } else {
        for (int j = 0; j < cnt; ++j) bits += lens[uraw[uint64_t(lane) * kChunkRaw + 2 * j + 1]];
    }

    // B. the unit's bits, published; the look-back's first window (64 units,
    // a word per lane) is requested now and resolved after the packing
    const uint32_t incl = wave_incl_scan(bits, lane);
    const uint32_t total = __shfl(incl, 63);
    const bool first_unit = u == us0;
    if (lane == 0) look_store(&look[u], (uint64_t(first_unit ? 2u : 1u) << 32) | total);
    const uint32_t nrel = (total + 31) >> 5;   // words of the unit's own stream
    const bool staged = uint32_t(__builtin_amdgcn_readfirstlane(nrel)) + 1 <= uint32_t(kPackWords);   // uniform
    int64_t base = int64_t(u) - 1;
    uint64_t lw = 0;
    auto request = [&]() {
        const int64_t j = base - lane;
        lw = j >= int64_t(us0) ? look_load(&look[j]) : (2ull << 32);
    };
    uint32_t u0 = 0;
    // sums the window back to the nearest stripe prefix, re-reading words
    // not yet published (bounded: a wave that gives up flags *status)
    auto resolve = [&]() {
        uint32_t spins = 0;
        for (;;) {
            const uint32_t f = uint32_t(lw >> 32), v = uint32_t(lw);
            const uint64_t pm = __ballot(f == 2u), zm = __ballot(f == 0u);
            if (pm) {
                const int lp = __builtin_ctzll(pm);
                if ((zm & ((2ull << lp) - 1ull)) == 0) {
                    u0 += wave_sum(lane <= lp ? v : 0u);
                    break;
                }
            } else if (zm == 0) {
                u0 += wave_sum(v);
                base -= 64;
                request();
                continue;
            }
            if (++spins > kSpinLimit) {
                if (lane == 0) atomicOr(status, 2u);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
            request();
        }
        if (lane == 0) look_store(&look[u], (2ull << 32) | uint64_t(u0 + total));
    };
    // records: lane bit counts, the subblock's start bit and symbol count,
    // the stripe record (its first unit) and the stripe's total (its last);
    // false when the unit would pass the stripe's bits (its input changed
    // since the histogram): it then writes no bitstream words
    const bool last_unit = u + 1 == n_units || (u + 1) % EG::kUnitsPerStripe == 0;
    uint32_t* words = reinterpret_cast<uint32_t*>(out + G.off + G.bits_off);
    auto records = [&]() -> bool {
        const uint32_t u1 = u0 + total;
        uint8_t* rec = out + G.off + K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * sbl;
        uint16_t* lane_bits = reinterpret_cast<uint16_t*>(rec + 8);
        lane_bits[half * kUnitChunks + lane] = uint16_t(bits);   // 0 for lanes past the layer's end
        if (u + 1 == n_units && half == 0) lane_bits[kUnitChunks + lane] = 0;
        if (half == 0 && lane == 0) {
            reinterpret_cast<uint32_t*>(rec)[0] = u0;
            reinterpret_cast<uint32_t*>(rec)[1] = min(EG::kSubSyms, G.n - sbl * EG::kSubSyms);
        }
        if (first_unit && lane < 8) {
            const uint32_t hv[8] = {G.raw, G.n, G.nbits, G.bit_bytes, s * EG::kSubPerStripe, G.nsb, G.bits_off, G.even_off};
            uint32_t x = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) x = lane == k ? hv[k] : x;
            reinterpret_cast<uint32_t*>(out + G.off)[lane] = x;
        }
        // the zero padding: after the subblock records (the stripe's first
        // unit), after the bitstream's last word and after the even plane
        // (its last unit)
        if (first_unit)
            for (uint32_t i = K3HUF_STRIPE_HDR_BYTES + K3HUF_SUBBLOCK_REC_BYTES * G.nsb + lane; i < G.bits_off; i += 64)
                out[G.off + i] = 0;
        if (last_unit) {
            for (uint32_t i = ((G.nbits + 31) >> 5) + lane; i < (G.even_off - G.bits_off) / 4; i += 64) words[i] = 0u;
            const uint64_t e0 = G.off + G.even_off + G.n, e1 = G.off + ((uint64_t(G.even_off) + G.n + 255) & ~255ull);
            for (uint64_t i = e0 + lane; i < e1; i += 64) out[i] = 0;
        }
        if (lane == 0 && ((last_unit && u1 != G.nbits) || u1 > G.nbits)) atomicOr(status, 1u);
        if (u1 > G.nbits) return false;
        // the unit's last word, when it ends inside it, is the OR of its part
        // and the next unit's (enc_edges): cleared here, where no other unit
        // writes it (the first word of a unit is the last of the one before)
        if (lane == 0 && (u1 & 31u)) words[u1 >> 5] = 0u;
        return true;
    };
    if (!first_unit) request();
    uint32_t* buf = stage[wave];
    if (!staged) {
        if (!first_unit) resolve();
        if (!records()) return;
        // the words only this unit writes start at zero (its lanes OR the
        // words they share); its first and last words, when neighbouring units
        // share them, are collected in buf[0] and buf[1] for its edge record
        const uint32_t u1 = u0 + total;
        for (uint32_t i = (u0 >> 5) + ((u0 & 31u) ? 1u : 0u) + lane; i < (u1 >> 5); i += 64) words[i] = 0u;
        if (lane < 2) buf[lane] = 0u;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
        wave_sync();
    }

    // C. the codes: into the wave's LDS buffer from bit 0 (staged), or
    // straight into the stripe's bitstream at the unit's start bit
    uint8_t* row = rows[wave];
    if (staged)
        for (uint32_t i = lane; i <= nrel; i += 64) buf[i] = 0u;
    // the unit's even plane (stripe symbol index)
    uint8_t* ueven = out + G.off + G.even_off + uint32_t(c0 % EG::kChunksPerStripe) * L;

    const uint32_t b0 = (staged ? 0u : u0) + incl - bits;
    // in-place packing: the unit's first and last words when shared
    const uint32_t wf = (u0 & 31u) ? (u0 >> 5) : ~0u, wl = ((u0 + total) & 31u) ? ((u0 + total) >> 5) : ~0u;
    uint32_t w = b0 >> 5;
    uint64_t acc = 0;            // pending bits, the earliest at bit 63
    uint32_t nacc = b0 & 31u;    // word w's bits before acc's top belong to the previous lane
    bool first = true;
    // word w of the unit's buffer or of the stripe's bitstream (bit 31 =
    // earliest); words two lanes share are OR-ed
    auto emit = [&](uint32_t v, bool shared) {
        if (staged) {
            if (shared)
                atomicOr(&buf[w], v);
            else
                buf[w] = v;
        } else if (w == wf) {
            atomicOr(&buf[0], v);
        } else if (w == wl) {
            atomicOr(&buf[1], v);
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
        atomicOr(&buf[w], full ? uint32_t(acc >> 32) : 0u);
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

    // phase ph's codes, from the lane's row
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
        uint2 evp[8];   // an even phase's even bytes, stored with the next phase's
        // phases 0-2's raw bytes are in rv, ra and rb from A, phase 3's are
        // read into rv during phase 2; unrolled, so the raw registers need no
        // copies between phases (a copy waits for every outstanding load and
        // store)
#pragma unroll
        for (int ph = 0; ph < kPackPhases; ++ph) {
            // stage this phase's odd bytes and keep its even bytes; the next
            // phase's raw bytes are requested before the even bytes are
            // written, so waiting for those loads never waits for these
            // stores (loads and stores retire in issue order)
            uint2 ev[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int ch = i * 8 + sub;
                const uint4 v = ph == 1 ? ra[i] : ph == 2 ? rb[i] : rv[i];
                uint32_t* r = reinterpret_cast<uint32_t*>(row + ch * kRowBytes + q * 8);
                r[0] = __builtin_amdgcn_perm(v.y, v.x, 0x07050301u);
                r[1] = __builtin_amdgcn_perm(v.w, v.z, 0x07050301u);
                ev[i] = make_uint2(__builtin_amdgcn_perm(v.y, v.x, 0x06040200u),
                                   __builtin_amdgcn_perm(v.w, v.z, 0x06040200u));
            }
            if (kPackPhases == 4 && ph == 2) load_raw(3);
            if (kPackPhases == 1) {
                // 64-byte chunks: eight consecutive chunks' even bytes are
                // four whole 128-byte lines
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<uint2*>(ueven + (i * 8 + sub) * L + q * 8) = ev[i];
            } else if (ph & 1) {
                // both halves of each 128-byte even-plane line, back to back
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    uint8_t* e = ueven + (i * 8 + sub) * L + (ph - 1) * kPhSyms + q * 8;
                    *reinterpret_cast<uint2*>(e) = evp[i];
                    *reinterpret_cast<uint2*>(e + kPhSyms) = ev[i];
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) evp[i] = ev[i];
            }
            wave_sync();
            pack_phase(ph);
            wave_sync();
        }
    } else {
#pragma unroll 1
        for (int ph = 0; ph < kPackPhases; ++ph) {
            for (int j = ph * kPhSyms; j < min(cnt, (ph + 1) * kPhSyms); ++j) {
                const uint8_t* p = uraw + uint64_t(lane) * kChunkRaw + 2 * j;
                row[lane * kRowBytes + (j - ph * kPhSyms)] = p[1];
                ueven[lane * L + j] = p[0];
            }
            wave_sync();
            pack_phase(ph);
            wave_sync();
        }
    }
    if (has && nacc > 0) emit(uint32_t(acc >> 32), true);
    wave_sync();
    if (!staged) {
        // packed in place: the edge record holds the shared words and the bit range
        if (lane < 4) {
            const uint32_t first_w = (u0 & 31u) ? bswap32(buf[0]) : 0u;
            const uint32_t last_w = ((u0 + total) & 31u) ? bswap32(buf[1]) : 0u;
            reinterpret_cast<uint32_t*>(edges + u)[lane] = lane == 0 ? first_w : lane == 1 ? last_w : lane == 2 ? u0 : u0 + total;
        }
        return;
    }

    // D. the start bit, the records, then the buffer shifted to the start
    // bit's position in its word and written out: word w0 + i of the stripe
    // takes the low r bits of buffer word i - 1 and the high 32 - r bits of
    // buffer word i (r = u0 mod 32; buf[nrel] is zero)
    if (!first_unit) resolve();
    if (!records()) return;
    const uint32_t u1 = u0 + total;
    const uint32_t r = u0 & 31u, w0 = u0 >> 5, nw = ((u1 + 31) >> 5) - w0;
    auto word = [&](uint32_t i) -> uint32_t {
        const uint32_t hi = buf[i], lo = i ? buf[i - 1] : 0u;
        return r ? (lo << (32u - r)) | (hi >> r) : hi;
    };
    // the unit's edge record: its first and last words when a neighbouring
    // unit shares them, and its bit range
    if (lane < 4) {
        const uint32_t first_w = r ? bswap32(word(0)) : 0u;
        const uint32_t last_w = (u1 & 31u) ? bswap32(word(nw - 1)) : 0u;
        reinterpret_cast<uint32_t*>(edges + u)[lane] = lane == 0 ? first_w : lane == 1 ? last_w : lane == 2 ? u0 : u1;
    }
    const uint32_t i0 = r ? 1u : 0u, i1 = (u1 & 31u) ? nw - 1 : nw;
    for (uint32_t i = i0 + lane; i < i1; i += 64) words[w0 + i] = bswap32(word(i));
}

// One thread per packing unit: the word holding the unit's first bit, when
// the unit before it (same stripe) ends inside it, is the OR of both units'
// parts, and the stripe's last unit also writes its own last word. Each such
// word is written by exactly one thread. enc_pack left every such word zero
// (a unit clears its last word when it ends inside it), so the parts are
// OR-ed onto zero; OR-ing also gives the right word when a unit's first and
// last words are one word.
template <uint32_t L>
__global__ void enc_edges(const UnitEdges* edges, uint64_t n_units, const StripeDev* g, uint8_t* out) {
    constexpr uint32_t kUnitsPerStripe = EGeo<L>::kUnitsPerStripe;
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

// Pinned host staging for the encoder's round trips through the host (the
// histograms in, the layer header and stripe geometry out, the status word
// in), so that they run as DMA in stream order: copies from pageable memory
// are staged by the host, which first waits for the stream. Buffers are
// leased from a process-wide pool (a call takes one and gives it back) and
// are never freed while the process runs; a lease given back while copies
// from it may be queued (an error path) waits for its stream first.
std::mutex g_pin_mu;
std::vector<std::pair<void*, size_t>> g_pin_pool;

struct PinnedLease {
    void* p = nullptr;
    size_t n = 0;
    explicit PinnedLease(size_t want) {
        std::lock_guard<std::mutex> lk(g_pin_mu);
        for (size_t i = 0; i < g_pin_pool.size(); ++i)
            if (g_pin_pool[i].second >= want) {
                p = g_pin_pool[i].first;
                n = g_pin_pool[i].second;
                g_pin_pool.erase(g_pin_pool.begin() + long(i));
                return;
            }
        if (!g_pin_pool.empty()) {   // too small for this call: replace it
            (void)hipHostFree(g_pin_pool.back().first);
            g_pin_pool.pop_back();
        }
        if (hipHostMalloc(&p, want, hipHostMallocDefault) != hipSuccess) {
            p = nullptr;
            return;
        }
        n = want;
    }
    ~PinnedLease() {
        if (!p) return;
        std::lock_guard<std::mutex> lk(g_pin_mu);
        g_pin_pool.emplace_back(p, n);
    }
    PinnedLease(const PinnedLease&) = delete;
    PinnedLease& operator=(const PinnedLease&) = delete;
};

// Waits for `st` on scope exit while work of the call may still be queued on
// it (an error path returns early), so that neither the host staging nor the
// work buffer is reused under a pending copy or kernel.
struct QueueGuard {
    hipStream_t st;
    bool queued = false;
    explicit QueueGuard(hipStream_t s) : st(s) {}
    ~QueueGuard() {
        if (queued) (void)hipStreamSynchronize(st);
    }
};

// Bytes of host staging a call needs for ns stripes: the histograms, the
// layer header with its stripe offsets, the stripe geometry, a status word.
struct HostStageLayout {
    size_t hist, hdr, geom, status, total;
};
HostStageLayout host_stage_layout(uint32_t ns) {
    HostStageLayout h;
    h.hist = 0;
    h.hdr = size_t(ns) * 256 * 8;
    h.geom = h.hdr + pad256(K3HUF_HDR_BYTES + 8ull * ns);
    h.status = h.geom + ((size_t(ns) * sizeof(StripeDev) + 15) & ~size_t(15));
    h.total = h.status + 16;
    return h;
}

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

// One encode: device layer raw -> container out with lane chunks of
// lane_syms symbols, with the device work buffer `work`
// (work_layout(raw_bytes, lane_syms).total bytes), host staging `host`
// (host_stage_layout(ns).total bytes) and stripe geometry storage g (ns
// entries). Allocates nothing; synchronous.
int64_t encode_dev(const uint8_t* raw, uint64_t raw_bytes, uint32_t lane_syms, uint8_t* out, uint64_t cap,
                   uint8_t* work, hipStream_t st, uint8_t* host, StripeGeom* g) {
    const WorkLayout wl = work_layout(raw_bytes, lane_syms);
    const uint32_t ns = k3huf_detail::stripes_for(raw_bytes);
    const uint64_t n_chunks = (raw_bytes / 2 + lane_syms - 1) / lane_syms;
    auto* hist = reinterpret_cast<unsigned long long*>(work + wl.hist);
    auto* geom = reinterpret_cast<StripeDev*>(work + wl.geom);
    auto* look = reinterpret_cast<uint64_t*>(work + wl.look);
    auto* status = reinterpret_cast<uint32_t*>(work + wl.status);   // [0] status, [1] block ticket
    auto* edges = reinterpret_cast<UnitEdges*>(work + wl.edges);
    const HostStageLayout hl = host_stage_layout(ns);
    const uint64_t* h = reinterpret_cast<const uint64_t*>(host + hl.hist);
    uint8_t* host_hdr = host + hl.hdr;
    StripeDev* gd = reinterpret_cast<StripeDev*>(host + hl.geom);
    uint32_t* host_status = reinterpret_cast<uint32_t*>(host + hl.status);
    QueueGuard guard(st);

    // 1. per-stripe histograms (the look-back words, the status word and the
    // block ticket are cleared with them, by a kernel)
    guard.queued = true;
    hipLaunchKernelGGL(enc_fill_zero, dim3(64), dim3(256), 0, st, reinterpret_cast<uint4*>(work),
                       wl.total / 16);
    const int hist_res = resident_blocks(enc_hist, kHistThreads);
    const unsigned hist_per_stripe = unsigned(std::max(1, (hist_res > 0 ? hist_res : 512) / int(ns)));
    hipLaunchKernelGGL(enc_hist, dim3(hist_per_stripe, ns), dim3(kHistThreads), 0, st, raw,
                       raw_bytes, hist);
    if (launched()) return K3HUF_E_HIP;
    if (hipMemcpyAsync(host + hl.hist, hist, hl.hdr - hl.hist, hipMemcpyDeviceToHost, st) != hipSuccess ||
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
    uint32_t nsb_total = 0;
    const uint64_t total = k3huf_detail::layout(raw_bytes, h, len, g, &nsb_total, lane_syms);
    if (total > cap) return K3HUF_E_ARG;
    k3huf_detail::write_layer_header(host_hdr, raw_bytes, len, g, nsb_total, total, lane_syms);
    for (uint32_t s = 0; s < ns; ++s)
        gd[s] = StripeDev{g[s].raw0, g[s].off, g[s].raw, g[s].n, g[s].nsb, g[s].nbits,
                          g[s].bit_bytes, g[s].bits_off, g[s].even_off, 0u};

    // 3. headers, then the byte work
    if (hipMemcpyAsync(out, host_hdr, hl.geom - hl.hdr, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(geom, gd, size_t(ns) * sizeof(StripeDev), hipMemcpyHostToDevice, st) != hipSuccess)
        return K3HUF_E_HIP;
    const uint64_t n_units = (n_chunks + kUnitChunks - 1) / kUnitChunks;
    const dim3 pack_grid(unsigned((n_units + kPackWaves - 1) / kPackWaves)), edge_grid(unsigned((n_units + 255) / 256));
    if (lane_syms == K3HUF_LANE_SYMS_SHORT) {
        hipLaunchKernelGGL(enc_pack<K3HUF_LANE_SYMS_SHORT>, pack_grid, dim3(kPackWaves * 64), 0, st, raw, raw_bytes,
                           n_chunks, ct, geom, edges, look, status + 1, status, out);
        hipLaunchKernelGGL(enc_edges<K3HUF_LANE_SYMS_SHORT>, edge_grid, dim3(256), 0, st, edges, n_units, geom, out);
    } else {
        hipLaunchKernelGGL(enc_pack<K3HUF_LANE_SYMS>, pack_grid, dim3(kPackWaves * 64), 0, st, raw, raw_bytes,
                           n_chunks, ct, geom, edges, look, status + 1, status, out);
        hipLaunchKernelGGL(enc_edges<K3HUF_LANE_SYMS>, edge_grid, dim3(256), 0, st, edges, n_units, geom, out);
    }
    if (launched()) return K3HUF_E_HIP;
    if (hipMemcpyAsync(host_status, status, 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return K3HUF_E_HIP;
    guard.queued = false;
    const uint32_t bad = *host_status;
    return (bad & 2u) ? K3HUF_E_HIP : bad ? K3HUF_E_CORRUPT : int64_t(total);
}

// Argument checks shared by the entry points (sizes, alignment, lane-chunk
// length, capacity).
bool encode_args_ok(const void* d_raw, uint64_t raw_bytes, const void* d_out, uint64_t cap,
                    uint32_t lane_syms = K3HUF_LANE_SYMS) {
    if (!d_raw || !d_out || !raw_bytes || (raw_bytes & 1) || !k3huf_detail::lane_syms_ok(lane_syms)) return false;
    if ((reinterpret_cast<uintptr_t>(d_raw) & 15) || (reinterpret_cast<uintptr_t>(d_out) & 15)) return false;
    const int64_t bound = k3huf_encode_bound_lanes(raw_bytes, lane_syms);
    return bound >= 0 && uint64_t(bound) <= cap;
}

// The entry point without allocation: its work buffer is this file-scope
// device array (one per GPU, kept until the process ends), its host staging
// and stripe geometry are file-scope host arrays. Layers up to
// K3HUF_STATIC_MAX_RAW bytes: 64 stripes and 131,072 packing units.
constexpr uint32_t kStaticStripes = uint32_t(K3HUF_STATIC_MAX_RAW / K3HUF_STRIPE_BYTES);
constexpr uint64_t kStaticUnits = K3HUF_STATIC_MAX_RAW / 2 / K3HUF_LANE_SYMS / kUnitChunks;
constexpr uint64_t kStaticWorkBytes = 256 * 8 * kStaticStripes + 256 + sizeof(StripeDev) * kStaticStripes +
                                      256 + sizeof(UnitEdges) * kStaticUnits + 256 + 8 * kStaticUnits + 256 +
                                      256;
static __device__ __align__(256) uint8_t scratch[kStaticWorkBytes];
alignas(64) uint8_t g_static_host[size_t(256) * 8 * kStaticStripes +
                                  256 * ((K3HUF_HDR_BYTES + 8 * kStaticStripes + 255) / 256) +
                                  sizeof(StripeDev) * kStaticStripes + 16 + 16];
StripeGeom g_static_geom[kStaticStripes];
std::mutex g_static_mu;                  // one call at a time uses the arrays
constexpr int kMaxDevices = 64;
uint8_t* g_scratch_ptr[kMaxDevices] = {};  // per device: the address of `scratch` there

}  // namespace

extern "C" {

int64_t k3huf_encode_work_bytes_lanes(uint64_t raw_bytes, uint32_t lane_syms) {
    if (!raw_bytes || (raw_bytes & 1) || !k3huf_detail::lane_syms_ok(lane_syms)) return K3HUF_E_ARG;
    return int64_t(work_layout(raw_bytes, lane_syms).total);
}

int64_t k3huf_encode_work_bytes(uint64_t raw_bytes) {
    return k3huf_encode_work_bytes_lanes(raw_bytes, K3HUF_LANE_SYMS);
}

int64_t k3huf_encode_layer_dev_lanes(const void* d_raw, uint64_t raw_bytes, uint32_t lane_syms, void* d_out,
                                     uint64_t cap, void* d_work, uint64_t work_bytes, void* stream) {
    if (!d_work || (reinterpret_cast<uintptr_t>(d_work) & 15) ||
        !encode_args_ok(d_raw, raw_bytes, d_out, cap, lane_syms))
        return K3HUF_E_ARG;
    if (work_bytes < work_layout(raw_bytes, lane_syms).total) return K3HUF_E_ARG;
    const uint32_t ns = k3huf_detail::stripes_for(raw_bytes);
    PinnedLease pin(host_stage_layout(ns).total);
    if (!pin.p) return K3HUF_E_HIP;
    std::vector<StripeGeom> g(ns);
    return encode_dev(static_cast<const uint8_t*>(d_raw), raw_bytes, lane_syms, static_cast<uint8_t*>(d_out), cap,
                      static_cast<uint8_t*>(d_work), static_cast<hipStream_t>(stream),
                      static_cast<uint8_t*>(pin.p), g.data());
}

int64_t k3huf_encode_layer_dev(const void* d_raw, uint64_t raw_bytes, void* d_out, uint64_t cap,
                               void* d_work, uint64_t work_bytes, void* stream) {
    return k3huf_encode_layer_dev_lanes(d_raw, raw_bytes, K3HUF_LANE_SYMS, d_out, cap, d_work, work_bytes, stream);
}

int64_t k3huf_encode_layer_dev_static(const void* d_raw, uint64_t raw_bytes, void* d_out, uint64_t cap,
                                      void* stream) {
    if (!encode_args_ok(d_raw, raw_bytes, d_out, cap) || raw_bytes > K3HUF_STATIC_MAX_RAW ||
        work_layout(raw_bytes).total > sizeof(scratch) ||
        host_stage_layout(k3huf_detail::stripes_for(raw_bytes)).total > sizeof(g_static_host))
        return K3HUF_E_ARG;
    std::lock_guard<std::mutex> lk(g_static_mu);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return K3HUF_E_HIP;
    if (!g_scratch_ptr[dev]) {
        // first call on this device (current here): the device address of
        // its copy of the array; host code uses only this address
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return K3HUF_E_HIP;
        g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
    }
    return encode_dev(static_cast<const uint8_t*>(d_raw), raw_bytes, K3HUF_LANE_SYMS, static_cast<uint8_t*>(d_out),
                      cap, g_scratch_ptr[dev], static_cast<hipStream_t>(stream), g_static_host, g_static_geom);
}

}  // extern "C"
