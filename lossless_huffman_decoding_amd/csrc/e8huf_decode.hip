// gfx950 decoder of the FP8 exponent codec (include/e8huf.h).
//
// What is computed (ECF8 page, "指数集中现象：GenAI模型权重压缩的理论基础",
// pwwt.cn/news/2030120): FP8 values (section 1.2) whose exponent fields were
// Huffman coded (codes of at most 16 bits, section 2.1) are rebuilt from the
// codes and the raw sign/mantissa nibbles. Section 2.2's decoder gives each
// thread its start bit from per-block metadata, decodes into on-chip memory
// and writes the output out coalesced; section 2.1's two-level table (8-bit
// first level, 8-bit second level) resolves the codes.
//
// How it is laid out on the GPU (not from the page): one wave decodes one
// block of 16,384 values; lane t decodes its lane chunk t (256 values) from
// the start bit the block record's prefix sum gives it. The block's codes are
// copied into the wave's LDS buffer first. The workgroup derives, from the
// two-level table, an LDS table on 12-bit prefixes whose entries hold up to
// three whole codes (the codes of frequent exponents are 2-4 bits long);
// codes longer than 12 bits go through the second level of the two-level
// table, kept in LDS too. Decoded exponents are staged in LDS rows, so that
// each output store instruction writes whole 128-byte lines, combined with
// the sign/mantissa nibbles on the way out.
//
// The page's decoder hands its output over as 16-bit floats (section 2.2);
// e8huf_decode_widen does that: each rebuilt FP8 value goes through the
// hardware's FP8-to-float conversion, is multiplied by the caller's scale in
// single precision and is rounded to bfloat16 or half (nearest even) by the
// packed narrowing conversion, on the way out.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "e8huf.h"

namespace {

// Waves per workgroup (one workgroup per CU): the decode is bound by each
// lane's chain of dependent LDS lookups, so more waves per CU run faster
// (measured on the FP8 trunk tensor: 0.375, 0.317, 0.283, 0.272 and 0.258 ms
// at 5, 6, 7, 8 and 9 waves); nine is what LDS leaves room for.
constexpr int kWaves = 9;
constexpr int kThreads = 64 * kWaves;
constexpr int kLanes = 64;
constexpr int kChunk = int(E8HUF_LANE_VALUES);        // values per lane chunk
constexpr int kPhase = 128;                           // values per lane per phase
constexpr int kPhases = kChunk / kPhase;              // 2
constexpr int kBufBytes = 6144;                       // per-wave bitstream buffer (a block's codes take ~5.2 KB on weights)
constexpr int kBufUnits = kBufBytes / 16;
// stage row: the phase's 128 symbols, up to two carried past it plus the
// unused third byte of the last lookup, and a spare spot where lanes outside
// the phase write; 35 dwords (odd, so rows start in different banks)
constexpr int kStageStride = kPhase + 12;
constexpr uint32_t kSpare = kPhase + 5;
constexpr int kWaveLds = kBufBytes + kLanes * kStageStride;
constexpr int kTabEntries = 4096;                     // 12-bit decode table
constexpr int kLookups = 5;                           // lookups per 64-bit window: five 12-bit codes fit
// LDS layout: the 12-bit table, the code lengths, each wave's buffer and
// stage rows (static), then the two-level table (dynamic, its actual size)
constexpr int kLenOff = kTabEntries * 4;
constexpr int kWaveOff = kLenOff + 64;
constexpr int kLdsStatic = kWaveOff + kWaves * kWaveLds;
static_assert(kLdsStatic + 16 + E8HUF_LUT_MAX * 2 <= 163840, "LDS budget, with the largest two-level table");

// 12-bit table entry:
//   [23:0]  up to three exponent symbols, one per byte, first code lowest;
//           each already shifted left by the mantissa width, so it is the
//           FP8 byte's exponent field in place
//   [27:24] symbols in the entry
//   [31:28] bits the entry's codes take (1..12)
// count and length are both 4-bit fields, so one field width (4, or 0 for a
// lane that has its symbols) masks both extractions. An escape entry (the
// first code is longer than 12 bits, or no code covers the prefix) has
// count and length 0 and holds in [7:0] the level-2 table of its first 8
// bits plus one (0: no code).
constexpr uint32_t kBadE = 1u << 7;   // in Lane::bad: a code that no table covers
constexpr uint32_t kCntPos = 24, kLenPos = 28;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// output kinds: FP8 bytes, or 16-bit floats (E8HUF_OUT_BF16, E8HUF_OUT_F16)
constexpr int kOutFp8 = 0;

// Output stage per kind: each lane stores 16 bytes per round, so FP8 output
// takes 16 values per lane (8 lanes per chunk's phase) and 16-bit output 8
// (16 lanes); either way a store instruction writes whole 128-byte lines.
template <int kOut>
struct OutStage {
    static constexpr int kVals = kOut == kOutFp8 ? 16 : 8;       // values per lane and round
    static constexpr int kPartLanes = kPhase / kVals;            // lanes storing one chunk's phase
    static constexpr int kPartShift = kPartLanes == 16 ? 4 : 3;
    static constexpr int kRounds = kPartLanes;                   // rounds per phase (64 / kPartLanes chunks each)
    static constexpr int kOutBytes = kOut == kOutFp8 ? 1 : 2;
    using Nib = typename std::conditional<kOut == kOutFp8, uint2, uint32_t>::type;   // the round's nibbles
    static_assert((1 << kPartShift) == kPartLanes, "phase of 128 values");
};

struct Args {
    const uint8_t* blob;
    uint64_t blob_bytes;
    const uint16_t* lut;
    uint32_t lut_entries;
    uint8_t* out;
    uint64_t n;
    uint32_t* status;
    float scale;   // 16-bit output: the factor each value is multiplied by
};

__device__ __forceinline__ uint32_t ld32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ uint64_t ld64(const uint8_t* p) { return *reinterpret_cast<const uint64_t*>(p); }
__device__ __forceinline__ uint32_t bswap32(uint32_t x) { return __builtin_amdgcn_perm(0u, x, 0x00010203u); }
__device__ __forceinline__ void flag(uint32_t* status, uint32_t bit) {
    if (status) atomicOr(status, bit);
}
__device__ __forceinline__ uint32_t bit(bool c) { return c ? 1u : 0u; }
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}
// inclusive prefix sum over the 64 lanes (DPP row shifts, then row broadcasts)
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);
    return x;
}
__device__ __forceinline__ uint32_t lane_value(uint32_t v, uint32_t l) { return __builtin_amdgcn_readlane(v, l); }

// The code at the start of the 16-bit string s16 (first bit = bit 15; bits
// the caller does not know are zeros) from the two-level table in LDS:
// (symbol << 8) | length, or 0 when no code covers it. A code longer than the
// known bits comes back too; the caller compares lengths.
__device__ __forceinline__ uint32_t two_level(const uint16_t* l2, uint32_t l2_last, uint32_t s16) {
    uint32_t e = l2[s16 >> 8];
    if (e & 0x20u) e = l2[min(256u * (1u + (e >> 8)) + (s16 & 0xFFu), l2_last)];
    return e;
}

// 12-bit table entry for prefix i: up to three whole codes of the 12 bits.
__device__ uint32_t make_entry(const uint16_t* l2, uint32_t l2_last, uint32_t i, uint32_t m) {
    uint32_t syms = 0, k = 0, pos = 0;
    const uint32_t first = two_level(l2, l2_last, i << 4);
    if ((first & 31u) == 0u) return 0u;   // no code
    if ((first & 31u) > 12u) return (l2[i >> 4] >> 8) + 1u;   // the level-1 link of the first 8 bits
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const uint32_t e = two_level(l2, l2_last, ((i << pos) & 0xFFFu) << 4);
        const uint32_t l = e & 31u;
        if (l == 0u || pos + l > 12u) break;
        syms |= ((e >> 8) << m) << (8 * k);
        ++k;
        pos += l;
    }
    return syms | (k << kCntPos) | (pos << kLenPos);
}

// 64-bit window whose top bit is the bit after buffer bit pm1 (buffer dwords
// held byte-swapped, bit 31 first).
__device__ __forceinline__ uint64_t window(const uint32_t* buf, uint32_t pm1) {
    const uint32_t* p = buf + (pm1 >> 5);
    const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
    const uint32_t r = ~pm1;
    return (uint64_t(__builtin_amdgcn_alignbit(d0, d1, r)) << 32) | __builtin_amdgcn_alignbit(d1, d2, r);
}

// per-lane decode state across a block's phases
struct Lane {
    uint32_t pm1;      // buffer bit index of the next code, minus one
    uint32_t cnt;      // symbols decoded so far (may pass the lane's count by two)
    uint32_t bad;      // kBadE: a code that no table covers
    uint32_t m;        // staged symbols are exponents shifted left by m (mantissa bits)
};

// Decode of a lane's symbols [base, target) into its stage row (byte i of the
// row is symbol base + i). Each 64-bit window feeds kLookups lookups of the
// 12-bit table; an entry's symbols are written as three bytes at the lane's
// write position p (bytes past the entry's symbols are overwritten by the
// next lookup or lie past the phase). A lane that has its symbols extracts
// both fields with width 0 (no bits, no symbols) until the wave's slowest
// lane is done; the bytes of its entries land after its last symbol. An
// escape entry (the first code is longer than 12 bits, or no code covers the
// prefix) yields nothing, so the lane stays on that code for the rest of the
// window; after the window, lanes on an escape take that one code through
// the second-level table, or flag it. Every window either yields a symbol on each live lane
// or resolves an escape, so 2 * 64 windows always finish a phase. A lookup
// that ends past the phase leaves up to two symbols in the row's bytes
// kPhase and kPhase + 1; they move to the start of the next phase's row. A
// lane with nothing to decode in the phase writes only to the spare bytes.
__device__ __forceinline__ void decode_phase(const uint32_t* tab, const uint16_t* l2, uint32_t l2_last,
                                             const uint32_t* buf, uint8_t* row, uint32_t target, uint32_t base,
                                             Lane& ls) {
    const bool act = target > base;
    uint8_t* p = row + kSpare;
    if (act) {
        const uint32_t j = ls.cnt - base;   // 0..2 symbols carried over
        if (j) {
            row[0] = row[kPhase];
            row[1] = row[kPhase + 1];
        }
        p = row + j;
    }
    uint8_t* const pend = act ? row + (target - base) : p;
    // each lookup's three bytes are written after the next table read has
    // been issued (a wave's LDS operations complete in order, so that read
    // waits for no write); the first pending write is a dummy in the spare
    // bytes, and the pending write goes out before an escape's own byte
    uint8_t* wp = row + kSpare;
    uint32_t we = 0;
#pragma unroll 1
    for (int win = 0; win < 2 * kPhase; ++win) {
        if (!__any(p < pend)) break;
        uint64_t acc = window(buf, ls.pm1);
        uint32_t t = 0;
#pragma unroll
        for (int q = 0; q < kLookups; ++q) {
            const uint32_t e = tab[uint32_t(acc >> 52)];
            wp[0] = uint8_t(we);
            wp[1] = uint8_t(we >> 8);
            wp[2] = uint8_t(we >> 16);
            // a lane that has its symbols extracts zero-width fields: no
            // bits, no symbols, and the mask stays off the chain of reads;
            // its entry's bytes go after its last symbol
            const uint32_t w = p < pend ? 4u : 0u;
            t = __builtin_amdgcn_ubfe(e, kLenPos, w);
            wp = p;
            we = e;
            p += __builtin_amdgcn_ubfe(e, kCntPos, w);
            ls.pm1 += t;
            acc <<= t;
        }
        // a live lane's lookup takes no bits only on an escape entry, which
        // it then repeats to the end of the window; at most 48 of the
        // window's bits were taken before it, so the window still holds the
        // code's 16 bits, and the pending entry is the escape entry (a
        // second-level entry of length 0, or no link: a bad code)
        if (__any(t == 0u && p < pend)) {
            wp[0] = uint8_t(we);
            wp[1] = uint8_t(we >> 8);
            wp[2] = uint8_t(we >> 16);
            if (t == 0u && p < pend) {
                const uint32_t link = we & 0xFFu;
                const uint32_t e2 = link ? l2[min(256u * link + uint32_t((acc >> 48) & 0xFFu), l2_last)] : 0u;
                const uint32_t l = e2 & 31u;
                *p++ = uint8_t((e2 >> 8) << ls.m);
                ls.bad |= l ? 0u : kBadE;
                ls.pm1 += l ? l : 16u;
            }
            wp = row + kSpare;
            we = 0;
        }
    }
    wp[0] = uint8_t(we);
    wp[1] = uint8_t(we >> 8);
    wp[2] = uint8_t(we >> 16);
    if (act) ls.cnt = base + uint32_t(p - row);
}

// the 16 staged exponents of chunk c at phase offset 16 part (rows are 4-byte
// aligned, so four dword reads)
__device__ __forceinline__ v4u staged16(const uint8_t* stage, int c, int part) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(stage + c * kStageStride + part * 16);
    v4u r;
    r.x = p[0];
    r.y = p[1];
    r.z = p[2];
    r.w = p[3];
    return r;
}

// FP8 bytes from 16 staged exponents (four dwords) and their 16 nibbles
// (eight bytes: value 2i low nibble, 2i + 1 high nibble).
__device__ __forceinline__ v4u combine(v4u ex, uint2 nib, uint32_t m, uint32_t smask, uint32_t mmask) {
    const uint32_t lo0 = nib.x & 0x0F0F0F0Fu, hi0 = (nib.x >> 4) & 0x0F0F0F0Fu;
    const uint32_t lo1 = nib.y & 0x0F0F0F0Fu, hi1 = (nib.y >> 4) & 0x0F0F0F0Fu;
    const uint32_t nb[4] = {__builtin_amdgcn_perm(hi0, lo0, 0x05010400u), __builtin_amdgcn_perm(hi0, lo0, 0x07030602u),
                            __builtin_amdgcn_perm(hi1, lo1, 0x05010400u), __builtin_amdgcn_perm(hi1, lo1, 0x07030602u)};
    v4u o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t e = i == 0 ? ex.x : i == 1 ? ex.y : i == 2 ? ex.z : ex.w;
        const uint32_t v = ((nb[i] << (7u - m)) & smask) | e | (nb[i] & mmask);
        if (i == 0) o.x = v;
        else if (i == 1) o.y = v;
        else if (i == 2) o.z = v;
        else o.w = v;
    }
    return o;
}

// the 8 staged exponents of chunk c at phase offset 8 part (two dword reads)
__device__ __forceinline__ uint2 staged8(const uint8_t* stage, int c, int part) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(stage + c * kStageStride + part * 8);
    return make_uint2(p[0], p[1]);
}

// FP8 bytes from 8 staged exponents (two dwords) and their 8 nibbles (four
// bytes: value 2i low nibble, 2i + 1 high nibble).
__device__ __forceinline__ uint2 combine8(uint2 ex, uint32_t nib, uint32_t m, uint32_t smask, uint32_t mmask) {
    const uint32_t lo = nib & 0x0F0F0F0Fu, hi = (nib >> 4) & 0x0F0F0F0Fu;
    const uint32_t n0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u), n1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
    return make_uint2(((n0 << (7u - m)) & smask) | ex.x | (n0 & mmask), ((n1 << (7u - m)) & smask) | ex.y | (n1 & mmask));
}

// Four FP8 values (one dword, value k in byte k) as floats: the hardware
// conversions take E4M3 (fp8) or E5M2 (bf8) from either 16-bit half.
template <bool kE5M2, bool kHigh>
__device__ __forceinline__ v2f fp8_pair(uint32_t x) {
    if constexpr (kE5M2)
        return __builtin_amdgcn_cvt_pk_f32_bf8(x, kHigh);
    else
        return __builtin_amdgcn_cvt_pk_f32_fp8(x, kHigh);
}

// Eight FP8 values (two dwords) times scale, rounded to the output kind:
// sixteen bytes of output, value k in halfword k.
template <int kOut, bool kE5M2>
__device__ __forceinline__ v4u widen8(uint2 f, float scale) {
    v2f v[4] = {fp8_pair<kE5M2, false>(f.x), fp8_pair<kE5M2, true>(f.x), fp8_pair<kE5M2, false>(f.y),
                fp8_pair<kE5M2, true>(f.y)};
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i].x *= scale;
        v[i].y *= scale;
        if (kOut == E8HUF_OUT_BF16)
            w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v[i], v2bf));
        else
            w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v[i], v2h));
    }
    v4u o;
    o.x = w[0];
    o.y = w[1];
    o.z = w[2];
    o.w = w[3];
    return o;
}

// The 16 output bytes of round rr's lane part: FP8 bytes, or 8 values
// widened to 16 bits.
template <int kOut, bool kE5M2>
__device__ __forceinline__ v4u out16(const uint8_t* stage, int c, int part, typename OutStage<kOut>::Nib nib,
                                     uint32_t m, uint32_t smask, uint32_t mmask, float scale) {
    if constexpr (kOut == kOutFp8)
        return combine(staged16(stage, c, part), nib, m, smask, mmask);
    else
        return widen8<kOut, kE5M2>(combine8(staged8(stage, c, part), nib, m, smask, mmask), scale);
}

// One phase's output: every chunk's 128 staged exponents with their nibbles
// (requested into nb before the phase's decode), as FP8 bytes or widened
// 16-bit values. A whole block in one pass stores every part unchecked and
// non-temporal; otherwise only the pass's chunks and the tensor's values.
template <int kOut, bool kE5M2>
__device__ __forceinline__ void store_phase(const Args& a, const uint8_t* stage,
                                            const typename OutStage<kOut>::Nib* nb, uint64_t v0, uint32_t nvals,
                                            int ph, bool whole, int l0, int l1, int lane, uint32_t m,
                                            uint32_t smask, uint32_t mmask) {
    using S = OutStage<kOut>;
    if (whole) {
#pragma unroll
        for (int rr = 0; rr < S::kRounds; ++rr) {
            const int c = rr * (kLanes / S::kPartLanes) + (lane >> S::kPartShift), part = lane & (S::kPartLanes - 1);
            const v4u o = out16<kOut, kE5M2>(stage, c, part, nb[rr], m, smask, mmask, a.scale);
            __builtin_nontemporal_store(o, reinterpret_cast<v4u*>(a.out + (v0 + uint64_t(c) * kChunk +
                                                                           uint64_t(ph * kPhase + part * S::kVals)) *
                                                                              S::kOutBytes));
        }
    } else {
#pragma unroll
        for (int rr = 0; rr < S::kRounds; ++rr) {
            const int c = rr * (kLanes / S::kPartLanes) + (lane >> S::kPartShift), part = lane & (S::kPartLanes - 1);
            const uint32_t v = uint32_t(c * kChunk + ph * kPhase + part * S::kVals);
            if (c < l0 || c >= l1 || v >= nvals) continue;
            const v4u o = out16<kOut, kE5M2>(stage, c, part, nb[rr], m, smask, mmask, a.scale);
            uint8_t* dst = a.out + (v0 + v) * S::kOutBytes;
            if (v + S::kVals <= nvals) {
                *reinterpret_cast<v4u*>(dst) = o;
            } else {
                for (uint32_t i = 0; i < (nvals - v) * S::kOutBytes; ++i) {
                    const uint32_t wd = i < 4 ? o.x : i < 8 ? o.y : i < 12 ? o.z : o.w;
                    dst[i] = uint8_t(wd >> (8 * (i & 3)));
                }
            }
        }
    }
}

template <int kOut>
__global__ __launch_bounds__(kThreads) void e8huf_decode_kernel(Args a) {
    using S = OutStage<kOut>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsStatic];
    __shared__ uint32_t local_ticket;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    uint32_t* tab = reinterpret_cast<uint32_t*>(lds);
    uint16_t* l2 = reinterpret_cast<uint16_t*>(lds_dyn);
    uint8_t* lenof = lds + kLenOff;   // code length per exponent value

    // header: must describe this call, and its planes must lie in the blob
    const uint8_t* b = a.blob;
    const uint32_t w1 = ld32(b + 4);
    const uint32_t exp_bits = (w1 >> 16) & 0xFFu;
    const uint64_t n_bits = ld64(b + 32), bits_off = ld64(b + 40), nib_off = ld64(b + 48);
    const uint32_t n_blocks = ld32(b + 24);
    const uint64_t nib_end = nib_off + (((a.n + 1) / 2 + 15) & ~15ull);
    const uint32_t hdr_ok =
        bit(ld32(b) == 0x46483845u /* "E8HF" */) & bit((w1 & 0xFFFFu) == 1u) & bit(exp_bits == 4u || exp_bits == 5u) &
        bit((w1 >> 24) == uint32_t(E8HUF_MAXLEN)) & bit(ld64(b + 8) == a.n) & bit(ld32(b + 16) == E8HUF_BLOCK_VALUES) &
        bit(ld32(b + 20) == E8HUF_LANE_VALUES) & bit(uint64_t(n_blocks) == (a.n + E8HUF_BLOCK_VALUES - 1) / E8HUF_BLOCK_VALUES) &
        bit(n_bits <= uint64_t(E8HUF_MAXLEN) * a.n) & bit((bits_off & 15) == 0) & bit((nib_off & 15) == 0) &
        bit(bits_off >= E8HUF_HDR_BYTES + uint64_t(E8HUF_BLOCK_REC_BYTES) * n_blocks) &
        bit(nib_off >= bits_off + (n_bits + 7) / 8) & bit(nib_off < a.blob_bytes) & bit(nib_end <= a.blob_bytes);
    if (!hdr_ok) {
        if (blockIdx.x == 0 && threadIdx.x == 0) flag(a.status, E8HUF_DEV_HEADER);
        return;
    }
    const uint32_t m = 7u - exp_bits;
    const uint32_t smask = 0x80808080u, mmask = ((1u << m) - 1u) * 0x01010101u;

    // the two-level table and the code lengths into LDS, then the 12-bit table
    // (the launcher sized the dynamic region to exactly lut_entries entries;
    // second-level indices are clamped to the last of them)
    const uint32_t l2_last = a.lut_entries - 1u;
    for (uint32_t i = threadIdx.x; i < a.lut_entries; i += kThreads) l2[i] = a.lut[i];
    if (threadIdx.x < 32) lenof[threadIdx.x] = b[64 + threadIdx.x];
    if (threadIdx.x == 0) local_ticket = 0u;
    __syncthreads();
    constexpr int kPer = (kTabEntries + kThreads - 1) / kThreads;
    uint32_t ent[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const uint32_t i = threadIdx.x + uint32_t(q) * kThreads;
        ent[q] = i < uint32_t(kTabEntries) ? make_entry(l2, l2_last, i, m) : 0u;
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const uint32_t i = threadIdx.x + uint32_t(q) * kThreads;
        if (i < uint32_t(kTabEntries)) tab[i] = ent[q];
    }
    __syncthreads();

    const int lane = int(threadIdx.x & 63);
    const uint32_t wave = uniform(threadIdx.x >> 6);
    uint8_t* wl = lds + kWaveOff + wave * kWaveLds;
    uint32_t* buf = reinterpret_cast<uint32_t*>(wl);
    uint8_t* stage = wl + kBufBytes;
    const uint8_t* bits = b + bits_off;
    const uint8_t* nib = b + nib_off;
    // last readable 16-byte unit (dword index from `bits`): reads stop inside
    // the padded nibble plane, which the header check keeps in the blob
    const int64_t dmax = int64_t(((nib_end - bits_off - 16) >> 2) & ~3ull);
    const uint32_t G = gridDim.x;
    uint32_t h = wave * G + blockIdx.x;   // position; block n_blocks - 1 - h

    while (h < n_blocks) {
        const uint32_t blk = n_blocks - 1u - h;
        const uint8_t* rec = b + E8HUF_HDR_BYTES + uint64_t(E8HUF_BLOCK_REC_BYTES) * blk;
        const uint64_t start = ld64(rec);
        const uint64_t next = blk + 1u < n_blocks ? ld64(rec + E8HUF_BLOCK_REC_BYTES) : n_bits;
        const uint32_t lb = reinterpret_cast<const uint16_t*>(rec + 8)[lane];
        const uint64_t v0 = uint64_t(blk) * E8HUF_BLOCK_VALUES;
        const uint32_t nvals = uint32_t(min(uint64_t(E8HUF_BLOCK_VALUES), a.n - v0));
        const int lane_cnt = min(max(int(nvals) - lane * kChunk, 0), kChunk);
        const uint32_t incl = wave_incl_scan(lb);
        const uint32_t total = lane_value(incl, 63);
        const bool lane_ok = lb >= uint32_t(lane_cnt) && lb <= uint32_t(lane_cnt) * E8HUF_MAXLEN;
        const bool blk_ok = start <= n_bits && start + total == next && next <= n_bits;
        if (!blk_ok || __any(!lane_ok)) {
            if (lane == 0) flag(a.status, E8HUF_DEV_INDEX);
        } else {
            const uint64_t lane_start = start + incl - lb, lane_end = start + incl;
            const bool full = nvals == E8HUF_BLOCK_VALUES;
            uint32_t bad = 0, end_bad = 0;
            // passes over consecutive lane ranges whose codes fit the buffer
            // (one pass unless the block's codes exceed it)
            for (int l0 = 0; l0 < kLanes;) {
                const int64_t j0 = ((int64_t(__builtin_amdgcn_readlane(uint32_t(lane_start), l0)) |
                                     (int64_t(__builtin_amdgcn_readlane(uint32_t(lane_start >> 32), l0)) << 32)) - 1) >> 5 & ~3ll;
                const int64_t my_end = ((int64_t(lane_end) - 1) >> 5) + 6 & ~3ll;
                const bool over = lane >= l0 && (my_end - j0) * 4 > kBufBytes;
                const uint64_t ovm = __ballot(over);
                const int l1 = ovm ? int(__builtin_ctzll(ovm)) : kLanes;   // > l0: one chunk always fits
                const uint32_t lhi = uint32_t(lane_value(uint32_t(my_end), uint32_t(l1 - 1)));
                const uint32_t hhi = uint32_t(lane_value(uint32_t(uint64_t(my_end) >> 32), uint32_t(l1 - 1)));
                const int64_t end_all = int64_t((uint64_t(hhi) << 32) | lhi);
                const int units = int((end_all - j0) / 4);
                const bool mine = lane >= l0 && lane < l1;
                // copy dwords [j0, j0 + 4 units) into the buffer, byte-swapped
                {
                    constexpr int kPerL = kBufUnits / kLanes;
                    uint4 v[kPerL];
#pragma unroll
                    for (int i = 0; i < kPerL; ++i) {
                        const int u = min(lane + kLanes * i, units - 1);
                        const int64_t j = min(j0 + 4 * int64_t(u), dmax);
                        v[i] = *reinterpret_cast<const uint4*>(bits + 4 * j);
                    }
#pragma unroll
                    for (int i = 0; i < kPerL; ++i)
                        reinterpret_cast<uint4*>(buf)[lane + kLanes * i] =
                            make_uint4(bswap32(v[i].x), bswap32(v[i].y), bswap32(v[i].z), bswap32(v[i].w));
                    wave_sync();
                }
                const uint32_t my_cnt = mine ? uint32_t(lane_cnt) : 0u;
                // lanes outside the pass keep their windows at the buffer start
                Lane ls = {mine ? uint32_t(lane_start - uint64_t(32 * j0) - 1) : 0u, 0u, 0u, m};
                const uint32_t pm1_0 = ls.pm1;
                uint8_t* row = stage + lane * kStageStride;
#pragma unroll 1
                for (int ph = 0; ph < kPhases; ++ph) {
                    const uint32_t base = uint32_t(ph * kPhase);
                    // the phase's nibbles, requested before its decode so that
                    // the loads overlap it
                    typename S::Nib nb[S::kRounds];
#pragma unroll
                    for (int rr = 0; rr < S::kRounds; ++rr) {
                        const uint32_t v = uint32_t((rr * (kLanes / S::kPartLanes) + (lane >> S::kPartShift)) * kChunk +
                                                    ph * kPhase + (lane & (S::kPartLanes - 1)) * S::kVals);
                        const uint64_t at = v < nvals ? (v0 + v) / 2 : 0ull;
                        nb[rr] = *reinterpret_cast<const typename S::Nib*>(nib + at);
                    }
                    decode_phase(tab, l2, l2_last, buf, row, min(base + kPhase, my_cnt), base, ls);
                    wave_sync();
                    const bool whole = full && l0 == 0 && l1 == kLanes;
                    if constexpr (kOut == kOutFp8) {
                        if (whole) {
#pragma unroll
                            for (int rr = 0; rr < S::kRounds; ++rr) {
                                const int c = rr * (kLanes / S::kPartLanes) + (lane >> S::kPartShift),
                                          part = lane & (S::kPartLanes - 1);
                                const v4u o = combine(staged16(stage, c, part), nb[rr], m, smask, mmask);
                                __builtin_nontemporal_store(o, reinterpret_cast<v4u*>(a.out + v0 + uint64_t(c) * kChunk +
                                                                                       uint64_t(ph * kPhase + part * 16)));
                            }
                        } else {
#pragma unroll
                            for (int rr = 0; rr < S::kRounds; ++rr) {
                                const int c = rr * (kLanes / S::kPartLanes) + (lane >> S::kPartShift),
                                          part = lane & (S::kPartLanes - 1);
                                const uint32_t v = uint32_t(c * kChunk + ph * kPhase + part * 16);
                                if (c < l0 || c >= l1 || v >= nvals) continue;
                                const v4u o = combine(staged16(stage, c, part), nb[rr], m, smask, mmask);
                                uint8_t* dst = a.out + v0 + v;
                                if (v + 16 <= nvals) {
                                    *reinterpret_cast<v4u*>(dst) = o;
                                } else {
                                    for (uint32_t i = 0; i < nvals - v; ++i) {
                                        const uint32_t wd = i < 4 ? o.x : i < 8 ? o.y : i < 12 ? o.z : o.w;
                                        dst[i] = uint8_t(wd >> (8 * (i & 3)));
                                    }
                                }
                            }
                        }
                    } else if (exp_bits == 5u)
                        store_phase<kOut, true>(a, stage, nb, v0, nvals, ph, whole, l0, l1, lane, m, smask, mmask);
                    else
                        store_phase<kOut, false>(a, stage, nb, v0, nvals, ph, whole, l0, l1, lane, m, smask, mmask);
                    wave_sync();
                }
                // the last lookup may have taken symbols past the lane's
                // count; their bits are not the lane's
                // (they sit in the row right after its last symbol)
                uint32_t used = ls.pm1 - pm1_0;
                if (my_cnt) {
                    const uint8_t* over = row + (my_cnt - (my_cnt - 1u) / kPhase * kPhase);
                    for (uint32_t j = 0; j < 2u && my_cnt + j < ls.cnt; ++j) used -= lenof[(over[j] >> m) & 31u];
                }
                bad |= mine ? (ls.bad & kBadE) : 0u;
                end_bad |= bit(mine && used != lb);
                l0 = l1;
            }
            // one status update per wave (every lane takes part in the votes)
            const bool any_bad = __any(bad != 0), any_end = __any(end_bad != 0);
            if (lane == 0 && any_bad) flag(a.status, E8HUF_DEV_CODE);
            if (lane == 0 && any_end) flag(a.status, E8HUF_DEV_LANE_END);
        }
        uint32_t ticket = 0;
        if (lane == 0) ticket = atomicAdd(&local_ticket, 1u);
        h = uniform(blockIdx.x + G * (kWaves + lane_value(ticket, 0)));
    }
}

std::mutex g_mu;
std::vector<int> g_cus;   // per device

int device_cus(int* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return K3HUF_E_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (int(g_cus.size()) <= dev) g_cus.resize(dev + 1, 0);
    if (!g_cus[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return K3HUF_E_HIP;
        g_cus[dev] = cus;
    }
    *out = g_cus[dev];
    return K3HUF_OK;
}

// Argument checks and the launch shared by both entry points.
template <int kOut>
int launch(const void* d_blob, size_t blob_bytes, const uint16_t* d_lut, int lut_entries, void* d_out,
           uint64_t n_values, float scale, void* stream, uint32_t* d_status) {
    if (!d_blob || !d_lut || !d_out) return K3HUF_E_ARG;
    if ((reinterpret_cast<uintptr_t>(d_blob) & 15) || (reinterpret_cast<uintptr_t>(d_out) & 15) ||
        (reinterpret_cast<uintptr_t>(d_lut) & 1) || (reinterpret_cast<uintptr_t>(d_status) & 3))
        return K3HUF_E_ARG;
    if (n_values == 0 || n_values > (1ull << 40) || blob_bytes < E8HUF_HDR_BYTES + E8HUF_BLOCK_REC_BYTES ||
        uint64_t(blob_bytes) >= (1ull << 44))
        return K3HUF_E_ARG;
    if (lut_entries < 256 || lut_entries > E8HUF_LUT_MAX || lut_entries % 256) return K3HUF_E_ARG;
    int cus = 0;
    int rc = device_cus(&cus);
    if (rc) return rc;
    const uint64_t blocks = (n_values + E8HUF_BLOCK_VALUES - 1) / E8HUF_BLOCK_VALUES;
    // one workgroup per CU (each takes most of its LDS), or one per block for
    // a tensor of fewer blocks than CUs
    const unsigned grid = unsigned(blocks < uint64_t(cus) ? blocks : uint64_t(cus));
    Args a;
    a.blob = static_cast<const uint8_t*>(d_blob);
    a.blob_bytes = blob_bytes;
    a.lut = d_lut;
    a.lut_entries = uint32_t(lut_entries);
    a.out = static_cast<uint8_t*>(d_out);
    a.n = n_values;
    a.status = d_status;
    a.scale = scale;
    hipLaunchKernelGGL(e8huf_decode_kernel<kOut>, dim3(grid), dim3(kThreads), size_t(lut_entries) * 2,
                       static_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? K3HUF_OK : K3HUF_E_HIP;
}

}  // namespace

extern "C" {

int e8huf_decode(const void* d_blob, size_t blob_bytes, const uint16_t* d_lut, int lut_entries, void* d_out,
                 uint64_t n_values, void* stream, uint32_t* d_status) {
    return launch<kOutFp8>(d_blob, blob_bytes, d_lut, lut_entries, d_out, n_values, 1.0f, stream, d_status);
}

int e8huf_decode_widen(const void* d_blob, size_t blob_bytes, const uint16_t* d_lut, int lut_entries, void* d_out,
                       uint64_t n_values, int out_kind, float scale, void* stream, uint32_t* d_status) {
    if (out_kind == E8HUF_OUT_BF16)
        return launch<E8HUF_OUT_BF16>(d_blob, blob_bytes, d_lut, lut_entries, d_out, n_values, scale, stream, d_status);
    if (out_kind == E8HUF_OUT_F16)
        return launch<E8HUF_OUT_F16>(d_blob, blob_bytes, d_lut, lut_entries, d_out, n_values, scale, stream, d_status);
    return K3HUF_E_ARG;
}

}  // extern "C"
