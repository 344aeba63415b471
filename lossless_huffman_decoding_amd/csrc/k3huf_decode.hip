// gfx950 decode path of the k3huf library: the decode kernel, its launcher
// and the layer-ring drivers (device-resident and host-fed containers).
// Container layout: include/k3huf.h.
//
// What is computed (K3 page = "Kimi K3 纯 CPU 推理中的无损 Trunk 压缩…",
// yfxerp.com/news/153994):
//   - "decode loop": a bit window whose top holds the head of the stream;
//     one lookup of the top 12 bits in the 4096-entry table gives the symbol
//     and its code length, and the window shifts by that length;
//   - "key design points": each decoded symbol is the high byte at an odd
//     offset; the raw even-plane byte goes back at the even offset before it.
// How it is laid out on the GPU (not from the pages): one wave decodes one
// half subblock (32 KiB of output, or 8 KiB in the layout of 64-symbol lane
// chunks); lane t decodes its lane chunk t (256 or 64 symbols, as the layer
// header says) starting at the bit offset the subblock index gives it (the ECF8
// page, section 2.1, keeps such per-thread bit offsets beside its code); the
// table lives in LDS; decoded bytes are staged in LDS so that the even-plane
// loads and the output stores of a wave cover whole 128-byte lines.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "k3huf.h"
#include "k3huf_bounds.h"

namespace {

// One 7-wave workgroup per CU (measured on the trunk layer: 7 waves per CU
// ran 6% faster than 12, and 6, 8, 9 or 10 were in between; 4 or 5 cannot
// hide the table lookups' latency). A work unit is half a subblock: 64 lane
// chunks of L symbols (256, or 64 for small layers), lane t decoding chunk t
// in L / 64 phases of 64 symbols. Every HBM line is read or written in one
// burst:
//   - the unit's bitstream is copied into the wave's LDS buffer with
//     coalesced 16-byte loads before its lanes decode (when a full unit's
//     codes exceed the buffer, each lane gathers its own codes phase by
//     phase instead; the layer's partial last unit is decoded in passes over
//     consecutive lane ranges);
//   - the even-plane bytes of two of a unit's phases (two whole 128-byte
//     lines per 256-symbol chunk) are requested together into registers
//     before the first of them (all four phases' at once on the gather
//     path; two at a time measured 5% faster on the 256 MiB heavy layer,
//     whose first round starts every wave's loads at once, and the same on
//     the trunk layer, but 3% slower on units that gather their codes);
//   - each phase's 64 symbols per chunk are staged in LDS, so every output
//     store instruction writes whole 128-byte lines.
constexpr int kWaves = 7;
constexpr int kThreads = 64 * kWaves;
constexpr int kUnitLanes = 64;                        // lane chunks per work unit
constexpr int kUnitsPerSub = K3HUF_LANES / kUnitLanes;   // 2
constexpr int kPhase = 64;                            // symbols per lane per phase
constexpr int kGroups = kPhase / 4;                   // 4-symbol groups per phase (tail path)
constexpr int kRounds = 64 / 8;                       // write-out rounds (8 chunks each)
constexpr int kBufBytes = 7680;                       // per-wave bitstream buffer
constexpr int kBufUnits = kBufBytes / 16;
// LDS bytes per chunk per phase: the phase's 64 symbols, then room for the
// bytes a lane writes past them (one symbol of the next phase, one unused)
constexpr int kStageStride = kPhase + 4;
constexpr int kWaveLds = kBufBytes + 64 * kStageStride;
// table lookups per bit window: each consumes at most 12 bits, five fit in 64
constexpr int kLookups = 5;
// bit windows per phase: every lookup yields a symbol, so 64 lookups always
// finish a phase
constexpr int kMaxWindows = (kPhase + kLookups - 1) / kLookups;
constexpr int kTabBytes = K3HUF_LUT_ENTRIES * 4;
constexpr int kLdsBytes = kTabBytes + kWaves * kWaveLds;
static_assert(kLdsBytes <= 163840, "LDS budget");

// Lane-chunk geometry of a layer: L symbols per lane chunk (K3HUF_LANE_SYMS,
// or K3HUF_LANE_SYMS_SHORT in the layout for small layers); a subblock holds
// K3HUF_LANES chunks, a work unit half of them, and a lane decodes its chunk
// in L / 64 phases.
template <uint32_t L>
struct Geo {
    static constexpr int kUnitSyms = kUnitLanes * int(L);                 // 16384 or 4096
    static constexpr int kPhases = int(L) / kPhase;                       // 4 or 1
    // phases per even-plane prefetch: two when the unit's codes are in the
    // buffer, all four on the gather path
    static constexpr int kSuperFill = kPhases < 2 ? kPhases : 2;
    static constexpr int kSuperGather = kPhases < 4 ? kPhases : 4;
    static constexpr uint32_t kSubSyms = K3HUF_LANES * L;                 // 32768 or 8192
    static constexpr uint32_t kSubBytes = 2 * kSubSyms;
    static constexpr uint32_t kSubPerStripe = K3HUF_STRIPE_BYTES / kSubBytes;   // 1024 or 4096
};

// LDS decode table, derived per workgroup from the 4096-entry
// (symbol << 4 | length) table: one lookup of the top 12 window bits yields
// the first code and, when the next code also lies inside those 12 bits, the
// second one too (the "double-symbol table" the K3 page names under "if
// revisited"; the container format is unchanged). A lookup thus yields one
// or two symbols; no entry is zero.
//   [7:0]   first symbol
//   [11:8]  bits consumed by the entry's symbols (T, 1..12)
//   [13:12] symbols in the entry (1 or 2)
//   [14]    index no code covers (decoded as one 12-bit code)
//   [23:16] second symbol (zero if the entry holds one)
//   [27:24] length of the first code
constexpr uint32_t kBad = 1u << 14;
__device__ __forceinline__ uint32_t ent_bits(uint32_t e) { return (e >> 8) & 15u; }
__device__ __forceinline__ uint32_t ent_syms(uint32_t e) { return (e >> 12) & 3u; }
__device__ __forceinline__ uint32_t ent_len1(uint32_t e) { return (e >> 24) & 15u; }

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Work distribution. Units are handed out in descending order: position p
// (0, 1, ...) stands for unit n - 1 - p, so the layer's last unit, the only
// one that can be partial (and decoded by the slower tail path), starts
// first. With T waves in the grid, wave slot v of workgroup b takes position
// v * blocks + b first (consecutive positions on different CUs, so a small
// layer spreads over the chip). Every later position is handed out on
// demand: position T + x + G i goes to whichever wave of workgroup group x
// (block mod G, G = min(4, blocks): workgroup b runs on XCD b mod 8, so a
// group spans two XCDs) takes ticket i from group x's counter. Four groups
// measured best on the trunk layer (1.4% faster than one per XCD, which lets
// one slow XCD finish late; two groups 0.5%; a single counter 27% slower, its
// atomics queueing). On-demand handout is needed because the waves of a CU
// do not progress at one rate: a SIMD issues from its oldest wave first (with
// three waves per SIMD the first ran about 1.5 times as fast as the third),
// and over many rounds the static order leaves some waves far behind. A
// wave asks for its next position halfway through its current unit, and
// reads the answer (and requests that unit's record) as its last phase
// starts, so it holds at most a quarter unit of work ahead and the grid's
// waves finish within about one unit's time of each other. Each counter has
// a 256-byte line to itself: atomics on one line are serialised, and eight
// counters sharing a line delayed the tickets enough to stall every unit.
// The counters live in this array, which exists once per device for the
// life of the process, in kSchedSlots slots; the last workgroup of a launch
// clears its slot. The first kSchedSlots streams of a device each get a slot
// of their own on first use: launches on one stream never overlap, so they
// can share it. Two launches running at the same time on one slot would take
// each other's tickets and leave units undecoded, so a launch that cannot
// have a slot to itself uses no device counter: launches on later streams,
// and launches captured into a graph (a graph may be replayed on any stream,
// beside a decode on the one it was captured on), keep each workgroup to its
// own share of positions (b, b + blocks, b + 2 blocks, ...) and hand that
// share to its waves from a counter in the workgroup's LDS, which shares
// nothing. That evens out the waves of a CU but not the CUs: on the trunk
// layer it takes 1.048 times as long as the device counters (every position
// handed out statically: 1.089 times). Layers of at most kDynRounds rounds of
// units take the workgroup counters too, as they are as fast there.
constexpr uint32_t kSchedSlots = 256;
constexpr uint32_t kDynRounds = 5;   // device counters only for layers of more rounds of units than this
constexpr uint32_t kGroupsPerSlot = 4;
constexpr uint32_t kCounterStride = 64;                               // words: one 256-byte line
constexpr uint32_t kSlotWords = (kGroupsPerSlot + 1) * kCounterStride;  // tickets per group, workgroups done
__device__ __attribute__((aligned(256))) uint32_t g_sched[kSlotWords * kSchedSlots];

struct DecodeArgs {
    const uint8_t* blob;
    uint64_t blob_bytes;
    const uint16_t* lut;
    uint8_t* out;
    uint64_t out_bytes;
    uint32_t n_stripes;
    uint32_t* status;
    uint32_t slot;        // work-counter slot of this launch (when dyn)
    uint32_t dyn;         // positions after the first round: 1 from the slot's counters, 0 from the workgroup's
};

__device__ __forceinline__ uint32_t ld32(const uint8_t* p) {
    return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ uint64_t ld64(const uint8_t* p) {
    return *reinterpret_cast<const uint64_t*>(p);
}
__device__ __forceinline__ uint32_t bswap32(uint32_t x) {
    return __builtin_amdgcn_perm(0u, x, 0x00010203u);
}
__device__ __forceinline__ void flag(uint32_t* status, uint32_t bit) {
    if (status) atomicOr(status, bit);
}
// a test's outcome as a bit, for checks combined with `&` so that every
// operand (and its load) is evaluated without branches
__device__ __forceinline__ uint32_t bit(bool c) { return c ? 1u : 0u; }
__device__ __forceinline__ uint32_t uniform(uint32_t x) {
    return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}
// Inclusive prefix sum over the 64 lanes with DPP row moves: a scan within
// each 16-lane row (shifts 1, 2, 4, 8, zero fill), then the last lane of
// row 0 added into row 1 and of row 2 into row 3, then lane 31 into rows 2-3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);    // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);    // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);    // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);    // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return x;
}
// s_waitcnt vmcnt(0), the other counters left alone. Placed where the
// counter is about to be drained anyway, it tells the compiler's wait
// analysis that nothing is outstanding there; without it, merging paths
// (the multi-pass decode, a record loaded without prefetch) makes the
// compiler wait for every outstanding store at later loop heads.
__device__ __forceinline__ void drain_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ uint32_t lane_value(uint32_t v, uint32_t l) {
    return __builtin_amdgcn_readlane(v, l);
}

// Table entry for 12-bit index i from two words of the (symbol << 4 |
// length) table: a = lut[i] and, when a's length l is 1..11, the entry of the
// code that follows, b = lut[(i << l) & 0xFFF] (else b = 0).
__device__ __forceinline__ uint32_t make_entry(uint32_t a, uint32_t b) {
    const uint32_t l1 = a & 15u;
    if (l1 == 0 || l1 > K3HUF_MAXLEN) return kBad | (12u << 24) | (1u << 12) | (12u << 8);
    const uint32_t e = (l1 << 24) | (1u << 12) | (l1 << 8) | ((a >> 4) & 0xFFu);
    const uint32_t l2 = b & 15u;
    if (l1 < K3HUF_MAXLEN && l2 && l1 + l2 <= K3HUF_MAXLEN)
        return e + (((b >> 4) & 0xFFu) << 16) + (1u << 12) + (l2 << 8);
    return e;
}
// index of the second word make_entry needs for index i, or -1
__device__ __forceinline__ int second_index(uint32_t i, uint32_t a) {
    const uint32_t l1 = a & 15u;
    return l1 != 0 && l1 < K3HUF_MAXLEN ? int((i << l1) & 0xFFFu) : -1;
}

__device__ __forceinline__ uint32_t peek(const uint32_t* tab, uint64_t acc) {
    return tab[uint32_t(acc >> 52)];
}

// 64-bit window whose top bit is the bit after buffer bit pm1: buffer dwords
// q..q+2 (q = pm1 / 32, held byte-swapped), shifted right by 31 - pm1 mod 32.
__device__ __forceinline__ uint64_t window(const uint32_t* buf, uint32_t pm1) {
    const uint32_t* p = buf + (pm1 >> 5);
    const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
    const uint32_t r = ~pm1;
    return (uint64_t(__builtin_amdgcn_alignbit(d0, d1, r)) << 32) |
           __builtin_amdgcn_alignbit(d1, d2, r);
}

// the 8 staged symbols (2 dwords) of chunk c at phase offset 8 part
__device__ __forceinline__ uint2 staged8(const uint8_t* stage, int c, int part) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(stage + c * kStageStride + part * 8);
    return make_uint2(p[0], p[1]);
}

struct Unit {
    const uint8_t* bits;   // stripe bitstream
    const uint8_t* even;   // this unit's even-plane bytes
    uint8_t* out;          // this unit's output bytes
    int dmax;              // last readable 16-byte unit (dwords from `bits`, within the stripe)
    uint32_t nsyms;        // symbols in this unit (64 L unless last in stripe)
};

// Per-lane decode state across the phases of a unit.
struct LaneState {
    uint32_t pm1;    // buffer bit index of the next code, minus one
    uint32_t cnt;    // symbols decoded in this unit (may pass the end by one)
    uint32_t last;   // the last table entry taken
    uint32_t bad;    // OR of all entries taken
    uint32_t abs;    // gather path: stripe bit index of the lane's next code
};

// Gather path, for a unit whose codes exceed the buffer: before each phase,
// every lane copies the codes it can need into its own slot of the buffer.
// A phase takes at most 65 table entries of at most 12 bits (780 bits); the
// slot starts at the 8-byte boundary at or before the bit preceding the
// lane's next code (its index in the slot, pm1, is at most 63), and a window
// reads two dwords past the one holding bit pm1 + 1: at most dword
// (63 + 780) / 32 + 2 = 28, so 29 dwords.
constexpr int kSlotDw = 30;
static_assert(64 * kSlotDw * 4 <= kBufBytes, "gather slots fit the buffer");

// Decode one phase of a lane: symbols [64 ph, 64 ph + 64) of its chunk into
// its stage row. Each 64-bit window feeds kLookups table lookups; each
// lookup yields one or two symbols, written as two bytes at the lane's count
// (a second byte past the entry's symbols is overwritten by the next lookup
// or lands past the phase). A lane that has its 64 symbols takes zero entries
// (no bits, no symbols) until the wave's slowest lane is done. A lookup that
// ends one symbol past the phase leaves that symbol at row offset 64; it is
// moved to offset 0 when the next phase starts. A wave's LDS operations run
// in order, so each lookup's writes are issued after the next lookup's table
// read, which then waits for no write; the lane mask enters through the
// field width of the length extraction (zero for a finished lane), so the
// dependent chain from one table read to the next is four ALU operations
// (measured on one wave per CU: 4% less time per unit).
__device__ __forceinline__ void decode_phase(const uint32_t* tab, const uint32_t* buf, uint8_t* row,
                                             int ph, LaneState& ls) {
    const uint32_t base = uint32_t(ph * kPhase), target = base + kPhase;
    if (ls.cnt > base) row[0] = uint8_t(ls.last >> 16);   // carried symbol
    // each lookup's two bytes are written after the next table read has been
    // issued, so that read does not queue behind them; the first pending
    // write is a dummy past the phase
    uint8_t* wp = row + kPhase + 2;
    uint32_t we = 0;
#pragma unroll 1
    for (int w = 0; w < kMaxWindows; ++w) {
        if (!__any(ls.cnt < target)) break;
        uint64_t acc = window(buf, ls.pm1);
#pragma unroll
        for (int i = 0; i < kLookups; ++i) {
            const uint32_t e = peek(tab, acc);
            wp[0] = uint8_t(we);
            wp[1] = uint8_t(we >> 16);
            const bool live = ls.cnt < target;
            const uint32_t t = __builtin_amdgcn_ubfe(e, 8u, live ? 4u : 0u);
            const uint32_t ez = live ? e : 0u;
            wp = row + (ls.cnt - base);
            we = ez;
            ls.last = ez ? ez : ls.last;
            ls.bad |= ez;
            ls.cnt += ent_syms(ez);
            ls.pm1 += t;
            acc <<= t;
        }
    }
    wp[0] = uint8_t(we);
    wp[1] = uint8_t(we >> 16);
}

// One super-phase (kSuper phases from sp) of a full unit (64 chunks of 256
// symbols, lane t decoding chunk t). The unit's codes are either in `buf`
// (kGather false: the caller copied them there) or gathered per lane and
// phase (kGather true). Loads and stores carry no per-chunk condition, so no
// store waits for the ones before it to complete (vmcnt counts stores too,
// and a store behind a branch makes the compiler wait for everything
// outstanding). `after(ph)` runs after each phase ph.
template <uint32_t L, bool kGather, class After>
__device__ __forceinline__ void decode_super(const uint32_t* tab, uint32_t* buf, uint8_t* stage,
                                             const Unit& un, int sp, int lane, LaneState& ls,
                                             After&& after) {
    constexpr int kSuper = kGather ? Geo<L>::kSuperGather : Geo<L>::kSuperFill;
    const int sub_line = lane >> 3, part = lane & 7;
    uint2 ev[kRounds][kSuper];
    // the super-phase's even-plane bytes: whole lines per chunk
#pragma unroll
    for (int rr = 0; rr < kRounds; ++rr) {
        const int c = rr * 8 + sub_line;
#pragma unroll
        for (int f = 0; f < kSuper; ++f) {
            const uint32_t u = uint32_t(c) * L + uint32_t((sp + f) * kPhase + part * 8);
            ev[rr][f] = *reinterpret_cast<const uint2*>(un.even + u);
        }
    }
#pragma unroll
    for (int q = 0; q < kSuper; ++q) {
        const int ph = sp + q;
        if (kGather) {
            // the lane's codes for this phase, into its own slot (in bounds:
            // the same clamp as fill_buffer)
            uint32_t* slot = buf + lane * kSlotDw;
            const int d0 = ((int(ls.abs) - 1) >> 5) & ~1;
            uint2 g[kSlotDw / 2];
#pragma unroll
            for (int i = 0; i < kSlotDw / 2; ++i)
                g[i] = *reinterpret_cast<const uint2*>(un.bits + k3huf_bounds::clamped_read_off(d0 + 2 * i, un.dmax));
#pragma unroll
            for (int i = 0; i < kSlotDw / 2; ++i)
                *reinterpret_cast<uint2*>(slot + 2 * i) = make_uint2(bswap32(g[i].x), bswap32(g[i].y));
            ls.pm1 = (ls.abs - 1u) - 32u * uint32_t(d0);
            const uint32_t p0 = ls.pm1;
            decode_phase(tab, slot, stage + lane * kStageStride, ph, ls);
            ls.abs += ls.pm1 - p0;
        } else {
            decode_phase(tab, buf, stage + lane * kStageStride, ph, ls);
        }
        wave_sync();
#pragma unroll
        for (int rr = 0; rr < kRounds; ++rr) {
            const int c = rr * 8 + sub_line;
            const uint2 sy = staged8(stage, c, part);
            const uint2 e = ev[rr][q];
            const uint32_t u = uint32_t(c) * L + uint32_t(ph * kPhase + part * 8);
            // the output is written once and not read back here: stream it
            // past the caches (non-temporal store)
            const v4u o = {__builtin_amdgcn_perm(sy.x, e.x, 0x05010400u),
                           __builtin_amdgcn_perm(sy.x, e.x, 0x07030602u),
                           __builtin_amdgcn_perm(sy.y, e.y, 0x05010400u),
                           __builtin_amdgcn_perm(sy.y, e.y, 0x07030602u)};
            __builtin_nontemporal_store(o, reinterpret_cast<v4u*>(un.out + 2 * u));
        }
        wave_sync();
        after(ph);
    }
}

// Decode a full unit: its super-phases, then the lane checks. With four
// phases, `mid` runs after the second phase and `late` after the third (the
// caller asks for its next unit, then learns it and requests its record);
// with one phase both run before it. kGather false: the caller has copied
// the unit's codes from stripe dword j0 on into `buf`.
template <uint32_t L, bool kGather, class Mid, class Late>
__device__ __forceinline__ void decode_unit(const DecodeArgs& a, const uint32_t* tab, uint32_t* buf,
                                            uint8_t* stage, const Unit& un, int j0,
                                            uint32_t lane_start, uint32_t lane_bits, int lane,
                                            Mid&& mid, Late&& late) {
    constexpr int kPhases = Geo<L>::kPhases, kSuper = kGather ? Geo<L>::kSuperGather : Geo<L>::kSuperFill;
    // the buffer starts at least one dword before the lane's first code, so
    // pm1 >= 0
    LaneState ls = {lane_start - 32u * uint32_t(j0) - 1u, 0u, 0u, 0u, lane_start};
    const uint32_t pm1_0 = ls.pm1;
    if (kPhases == 1) {
        mid();
        late();
    }
#pragma unroll 1
    for (int sp = 0; sp < kPhases; sp += kSuper) {
        decode_super<L, kGather>(tab, buf, stage, un, sp, lane, ls, [&](int ph) {
            if (kPhases > 1 && ph == 1) mid();
            if (kPhases > 1 && ph == 2) late();
        });
    }
    // a last lookup that ran one symbol past the chunk took that symbol's
    // bits too
    uint32_t used = kGather ? ls.abs - lane_start : ls.pm1 - pm1_0;
    if (ls.cnt > L) used -= ent_bits(ls.last) - ent_len1(ls.last);
    // one status update per wave (a corrupt layer would otherwise send an
    // atomic per lane to the one status word)
    const bool code_bad = __any((ls.bad & kBad) != 0u), end_bad = __any(used != lane_bits);
    if (lane == 0 && code_bad) flag(a.status, K3HUF_DEV_CODE);
    if (lane == 0 && end_bad) flag(a.status, K3HUF_DEV_LANE_END);
}

// The same for the layer's last unit when it holds fewer than 64 L symbols:
// lane t decodes clamp(nsyms - L t, 0, L) symbols one code per table step;
// kept plain (it runs at most once per layer).
template <uint32_t L>
__device__ __forceinline__ void decode_lanes_tail(const DecodeArgs& a, const uint32_t* tab,
                                                  const uint32_t* buf, uint8_t* stage, const Unit& un,
                                                  int j0, uint32_t lane_start, uint32_t lane_bits,
                                                  int l0, int l1, int lane) {
    const bool mine = lane >= l0 && lane < l1;
    constexpr int kPhases = Geo<L>::kPhases;
    const int lane_cnt = min(max(int(un.nsyms) - lane * int(L), 0), int(L));
    uint32_t pm1 = lane_start - 32u * uint32_t(j0) - 1u;
    const uint32_t pm1_0 = pm1;
    uint32_t bad = 0;
    const int sub_line = lane >> 3, part = lane & 7;
    uint32_t* row = reinterpret_cast<uint32_t*>(stage + lane * kStageStride);
#pragma unroll 1
    for (int ph = 0; ph < kPhases; ++ph) {
        // phases and groups past every lane's symbols are skipped (the
        // wave's lanes agree on each test)
        if (!__any(mine && ph * kPhase < lane_cnt)) break;
        if (mine) {
#pragma unroll 1
            for (int g = 0; g < kGroups; ++g) {
                if (!__any(ph * kPhase + g * 4 < lane_cnt)) break;
                uint64_t acc = window(buf, pm1);
                uint32_t ww = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t e = peek(tab, acc);
                    const bool live = ph * kPhase + g * 4 + t < lane_cnt;
                    const uint32_t l = live ? ent_len1(e) : 0u;
                    if (live) bad |= e;
                    acc <<= l;
                    pm1 += l;
                    // the entry's first symbol into byte t of ww
                    constexpr uint32_t sel[4] = {0x03020104u, 0x03020400u, 0x03040100u, 0x04020100u};
                    ww = __builtin_amdgcn_perm(e, ww, sel[t]);
                }
                row[g] = ww;
            }
        }
        wave_sync();
#pragma unroll 1
        for (int rr = 0; rr < kRounds; ++rr) {
            const int c = rr * 8 + sub_line;
            const uint32_t u = uint32_t(c) * L + uint32_t(ph * kPhase + part * 8);
            if (c < l0 || c >= l1 || u >= un.nsyms) continue;
            const uint2 sy = staged8(stage, c, part);
            const uint2 e = *reinterpret_cast<const uint2*>(un.even + u);
            const uint32_t m = min(un.nsyms - u, 8u);
            for (uint32_t i = 0; i < m; ++i) {
                const uint32_t e8 = i < 4 ? (e.x >> (8 * i)) : (e.y >> (8 * (i - 4)));
                const uint32_t s8 = i < 4 ? (sy.x >> (8 * i)) : (sy.y >> (8 * (i - 4)));
                *reinterpret_cast<uint16_t*>(un.out + 2 * (u + i)) = uint16_t((e8 & 0xFFu) | ((s8 & 0xFFu) << 8));
            }
        }
        wave_sync();
    }
    const bool code_bad = __any(mine && (bad & kBad)), end_bad = __any(mine && pm1 - pm1_0 != lane_bits);
    if (lane == 0 && code_bad) flag(a.status, K3HUF_DEV_CODE);
    if (lane == 0 && end_bad) flag(a.status, K3HUF_DEV_LANE_END);
}

// Copy bitstream dwords [j0, j0 + 4 * units) into `buf`, byte-swapped so
// that bit 31 of each dword is the earliest stream bit. Every slot of the
// buffer is written: slots past `units` repeat the last 16-byte unit (the
// same address, so no extra line is fetched). Keeping the loads and stores
// unconditional lets the compiler count outstanding loads exactly instead of
// waiting for all memory operations at later register reuse.
__device__ __forceinline__ void fill_buffer(uint32_t* buf, const Unit& un, int j0, int units, int lane) {
    constexpr int kPer = (kBufUnits + 63) / 64;
    uint4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int u = min(lane + 64 * i, units - 1);
        v[i] = *reinterpret_cast<const uint4*>(un.bits + k3huf_bounds::clamped_read_off(j0 + 4 * u, un.dmax));
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (kBufUnits % 64 == 0 || i < kPer - 1 || lane + 64 * i < kBufUnits)
            *reinterpret_cast<uint4*>(buf + 4 * (lane + 64 * i)) =
                make_uint4(bswap32(v[i].x), bswap32(v[i].y), bswap32(v[i].z), bswap32(v[i].w));
    wave_sync();
}

// first buffer dword for codes starting at stripe bit p: the 16-byte unit
// holding the dword before bit p
__device__ __forceinline__ int first_dword(uint32_t p) { return ((int(p) - 1) >> 5) & ~3; }
// end (exclusive, 16-byte aligned) of the dwords windows may read for codes
// ending at stripe bit p
__device__ __forceinline__ int end_dword(uint32_t p) { return (((int(p) - 1) >> 5) + 3 + 3) & ~3; }

// Stripe values of the 64 stripes 64 blk .. 64 blk + 63, lane l holding stripe
// 64 blk + l: the record offset in 16-byte units, both plane offsets and the
// bit count, or n_bits = kNoStripe where the stripe does not exist or its
// record fails the checks (bounds, geometry, n_bits <= 12 n_syms, which keeps
// valid counts below kNoStripe). Offsets below 2^36 fit the 16-byte unit
// count; the launcher rejects larger blobs.
constexpr uint32_t kNoStripe = 0xFFFFFFFFu;
struct StripeLane {
    uint32_t off16, bits_off, even_off, n_bits;
};

__device__ __forceinline__ uint64_t stripe_raw(const DecodeArgs& a, uint32_t s) {
    return min(uint64_t(K3HUF_STRIPE_BYTES), a.out_bytes - uint64_t(s) * K3HUF_STRIPE_BYTES);
}
template <uint32_t L>
__device__ __forceinline__ uint32_t stripe_subblocks(uint32_t n_syms) {
    return (n_syms + Geo<L>::kSubSyms - 1) / Geo<L>::kSubSyms;
}

// Branch-free: every lane issues its loads (a stripe that does not exist,
// or whose offset fails the checks, reads the blob's first 32 bytes instead
// and is then rejected), and every check is evaluated, so the loads of all
// lanes go out together instead of one dependent round trip per check. In
// two halves: the record offsets, then the records (a caller can issue
// other loads that need only the offsets in between).
struct StripeOff {
    uint64_t so;   // the lane's stripe record offset, or 0 where it fails the checks
    uint32_t in;   // 1 where it passes
};
__device__ __forceinline__ StripeOff stripe_offsets(const DecodeArgs& a, uint32_t blk, int lane) {
    const uint32_t s = blk * 64u + uint32_t(lane);
    const uint32_t sc = s < a.n_stripes ? s : 0u;
    const uint64_t soff = ld64(a.blob + K3HUF_HDR_BYTES + 8ull * sc);
    const uint32_t in = bit((soff & 15) == 0) & bit(soff + K3HUF_STRIPE_HDR_BYTES <= a.blob_bytes);
    return {in ? soff : 0ull, in};
}
template <uint32_t L>
__device__ __forceinline__ StripeLane stripe_values(const DecodeArgs& a, uint32_t blk, int lane, StripeOff o) {
    const uint32_t s = blk * 64u + uint32_t(lane);
    const bool has = s < a.n_stripes;
    const uint32_t sc = has ? s : 0u;
    const uint64_t raw_s = stripe_raw(a, sc);
    const uint32_t n = uint32_t(raw_s / 2);
    const uint32_t nsb = stripe_subblocks<L>(n);
    const uint64_t so = o.so;
    const uint4 r0 = *reinterpret_cast<const uint4*>(a.blob + so);
    const uint4 r1 = *reinterpret_cast<const uint4*>(a.blob + so + 16);
    const uint32_t n_bits = r0.z, bit_bytes = r0.w, bits_off = r1.z, even_off = r1.w;
    const uint32_t ok = bit(has) & o.in & bit(r0.x == uint32_t(raw_s)) & bit(r0.y == n) &
                        bit(r1.x == sc * Geo<L>::kSubPerStripe) & bit(r1.y == nsb) &
                        bit(uint64_t(n_bits) <= uint64_t(K3HUF_MAXLEN) * n) &
                        bit(k3huf_bounds::stripe_planes_ok(a.blob_bytes, so, n, nsb, n_bits, bit_bytes,
                                                           bits_off, even_off));
    StripeLane t;
    t.off16 = ok ? uint32_t(so >> 4) : 0u;
    t.bits_off = ok ? bits_off : 0u;
    t.even_off = ok ? even_off : 0u;
    t.n_bits = ok ? n_bits : kNoStripe;
    return t;
}
template <uint32_t L>
__device__ __forceinline__ StripeLane load_stripes(const DecodeArgs& a, uint32_t blk, int lane) {
    return stripe_values<L>(a, blk, lane, stripe_offsets(a, blk, lane));
}

// A subblock record as vector registers: lanes 0 and 1 hold start_bit and
// n_syms, lane 2 the next record's start_bit (when the stripe has one), and
// lane t holds lane bit counts t and 64 + t. Vector loads, so the record of
// the next unit can be requested a whole unit before it is used.
struct RecLanes {
    uint32_t hd, lo, hi;
};

__device__ __forceinline__ RecLanes load_rec(const uint8_t* rec, bool has_next, int lane) {
    const uint32_t off = lane == 2 ? (has_next ? K3HUF_SUBBLOCK_REC_BYTES : 0u) : 4u * uint32_t(lane & 1);
    const uint16_t* lbits = reinterpret_cast<const uint16_t*>(rec + 8);
    RecLanes r;
    r.hd = ld32(rec + off);
    r.lo = lbits[lane];
    r.hi = lbits[kUnitLanes + lane];
    return r;
}

// The kernel for a layer of lane chunks of L symbols. lds: the workgroup's
// kLdsBytes; local_ticket: its own counter (launches without a slot).
template <uint32_t L>
__device__ __forceinline__ void decode_layer_body(const DecodeArgs& a, uint8_t* lds, uint32_t& local_ticket) {
    using G = Geo<L>;
    uint32_t* tab = reinterpret_cast<uint32_t*>(lds);  // at LDS address 0
    const uint32_t n_sub = uint32_t((a.out_bytes + G::kSubBytes - 1) / G::kSubBytes);

    // layer header must describe exactly this call (uniform over the grid;
    // every field is tested, so the loads go out together). The set-up below
    // reads nothing whose place the header decides, so the test is taken
    // after it and the header's loads travel with its first round trip.
    const uint8_t* b = a.blob;
    const uint32_t hdr_ok = bit(ld32(b) == 0x4648334Bu /* "K3HF" */) & bit(ld32(b + 4) == (1u | (12u << 16))) &
                            bit(ld32(b + 8) == K3HUF_STRIPE_BYTES) & bit(ld32(b + 12) == G::kSubBytes) &
                            bit(ld32(b + 16) == L) & bit(ld32(b + 20) == a.n_stripes) &
                            bit(ld64(b + 24) == a.out_bytes) & bit(ld32(b + 32) == n_sub) &
                            bit(ld64(b + 40) <= a.blob_bytes);

    const int lane = threadIdx.x & 63;
    const uint32_t wave = uniform(threadIdx.x >> 6);
    const uint32_t n_units = n_sub * kUnitsPerSub;
    const uint32_t T = gridDim.x * kWaves;
    const uint32_t groups = min(kGroupsPerSlot, gridDim.x);
    const uint32_t group = blockIdx.x % groups;
    uint32_t* slot = &g_sched[kSlotWords * a.slot];
    auto unit_of = [&](uint32_t p) { return n_units - 1u - p; };   // p < n_units
    uint32_t h = wave * gridDim.x + blockIdx.x;                    // position of this wave's unit

    // The set-up's loads go out in two round trips: the header, the table's
    // first words and the stripe offsets; then the stripe records, the
    // table's second words and the first unit's record (its address needs
    // only its stripe's offset).
    constexpr int kPerThread = (K3HUF_LUT_ENTRIES + kThreads - 1) / kThreads;
    uint32_t ta[kPerThread], tb[kPerThread];
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int i = int(threadIdx.x) + q * kThreads;
        ta[q] = i < K3HUF_LUT_ENTRIES ? uint32_t(a.lut[i]) : 0u;
    }
    // stripe values of the block holding this wave's first unit
    uint32_t blk = h < n_units ? unit_of(h) / (kUnitsPerSub * G::kSubPerStripe * 64u) : 0u;
    const StripeOff so0 = stripe_offsets(a, blk, lane);
    uint32_t pf_h = 0xFFFFFFFFu;   // position whose unit's record `pf` holds
    RecLanes pf = {0u, 0u, 0u};
    if (h < n_units) {
        // a record outside the blob is read from the blob's start instead;
        // the records of a stripe that passes its checks lie inside, so the
        // record is the right one whenever the unit is decoded
        const uint32_t kn = unit_of(h) / kUnitsPerSub;
        const uint32_t sn = kn / G::kSubPerStripe, jn = kn % G::kSubPerStripe;
        const uint64_t son = uint64_t(lane_value(uint32_t(so0.so >> 4), sn & 63u)) << 4;
        const bool nx = jn + 1 < stripe_subblocks<L>(uint32_t(stripe_raw(a, sn) / 2));
        const uint64_t ro = k3huf_bounds::subblock_rec_in_blob(a.blob_bytes, son, jn, nx)
                                ? son + K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * jn
                                : 0ull;
        pf = load_rec(b + ro, nx, lane);
        pf_h = h;
    }
    StripeLane sl = stripe_values<L>(a, blk, lane, so0);
    // request the record of position p's unit (when its stripe is in `sl`)
    auto request_rec = [&](uint32_t p) {
        pf_h = 0xFFFFFFFFu;
        if (p < n_units) {
            const uint32_t kn = unit_of(p) / kUnitsPerSub;
            const uint32_t sn = kn / G::kSubPerStripe, jn = kn % G::kSubPerStripe;
            if ((sn >> 6) == blk && lane_value(sl.n_bits, sn & 63u) != kNoStripe) {
                const uint8_t* stn = b + (uint64_t(lane_value(sl.off16, sn & 63u)) << 4);
                pf = load_rec(stn + K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * jn,
                              jn + 1 < stripe_subblocks<L>(uint32_t(stripe_raw(a, sn) / 2)), lane);
                pf_h = p;
            }
        }
    };
    if (threadIdx.x == 0) local_ticket = 0u;
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int i = int(threadIdx.x) + q * kThreads;
        const int i2 = i < K3HUF_LUT_ENTRIES ? second_index(uint32_t(i), ta[q]) : -1;
        tb[q] = i2 >= 0 ? uint32_t(a.lut[i2]) : 0u;
    }
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int i = int(threadIdx.x) + q * kThreads;
        if (i < K3HUF_LUT_ENTRIES) tab[i] = make_entry(ta[q], tb[q]);
    }
    __syncthreads();
    if (!hdr_ok) {
        if (blockIdx.x == 0 && threadIdx.x == 0) flag(a.status, K3HUF_DEV_HEADER);
        return;
    }

    uint8_t* wl = lds + kTabBytes + wave * kWaveLds;
    uint32_t* buf = reinterpret_cast<uint32_t*>(wl);
    uint8_t* stage = wl + kBufBytes;
    uint32_t ticket = 0;           // lane 0: the answer to this unit's request

    while (h < n_units) {
        // the last two rounds of units are the grid's critical path: their
        // waves issue ahead of waves still busy with earlier units
        if (h + 2 * T >= n_units) __builtin_amdgcn_s_setprio(1);
        if (h + T >= n_units) __builtin_amdgcn_s_setprio(3);
        // the next position: asked for halfway through a full unit (`ask`),
        // read and its record requested as the unit's last phase starts
        // (`learn`); other units do both at their end
        bool asked = false;
        uint32_t h_next = 0xFFFFFFFFu;
        auto ask = [&]() {
            if (lane == 0)
                ticket = a.dyn ? atomicAdd(&slot[group * kCounterStride], 1u) : atomicAdd(&local_ticket, 1u);
            asked = true;
        };
        // with the device counters: position T + group + groups * ticket;
        // with the workgroup's own: the workgroup's share b + blocks * j, j
        // past the first round's kWaves
        auto next_pos = [&]() {
            return a.dyn ? uniform(T + group + groups * lane_value(ticket, 0))
                         : uniform(blockIdx.x + gridDim.x * (kWaves + lane_value(ticket, 0)));
        };
        auto learn = [&]() {
            h_next = next_pos();
            request_rec(h_next);
        };
        const uint32_t un_idx = unit_of(h);
        const uint32_t k = un_idx / kUnitsPerSub, half = un_idx % kUnitsPerSub;
        const uint32_t s = k / G::kSubPerStripe, jsb = k % G::kSubPerStripe;
        if ((s >> 6) != blk) {
            blk = s >> 6;
            sl = load_stripes<L>(a, blk, lane);
        }
        const uint32_t n_bits = lane_value(sl.n_bits, s & 63u);
        const uint64_t soff = uint64_t(lane_value(sl.off16, s & 63u)) << 4;
        const uint32_t bits_off = lane_value(sl.bits_off, s & 63u);
        const uint32_t even_off = lane_value(sl.even_off, s & 63u);
        const uint32_t n = uint32_t(stripe_raw(a, s) / 2);
        const uint32_t nsb = stripe_subblocks<L>(n);
        const uint8_t* st = b + soff;
        if (pf_h != h && n_bits != kNoStripe) {
            pf = load_rec(st + K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * jsb,
                          jsb + 1 < nsb, lane);
            drain_vm();
        }
        // everything this unit needs from its record, read before the
        // registers are refilled with the next unit's record
        const uint32_t start_bit = lane_value(pf.hd, 0);
        const uint32_t rec_syms = lane_value(pf.hd, 1);
        const uint32_t next_start = jsb + 1 < nsb ? lane_value(pf.hd, 2) : n_bits;
        const uint32_t lb = half ? pf.hi : pf.lo;
        const uint32_t incl = wave_incl_scan(lb);   // prefix within this unit
        const uint32_t unit_bits = lane_value(incl, 63);
        const uint32_t other_bits = lane_value(wave_incl_scan(half ? pf.lo : pf.hi), 63);
        do {
        if (n_bits == kNoStripe) {
            if (lane == 0 && half == 0) flag(a.status, K3HUF_DEV_STRIPE);
            continue;
        }
        const uint32_t nsyms = min(G::kSubSyms, n - jsb * G::kSubSyms);
        const uint32_t total = unit_bits + other_bits;
        const int gl = int(half) * kUnitLanes + lane;    // lane chunk within the subblock
        const int cnt = min(max(int(nsyms) - gl * int(L), 0), int(L));
        // the prefix must also be monotone and end at the unit's sum, which
        // keeps every lane's bit range inside the unit's codes
        const bool lane_ok = lb >= uint32_t(cnt) && lb <= uint32_t(cnt) * K3HUF_MAXLEN &&
                             incl >= lb && incl <= unit_bits;
        const bool sb_ok = rec_syms == nsyms && start_bit <= n_bits &&
                           uint64_t(start_bit) + total == next_start && next_start <= n_bits;
        if (!sb_ok || __any(!lane_ok)) {
            if (lane == 0) flag(a.status, K3HUF_DEV_INDEX);
            continue;
        }
        Unit un;
        un.nsyms = uint32_t(min(max(int(nsyms) - int(half) * G::kUnitSyms, 0), G::kUnitSyms));
        if (un.nsyms == 0) continue;
        const uint32_t unit_start = start_bit + (half ? other_bits : 0u);
        un.bits = st + bits_off;
        un.dmax = k3huf_bounds::stripe_read_dmax(bits_off, even_off, n);
        un.even = st + even_off + uint64_t(jsb) * G::kSubSyms + uint64_t(half) * G::kUnitSyms;
        un.out = a.out + uint64_t(k) * G::kSubBytes + 2ull * half * G::kUnitSyms;
        const uint32_t lane_start = unit_start + incl - lb;
        const uint32_t lane_end = unit_start + incl;

        if (un.nsyms == uint32_t(G::kUnitSyms)) {
            const int j0 = first_dword(lane_value(lane_start, 0));
            const int units = (end_dword(lane_value(lane_end, 63)) - j0) / 4;
            if (units * 16 <= kBufBytes) {
                fill_buffer(buf, un, j0, units, lane);
                drain_vm();   // fill_buffer has just drained it
                decode_unit<L, false>(a, tab, buf, stage, un, j0, lane_start, lb, lane, ask, learn);
            } else {
                // codes exceed the buffer (long codes, e.g. a vector of
                // norm gains): each lane gathers its codes phase by phase
                decode_unit<L, true>(a, tab, buf, stage, un, 0, lane_start, lb, lane, ask, learn);
            }
        } else {
            // the layer's partial last unit: passes over consecutive lane
            // ranges whose codes fit the buffer
            for (int l0 = 0; l0 < 64;) {
                const int j0 = first_dword(lane_value(lane_start, l0));
                const bool over = lane >= l0 && (end_dword(lane_end) - j0) * 4 > kBufBytes;
                const uint64_t m = __ballot(over);
                const int l1 = m ? int(__builtin_ctzll(m)) : 64;   // > l0: one chunk always fits
                const int units = (end_dword(lane_value(lane_end, l1 - 1)) - j0) / 4;
                fill_buffer(buf, un, j0, units, lane);
                decode_lanes_tail<L>(a, tab, buf, stage, un, j0, lane_start, lb, l0, l1, lane);
                l0 = l1;
            }
        }
        } while (false);   // the checks above leave a bad unit with `continue`
        if (h_next == 0xFFFFFFFFu) {   // no mid-unit steps ran
            if (!asked) ask();
            h_next = next_pos();
        }
        h = h_next;
    }

    // the last workgroup to finish clears this launch's counter slot
    __syncthreads();
    if (a.dyn && threadIdx.x == 0) {
        const uint32_t done = atomicAdd(&slot[kGroupsPerSlot * kCounterStride], 1u);
        if (done == gridDim.x - 1)
            for (uint32_t g = 0; g <= kGroupsPerSlot; ++g) atomicExch(&slot[g * kCounterStride], 0u);
    }
}

// The layer's lane-chunk length picks the body (uniform over the grid; any
// other value fails the body's header check).
__global__ __launch_bounds__(kThreads) void k3huf_decode_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    __shared__ uint32_t local_ticket;
    if (ld32(a.blob + 16) == K3HUF_LANE_SYMS_SHORT)
        decode_layer_body<K3HUF_LANE_SYMS_SHORT>(a, lds, local_ticket);
    else
        decode_layer_body<K3HUF_LANE_SYMS>(a, lds, local_ticket);
}

struct DevInfo {
    int cus = 0;
    int wg_per_cu = 0;
};

std::mutex g_mu;
std::vector<DevInfo> g_dev;
constexpr uint32_t kNoSlot = 0xFFFFFFFFu;
std::map<std::pair<int, void*>, uint32_t> g_stream_slot;   // (device, stream) -> counter slot
std::vector<uint32_t> g_next_slot;                        // per device

// The device's launch geometry and the counter slot of `stream` on it
// (kNoSlot once the device's kSchedSlots slots are taken).
int device_info(void* stream, DevInfo* out, uint32_t* slot) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return K3HUF_E_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (int(g_next_slot.size()) <= dev) g_next_slot.resize(dev + 1, 0u);
    // streams past the slots are not recorded, so the map stays bounded
    // however many streams a process creates. hipStreamPerThread names a
    // different stream in each host thread, so launches through that one
    // handle can overlap: it never gets a slot.
    auto it = g_stream_slot.find({dev, stream});
    if (stream == static_cast<void*>(hipStreamPerThread))
        *slot = kNoSlot;
    else if (it != g_stream_slot.end())
        *slot = it->second;
    else if (g_next_slot[dev] < kSchedSlots)
        *slot = g_stream_slot.emplace(std::make_pair(dev, stream), g_next_slot[dev]++).first->second;
    else
        *slot = kNoSlot;
    if (int(g_dev.size()) <= dev) g_dev.resize(dev + 1);
    DevInfo& d = g_dev[dev];
    if (!d.cus) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return K3HUF_E_HIP;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k3huf_decode_kernel, kThreads, 0) !=
            hipSuccess)
            return K3HUF_E_HIP;
        d.cus = cus;
        d.wg_per_cu = per > 0 ? per : 1;
    }
    *out = d;
    return K3HUF_OK;
}

}  // namespace

extern "C" {

int k3huf_decode_layer(const void* d_blob, size_t blob_bytes, const uint16_t* d_lut, void* d_out,
                       size_t out_bytes, void* stream, uint32_t* d_status) {
    if (!d_blob || !d_lut || !d_out) return K3HUF_E_ARG;
    if ((reinterpret_cast<uintptr_t>(d_blob) & 15) || (reinterpret_cast<uintptr_t>(d_out) & 15) ||
        (reinterpret_cast<uintptr_t>(d_lut) & 1) || (reinterpret_cast<uintptr_t>(d_status) & 3))
        return K3HUF_E_ARG;
    if (blob_bytes < K3HUF_HDR_BYTES + 8 || out_bytes == 0 || (out_bytes & 1)) return K3HUF_E_ARG;
    // subblocks of the 256-symbol and of the 64-symbol layout (the kernel
    // reads which one the blob uses from its header)
    const uint64_t n_sub = (uint64_t(out_bytes) + K3HUF_SUBBLOCK_BYTES - 1) / K3HUF_SUBBLOCK_BYTES;
    const uint64_t n_sub_short = (uint64_t(out_bytes) + Geo<K3HUF_LANE_SYMS_SHORT>::kSubBytes - 1) /
                                 Geo<K3HUF_LANE_SYMS_SHORT>::kSubBytes;
    const uint64_t n_stripes = (uint64_t(out_bytes) + K3HUF_STRIPE_BYTES - 1) / K3HUF_STRIPE_BYTES;
    if (n_sub > 0xFFFFFFFFull || blob_bytes < K3HUF_HDR_BYTES + 8 * n_stripes ||
        uint64_t(blob_bytes) >= (1ull << 36) || uint64_t(out_bytes) > 2ull * blob_bytes)
        return K3HUF_E_ARG;
    DevInfo di;
    uint32_t slot = 0;
    int rc = device_info(stream, &di, &slot);
    if (rc) return rc;
    // a launch captured into a graph may later run beside any other launch:
    // it uses the workgroup counters (so does one whose capture state cannot
    // be read; the failed query's error is cleared)
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &capture) != hipSuccess) {
        (void)hipGetLastError();
        capture = hipStreamCaptureStatusActive;
    }
    // device counters pay off only over many rounds of units: at up to about
    // five rounds the workgroup counters measured as fast or faster
    // (trunk-recipe layers: 0.94-1.00x of the device-counter time at 1.1-4.6
    // rounds, 1.03-1.05x at 6.9-20 rounds)
    const uint64_t want = n_sub * kUnitsPerSub;
    const uint64_t want_short = n_sub_short * kUnitsPerSub;
    const uint64_t resident = uint64_t(di.cus) * uint64_t(di.wg_per_cu);
    // one workgroup per unit of the finer layout, up to a full chip
    const unsigned grid = unsigned(want_short < resident ? want_short : resident);
    const bool dyn = slot != kNoSlot && capture == hipStreamCaptureStatusNone &&
                     want > uint64_t(kDynRounds) * grid * kWaves;
    DecodeArgs a;
    a.blob = static_cast<const uint8_t*>(d_blob);
    a.blob_bytes = blob_bytes;
    a.lut = d_lut;
    a.out = static_cast<uint8_t*>(d_out);
    a.out_bytes = out_bytes;
    a.n_stripes = uint32_t(n_stripes);
    a.status = d_status;
    a.slot = dyn ? slot : 0u;
    a.dyn = dyn ? 1u : 0u;
    // one workgroup per unit up to a full chip (grid above): the first round's
    // positions are wave-major, so a layer of fewer units than CUs gets a CU
    // per unit
    hipLaunchKernelGGL(k3huf_decode_kernel, dim3(grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? K3HUF_OK : K3HUF_E_HIP;
}

int k3huf_decode_ring(const k3huf_ring_layer* layers, int n_layers, void* const* d_slots,
                      int n_slots, size_t slot_bytes, void* const* streams, int n_streams,
                      k3huf_ring_cb cb, void* user, uint32_t* d_status) {
    if (!layers || n_layers < 0 || !d_slots || n_slots < 1 || !streams || n_streams < 1)
        return K3HUF_E_ARG;
    for (int k = 0; k < n_layers; ++k)
        if (layers[k].raw_bytes > slot_bytes) return K3HUF_E_ARG;
    for (int s = 0; s < n_slots; ++s)
        if (!d_slots[s]) return K3HUF_E_ARG;
    std::vector<hipEvent_t> slot_free(n_slots, nullptr);
    std::vector<char> used(n_slots, 0);
    int rc = K3HUF_OK;
    for (int s = 0; s < n_slots && rc == K3HUF_OK; ++s)
        if (hipEventCreateWithFlags(&slot_free[s], hipEventDisableTiming) != hipSuccess) rc = K3HUF_E_HIP;
    for (int k = 0; k < n_layers && rc == K3HUF_OK; ++k) {
        const int s = k % n_slots;
        hipStream_t st = static_cast<hipStream_t>(streams[k % n_streams]);
        if (used[s] && hipStreamWaitEvent(st, slot_free[s], 0) != hipSuccess) {
            rc = K3HUF_E_HIP;
            break;
        }
        rc = k3huf_decode_layer(layers[k].d_blob, layers[k].blob_bytes, layers[k].d_lut, d_slots[s],
                                layers[k].raw_bytes, st, d_status);
        if (rc) break;
        if (cb) cb(k, d_slots[s], layers[k].raw_bytes, st, user);
        if (hipEventRecord(slot_free[s], st) != hipSuccess) rc = K3HUF_E_HIP;
        used[s] = 1;
    }
    for (int s = 0; s < n_slots; ++s)
        if (slot_free[s]) (void)hipEventDestroy(slot_free[s]);
    return rc;
}

int k3huf_decode_ring_host(const k3huf_host_layer* layers, int n_layers, void* const* d_stage,
                           int n_stage, size_t stage_bytes, void* const* d_slots, int n_slots,
                           size_t slot_bytes, void* copy_stream, void* const* streams,
                           int n_streams, k3huf_ring_cb cb, void* user, uint32_t* d_status) {
    if (!layers || n_layers < 0 || !d_stage || n_stage < 1 || !d_slots || n_slots < 1 || !streams ||
        n_streams < 1)
        return K3HUF_E_ARG;
    for (int k = 0; k < n_layers; ++k)
        if (!layers[k].h_blob || !layers[k].d_lut || layers[k].blob_bytes > stage_bytes ||
            layers[k].raw_bytes > slot_bytes)
            return K3HUF_E_ARG;
    for (int s = 0; s < n_stage; ++s)
        if (!d_stage[s] || (reinterpret_cast<uintptr_t>(d_stage[s]) & 15)) return K3HUF_E_ARG;
    for (int s = 0; s < n_slots; ++s)
        if (!d_slots[s]) return K3HUF_E_ARG;
    hipStream_t cs = static_cast<hipStream_t>(copy_stream);
    // copied[s]: stage buffer s holds its layer; stage_free[s]: the decode
    // that read it is done; slot_free[o]: slot o's consumer is done
    std::vector<hipEvent_t> ev(2 * size_t(n_stage) + size_t(n_slots), nullptr);
    hipEvent_t* copied = ev.data();
    hipEvent_t* stage_free = copied + n_stage;
    hipEvent_t* slot_free = stage_free + n_stage;
    std::vector<char> stage_used(n_stage, 0), slot_used(n_slots, 0);
    int rc = K3HUF_OK;
    for (auto& e : ev)
        if (rc == K3HUF_OK && hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess)
            rc = K3HUF_E_HIP;
    for (int k = 0; k < n_layers && rc == K3HUF_OK; ++k) {
        const int s = k % n_stage, o = k % n_slots;
        hipStream_t st = static_cast<hipStream_t>(streams[k % n_streams]);
        // the copy into stage s waits for the decode that last read it
        if (stage_used[s] && hipStreamWaitEvent(cs, stage_free[s], 0) != hipSuccess) rc = K3HUF_E_HIP;
        if (rc == K3HUF_OK &&
            (hipMemcpyAsync(d_stage[s], layers[k].h_blob, layers[k].blob_bytes, hipMemcpyHostToDevice,
                            cs) != hipSuccess ||
             hipEventRecord(copied[s], cs) != hipSuccess || hipStreamWaitEvent(st, copied[s], 0) != hipSuccess))
            rc = K3HUF_E_HIP;
        if (rc == K3HUF_OK && slot_used[o] && hipStreamWaitEvent(st, slot_free[o], 0) != hipSuccess)
            rc = K3HUF_E_HIP;
        if (rc) break;
        rc = k3huf_decode_layer(d_stage[s], layers[k].blob_bytes, layers[k].d_lut, d_slots[o],
                                layers[k].raw_bytes, st, d_status);
        if (rc) break;
        if (hipEventRecord(stage_free[s], st) != hipSuccess) rc = K3HUF_E_HIP;
        stage_used[s] = 1;
        if (cb) cb(k, d_slots[o], layers[k].raw_bytes, st, user);
        if (rc == K3HUF_OK && hipEventRecord(slot_free[o], st) != hipSuccess) rc = K3HUF_E_HIP;
        slot_used[o] = 1;
    }
    for (auto& e : ev)
        if (e) (void)hipEventDestroy(e);
    return rc;
}

}  // extern "C"
