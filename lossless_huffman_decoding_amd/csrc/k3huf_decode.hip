// gfx950 decode path of the k3huf library: the decode kernel, its launcher
// and the layer-ring driver. Container layout: include/k3huf.h.
//
// What is computed (K3 page = "Kimi K3 纯 CPU 推理中的无损 Trunk 压缩…",
// yfxerp.com/news/153994):
//   - "decode loop": a bit window whose top holds the head of the stream;
//     one lookup of the top 12 bits in the 4096-entry table gives the symbol
//     and its code length, and the window shifts by that length;
//   - "key design points": each decoded symbol is the high byte at an odd
//     offset; the raw even-plane byte goes back at the even offset before it.
// How it is laid out on the GPU (not from the pages): one wave decodes one
// 64 KiB-output subblock; lane t decodes lane chunk t (512 symbols) starting
// at the bit offset the subblock index gives it (the ECF8 page, section 2.1,
// keeps such per-thread bit offsets beside its code); the table lives in LDS;
// decoded bytes are staged in LDS so that the even-plane loads and the output
// stores of a wave cover whole 128-byte lines.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "k3huf.h"

namespace {

// One workgroup per CU; each wave decodes whole subblocks, one lane chunk per
// lane. Every global load is issued at least one phase before its data is
// used: the bitstream reaches the decoder through a per-lane ring in LDS that
// is topped up a phase ahead, and the even-plane bytes a phase writes out are
// requested when the phase starts.
constexpr int kWaves = 12;
constexpr int kThreads = 64 * kWaves;
constexpr int kPhase = 32;                            // symbols per lane per phase
constexpr int kPhases = K3HUF_LANE_SYMS / kPhase;    // 16
constexpr int kGroups = kPhase / 4;                   // window refills per phase
constexpr int kRing = 32;                             // ring capacity in dwords
constexpr int kRingStride = 36;                       // dwords per lane: 32 slots, 3 mirror, 1 pad
// dwords a phase may read at or after the dword holding its first bit:
// 28 symbols of at most 12 bits before the last window, plus a 64-bit window
constexpr int kNeed = 14;
constexpr int kPre = 2;                               // 16-byte units requested ahead per phase
constexpr int kStageStride = 48;                      // LDS bytes per lane chunk (32 + 16 pad)
constexpr uint32_t kSubPerStripe = K3HUF_STRIPE_BYTES / K3HUF_SUBBLOCK_BYTES;

// LDS decode table, derived per workgroup from the 4096-entry
// (symbol << 4 | length) table: one lookup of the top 12 window bits yields
// the first code and, when the next code also lies inside those 12 bits, the
// second one too (the "double-symbol table" the K3 page names under "if
// revisited"; the container format is unchanged).
//   [4:0]   bits consumed by the entry's symbols (T)
//   [15:8]  first symbol      [23:16] second symbol (if kFit)
//   [27:24] length of the first code
constexpr uint32_t kT = 31u;
constexpr uint32_t kFit = 1u << 28;   // entry holds two symbols
constexpr uint32_t kBad = 1u << 29;   // index no code covers (decoded as 12 bits)

struct DecodeArgs {
    const uint8_t* blob;
    uint64_t blob_bytes;
    const uint16_t* lut;
    uint8_t* out;
    uint64_t out_bytes;
    uint32_t n_sub;
    uint32_t n_stripes;
    uint32_t* status;
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
__device__ __forceinline__ uint32_t uniform(uint32_t x) {
    return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Table entry for 12-bit index i from the (symbol << 4 | length) table.
__device__ uint32_t make_entry(const uint16_t* lut, uint32_t i) {
    const uint32_t a = lut[i];
    const uint32_t l1 = a & 15u;
    if (l1 == 0 || l1 > K3HUF_MAXLEN) return kBad | kFit | (12u << 24) | 12u;
    uint32_t e = (l1 << 24) | (((a >> 4) & 0xFFu) << 8) | l1;
    if (l1 < K3HUF_MAXLEN) {
        const uint32_t b = lut[(i << l1) & 0xFFFu];
        const uint32_t l2 = b & 15u;
        if (l2 && l1 + l2 <= K3HUF_MAXLEN)
            e = (e & ~kT) | kFit | (((b >> 4) & 0xFFu) << 16) | (l1 + l2);
    }
    return e;
}

// Two symbols from the top of the window, then shift them out. An entry that
// holds one symbol is completed with a second lookup after its first code.
__device__ __forceinline__ uint32_t step2(const uint32_t* tab, uint64_t& acc) {
    uint32_t e = tab[uint32_t(acc >> 52)];
    if (!(e & kFit)) {
        const uint32_t t = e & kT;
        const uint32_t e2 = tab[uint32_t((acc << t) >> 52)];
        e = (e & 0xFF00u) | (((e2 >> 8) & 0xFFu) << 16) | (t + ((e2 >> 24) & 15u)) | kFit |
            ((e | e2) & kBad);
    }
    acc <<= (e & kT);
    return e;
}

// 64-bit window starting at stream bit `pos` from the lane's ring (dwords
// held byte-swapped, dword d at slot d mod 32, slots 32..34 mirror 0..2):
// dwords j..j+2 with j = floor((pos - 1) / 32), shifted right by (-pos) mod 32.
__device__ __forceinline__ uint64_t window(const uint32_t* ring, uint32_t pos) {
    const int j = (int(pos) - 1) >> 5;
    const uint32_t* rp = ring + (uint32_t(j) & (kRing - 1));
    const uint32_t d0 = rp[0], d1 = rp[1], d2 = rp[2];
    const uint32_t r = 0u - pos;
    return (uint64_t(__builtin_amdgcn_alignbit(d0, d1, r)) << 32) |
           __builtin_amdgcn_alignbit(d1, d2, r);
}

// 16-byte unit of the bitstream starting at dword d (a multiple of 4), read
// from at most dword dmax so the read stays inside the blob.
__device__ __forceinline__ uint4 load_unit(const uint8_t* bits, int d, int dmax) {
    return *reinterpret_cast<const uint4*>(bits + 4 * min(d, dmax));
}
__device__ __forceinline__ void put_unit(uint32_t* ring, int d, uint4 v) {
    const uint4 b = make_uint4(bswap32(v.x), bswap32(v.y), bswap32(v.z), bswap32(v.w));
    const uint32_t s = uint32_t(d) & (kRing - 1);
    *reinterpret_cast<uint4*>(ring + s) = b;
    if (s == 0) *reinterpret_cast<uint4*>(ring + kRing) = b;
}

// Decode one subblock with one wave. FULL: all 64 lane chunks hold 512
// symbols (two symbols per table step); otherwise lane t holds
// clamp(nsyms - 512 t, 0, 512) and decodes one symbol per step.
template <bool FULL>
__device__ __forceinline__ void decode_subblock(const DecodeArgs& a, const uint32_t* tab,
                                                uint32_t* ring, uint8_t* stage,
                                                const uint8_t* bits, int dmax,
                                                const uint8_t* even_sb, uint8_t* out_sb,
                                                uint32_t lane_start, uint32_t lane_bits,
                                                uint32_t nsyms, int lane) {
    const int lane_cnt = FULL ? int(K3HUF_LANE_SYMS)
                              : min(max(int(nsyms) - lane * int(K3HUF_LANE_SYMS), 0),
                                    int(K3HUF_LANE_SYMS));
    uint32_t pos = lane_start;
    uint32_t bad = 0;
    // fill the ring with the 32 dwords from the 16-byte unit holding the
    // lane's first window dword
    int hi = ((int(pos) - 1) >> 5) & ~3;
    {
        uint4 u[kRing / 4];
#pragma unroll
        for (int q = 0; q < kRing / 4; ++q) u[q] = load_unit(bits, hi + 4 * q, dmax);
#pragma unroll
        for (int q = 0; q < kRing / 4; ++q) put_unit(ring, hi + 4 * q, u[q]);
        hi += kRing;
    }
    const int sub_line = lane >> 2, part = lane & 3;

    for (int ph = 0; ph < kPhases; ++ph) {
        // request the next units while there is room behind the live window
        const int j0 = (int(pos) - 1) >> 5;
        const int room = (j0 + kRing - hi) >> 2;
        uint4 pre[kPre];
#pragma unroll
        for (int q = 0; q < kPre; ++q)
            if (q < room) pre[q] = load_unit(bits, hi + 4 * q, dmax);
        // even-plane bytes this phase writes out
        uint2 ev[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const uint32_t u = uint32_t(rr * 16 + sub_line) * K3HUF_LANE_SYMS + uint32_t(ph * kPhase + part * 8);
            if (FULL || u < nsyms) ev[rr] = *reinterpret_cast<const uint2*>(even_sb + u);
        }

        uint32_t w[kGroups];
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            uint64_t acc = window(ring, pos);
            if (FULL) {
                const uint32_t e1 = step2(tab, acc);
                const uint32_t e2 = step2(tab, acc);
                pos += (e1 + e2) & 0xFFu;
                bad |= e1 | e2;
                w[g] = __builtin_amdgcn_perm(e2, e1, 0x06050201u);
            } else {
                uint32_t ww = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t e = tab[uint32_t(acc >> 52)];
                    const bool live = ph * kPhase + g * 4 + t < lane_cnt;
                    const uint32_t l = live ? (e >> 24) & 15u : 0u;
                    if (live) bad |= e;
                    acc <<= l;
                    pos += l;
                    constexpr uint32_t sel[4] = {0x03020105u, 0x03020500u, 0x03050100u, 0x05020100u};
                    ww = __builtin_amdgcn_perm(e, ww, sel[t]);
                }
                w[g] = ww;
            }
        }

        // ring upkeep for the next phase
#pragma unroll
        for (int q = 0; q < kPre; ++q)
            if (q < room) put_unit(ring, hi + 4 * q, pre[q]);
        hi += 4 * max(min(room, kPre), 0);
        const int j1 = (int(pos) - 1) >> 5;
        while (__any(hi < j1 + kNeed)) {  // at most 3 rounds: hi >= j1 + 2 here
            if (hi < j1 + kNeed) {
                put_unit(ring, hi, load_unit(bits, hi, dmax));
                hi += 4;
            }
        }

        // stage this phase's symbols, then interleave with the even plane
        uint8_t* my_stage = stage + lane * kStageStride;
        *reinterpret_cast<uint4*>(my_stage) = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint4*>(my_stage + 16) = make_uint4(w[4], w[5], w[6], w[7]);
        wave_sync();
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int line = rr * 16 + sub_line;
            const uint2 sy = *reinterpret_cast<const uint2*>(stage + line * kStageStride + part * 8);
            const uint32_t u = uint32_t(line) * K3HUF_LANE_SYMS + uint32_t(ph * kPhase + part * 8);
            if (FULL || u + 8 <= nsyms) {
                uint4 o;
                o.x = __builtin_amdgcn_perm(sy.x, ev[rr].x, 0x05010400u);
                o.y = __builtin_amdgcn_perm(sy.x, ev[rr].x, 0x07030602u);
                o.z = __builtin_amdgcn_perm(sy.y, ev[rr].y, 0x05010400u);
                o.w = __builtin_amdgcn_perm(sy.y, ev[rr].y, 0x07030602u);
                *reinterpret_cast<uint4*>(out_sb + 2 * u) = o;
            } else if (u < nsyms) {
                const uint32_t m = nsyms - u;
                for (uint32_t i = 0; i < m; ++i) {
                    const uint32_t e8 = i < 4 ? (ev[rr].x >> (8 * i)) : (ev[rr].y >> (8 * (i - 4)));
                    const uint32_t s8 = i < 4 ? (sy.x >> (8 * i)) : (sy.y >> (8 * (i - 4)));
                    *reinterpret_cast<uint16_t*>(out_sb + 2 * (u + i)) =
                        uint16_t((e8 & 0xFFu) | ((s8 & 0xFFu) << 8));
                }
            }
        }
        wave_sync();
    }
    if (bad & kBad) flag(a.status, K3HUF_DEV_CODE);
    if (pos != lane_start + lane_bits) flag(a.status, K3HUF_DEV_LANE_END);
}

__global__ __launch_bounds__(kThreads) void k3huf_decode_kernel(DecodeArgs a) {
    __shared__ uint32_t tab[K3HUF_LUT_ENTRIES];
    __shared__ __attribute__((aligned(16))) uint32_t ring_all[kWaves * 64 * kRingStride];
    __shared__ __attribute__((aligned(16))) uint8_t stage_all[kWaves * 64 * kStageStride];

    // layer header must describe exactly this call (uniform over the grid)
    const uint8_t* b = a.blob;
    const bool hdr_ok = ld32(b) == 0x4648334Bu /* "K3HF" */ && ld32(b + 4) == (1u | (12u << 16)) &&
                        ld32(b + 8) == K3HUF_STRIPE_BYTES && ld32(b + 12) == K3HUF_SUBBLOCK_BYTES &&
                        ld32(b + 16) == K3HUF_LANE_SYMS && ld32(b + 20) == a.n_stripes &&
                        ld64(b + 24) == a.out_bytes && ld32(b + 32) == a.n_sub &&
                        ld64(b + 40) <= a.blob_bytes;
    if (!hdr_ok) {
        if (blockIdx.x == 0 && threadIdx.x == 0) flag(a.status, K3HUF_DEV_HEADER);
        return;
    }

    for (int i = threadIdx.x; i < K3HUF_LUT_ENTRIES; i += kThreads) tab[i] = make_entry(a.lut, i);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const uint32_t wave = uniform(threadIdx.x >> 6);
    uint32_t* ring = ring_all + (wave * 64 + lane) * kRingStride;
    uint8_t* stage = stage_all + wave * (64 * kStageStride);

    for (uint32_t k = blockIdx.x * kWaves + wave; k < a.n_sub; k += gridDim.x * kWaves) {
        const uint32_t s = k / kSubPerStripe, jsb = k % kSubPerStripe;
        const uint64_t soff = ld64(b + K3HUF_HDR_BYTES + 8ull * s);
        const uint64_t raw_s = min(uint64_t(K3HUF_STRIPE_BYTES), a.out_bytes - uint64_t(s) * K3HUF_STRIPE_BYTES);
        const uint32_t n = uint32_t(raw_s / 2);
        const uint32_t nsb = (n + K3HUF_SUBBLOCK_SYMS - 1) / K3HUF_SUBBLOCK_SYMS;
        bool ok = (soff & 15) == 0 && soff + K3HUF_STRIPE_HDR_BYTES <= a.blob_bytes;
        const uint8_t* st = b + soff;
        uint32_t n_bits = 0, bit_bytes = 0, bits_off = 0, even_off = 0;
        if (ok) {
            n_bits = ld32(st + 8);
            bit_bytes = ld32(st + 12);
            bits_off = ld32(st + 24);
            even_off = ld32(st + 28);
            ok = ld32(st) == uint32_t(raw_s) && ld32(st + 4) == n && ld32(st + 16) == s * kSubPerStripe &&
                 ld32(st + 20) == nsb && (bits_off & 15) == 0 && (even_off & 15) == 0 &&
                 bits_off >= K3HUF_STRIPE_HDR_BYTES + K3HUF_SUBBLOCK_REC_BYTES * nsb &&
                 uint64_t(n_bits) <= 8ull * bit_bytes &&
                 uint64_t(even_off) >= uint64_t(bits_off) + bit_bytes &&
                 soff + even_off + ((uint64_t(n) + 15) & ~15ull) <= a.blob_bytes;
        }
        if (!ok) {
            if (lane == 0) flag(a.status, K3HUF_DEV_STRIPE);
            continue;
        }
        const uint8_t* rec = st + K3HUF_STRIPE_HDR_BYTES + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * jsb;
        const uint32_t start_bit = ld32(rec);
        const uint32_t nsyms = min(uint32_t(K3HUF_SUBBLOCK_SYMS), n - jsb * K3HUF_SUBBLOCK_SYMS);
        const uint32_t next_start = jsb + 1 < nsb ? ld32(rec + K3HUF_SUBBLOCK_REC_BYTES) : n_bits;
        const uint32_t lb = *reinterpret_cast<const uint16_t*>(rec + 8 + 2 * lane);
        // inclusive prefix sum of the lane chunks' bit counts over the wave
        uint32_t incl = lb;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        const uint32_t total = uniform(__shfl(incl, 63, 64));
        const int cnt = min(max(int(nsyms) - lane * int(K3HUF_LANE_SYMS), 0), int(K3HUF_LANE_SYMS));
        const bool lane_ok = lb >= uint32_t(cnt) && lb <= uint32_t(cnt) * K3HUF_MAXLEN;
        const bool sb_ok = ld32(rec + 4) == nsyms && start_bit <= n_bits &&
                           uint64_t(start_bit) + total == next_start && next_start <= n_bits;
        if (!sb_ok || __any(!lane_ok)) {
            if (lane == 0) flag(a.status, K3HUF_DEV_INDEX);
            continue;
        }
        const uint8_t* bits = st + bits_off;
        // last 16-byte unit (in dwords from the bitstream start) inside the blob
        const int dmax = int(((a.blob_bytes - (soff + bits_off) - 16) / 4) & ~3ull);
        const uint8_t* even_sb = st + even_off + uint64_t(jsb) * K3HUF_SUBBLOCK_SYMS;
        uint8_t* out_sb = a.out + uint64_t(k) * K3HUF_SUBBLOCK_BYTES;
        const uint32_t lane_start = start_bit + incl - lb;
        if (nsyms == K3HUF_SUBBLOCK_SYMS)
            decode_subblock<true>(a, tab, ring, stage, bits, dmax, even_sb, out_sb, lane_start, lb,
                                  nsyms, lane);
        else
            decode_subblock<false>(a, tab, ring, stage, bits, dmax, even_sb, out_sb, lane_start, lb,
                                   nsyms, lane);
    }
}

struct DevInfo {
    int cus = 0;
    int wg_per_cu = 0;
};

std::mutex g_mu;
std::vector<DevInfo> g_dev;

int device_info(DevInfo* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return K3HUF_E_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
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
    const uint64_t n_sub = (uint64_t(out_bytes) + K3HUF_SUBBLOCK_BYTES - 1) / K3HUF_SUBBLOCK_BYTES;
    const uint64_t n_stripes = (uint64_t(out_bytes) + K3HUF_STRIPE_BYTES - 1) / K3HUF_STRIPE_BYTES;
    if (n_sub > 0xFFFFFFFFull || blob_bytes < K3HUF_HDR_BYTES + 8 * n_stripes) return K3HUF_E_ARG;
    DevInfo di;
    int rc = device_info(&di);
    if (rc) return rc;
    DecodeArgs a;
    a.blob = static_cast<const uint8_t*>(d_blob);
    a.blob_bytes = blob_bytes;
    a.lut = d_lut;
    a.out = static_cast<uint8_t*>(d_out);
    a.out_bytes = out_bytes;
    a.n_sub = uint32_t(n_sub);
    a.n_stripes = uint32_t(n_stripes);
    a.status = d_status;
    const uint64_t want = (n_sub + kWaves - 1) / kWaves;
    const uint64_t resident = uint64_t(di.cus) * uint64_t(di.wg_per_cu);
    const unsigned grid = unsigned(want < resident ? want : resident);
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

}  // extern "C"
