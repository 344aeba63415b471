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
// runs in four kernels:
//   enc_hist   per-stripe histograms of the odd bytes;
//   enc_count  code bits of every 256-symbol lane chunk;
//   enc_scan   per stripe: chunk start bits, the subblock records and the
//              stripe record;
//   enc_pack   one thread per lane chunk: its codes from its start bit (words
//              it shares with a neighbour are OR-ed in atomically), and its
//              even bytes.
#include <hip/hip_runtime.h>

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
constexpr int kHistBlocksPerStripe = 64;
constexpr int kScanThreads = 1024;
constexpr int kChunkThreads = 256;

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
    uint64_t hist, geom, chunks, status, total;
};

WorkLayout work_layout(uint64_t raw_bytes) {
    const uint64_t ns = k3huf_detail::stripes_for(raw_bytes);
    const uint64_t n_chunks = (raw_bytes / 2 + K3HUF_LANE_SYMS - 1) / K3HUF_LANE_SYMS;
    WorkLayout w;
    w.hist = 0;
    w.geom = align256(w.hist + 256 * 8 * ns);
    w.chunks = align256(w.geom + sizeof(StripeDev) * ns);
    w.status = align256(w.chunks + 4 * n_chunks);
    w.total = w.status + 256;
    return w;
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

// Per-stripe histograms of the odd bytes: grid (kHistBlocksPerStripe,
// stripes). Each block counts a slice of its stripe into 32 interleaved LDS
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
         i += uint64_t(kHistBlocksPerStripe) * kHistThreads) {
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

// Code bits of lane chunk c (symbols [256 c, min(256 c + 256, n))): one
// thread per chunk.
__global__ __launch_bounds__(kChunkThreads) void enc_count(const uint8_t* raw, uint64_t raw_bytes,
                                                           uint64_t n_chunks, CodeTable ct,
                                                           uint32_t* chunk) {
    __shared__ uint8_t len[256];
    if (threadIdx.x < 256) len[threadIdx.x] = uint8_t(ct.e[threadIdx.x] >> 16);
    __syncthreads();
    const uint64_t c = uint64_t(blockIdx.x) * kChunkThreads + threadIdx.x;
    if (c >= n_chunks) return;
    const uint64_t b0 = c * 2 * K3HUF_LANE_SYMS;
    const uint64_t b1 = min(b0 + 2 * K3HUF_LANE_SYMS, raw_bytes);
    uint32_t bits = 0;
    if (b1 - b0 == 2 * K3HUF_LANE_SYMS) {
        const uint4* p = reinterpret_cast<const uint4*>(raw + b0);
#pragma unroll 4
        for (int i = 0; i < 32; ++i) {
            const uint4 v = p[i];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) bits += len[(w[k] >> 8) & 0xFFu] + len[w[k] >> 24];
        }
    } else {
        for (uint64_t i = b0; i < b1; i += 2) bits += len[raw[i + 1]];
    }
    chunk[c] = bits;
}

// Per stripe (one block each): exclusive prefix of the chunk bit counts.
// Writes the stripe record, the subblock records (start bit, symbol count,
// lane bit counts) and replaces chunk[] with stripe-relative start bits. A
// total that differs from the host's count (the input changed during the
// call) sets *status.
__global__ __launch_bounds__(kScanThreads) void enc_scan(uint8_t* out, const StripeDev* g,
                                                         uint32_t* chunk, uint32_t* status) {
    __shared__ uint32_t part[kScanThreads];
    const uint32_t s = blockIdx.x;
    const StripeDev G = g[s];
    const uint32_t nc = (G.n + K3HUF_LANE_SYMS - 1) / K3HUF_LANE_SYMS;
    uint32_t* cb = chunk + uint64_t(s) * kChunksPerStripe;
    const uint32_t per = (nc + kScanThreads - 1) / kScanThreads;
    const uint32_t j0 = min(threadIdx.x * per, nc), j1 = min(j0 + per, nc);
    uint32_t sum = 0;
    for (uint32_t j = j0; j < j1; ++j) sum += cb[j];
    part[threadIdx.x] = sum;
    __syncthreads();
    // inclusive scan of the per-thread sums (Hillis-Steele in LDS)
    for (int d = 1; d < kScanThreads; d <<= 1) {
        const uint32_t v = threadIdx.x >= uint32_t(d) ? part[threadIdx.x - d] : 0u;
        __syncthreads();
        part[threadIdx.x] += v;
        __syncthreads();
    }
    uint32_t pos = part[threadIdx.x] - sum;
    uint8_t* recs = out + G.off + K3HUF_STRIPE_HDR_BYTES;
    for (uint32_t j = j0; j < j1; ++j) {
        const uint32_t bits = cb[j];
        const uint32_t b = j / K3HUF_LANES, t = j % K3HUF_LANES;
        uint8_t* rec = recs + uint64_t(K3HUF_SUBBLOCK_REC_BYTES) * b;
        *reinterpret_cast<uint16_t*>(rec + 8 + 2 * t) = uint16_t(bits);
        if (t == 0) {
            *reinterpret_cast<uint32_t*>(rec) = pos;
            *reinterpret_cast<uint32_t*>(rec + 4) = min(uint32_t(K3HUF_SUBBLOCK_SYMS), G.n - b * K3HUF_SUBBLOCK_SYMS);
        }
        cb[j] = pos;
        pos += bits;
    }
    if (threadIdx.x == kScanThreads - 1) {
        if (part[kScanThreads - 1] != G.nbits) atomicOr(status, 1u);
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

// One thread per lane chunk: its codes, MSB first, from its start bit, and
// its even bytes. Words wholly inside the chunk's bit range are stored;
// its first and last words may hold a neighbour's bits and are OR-ed in
// (enc_zero_stripes cleared them).
__global__ __launch_bounds__(kChunkThreads) void enc_pack(const uint8_t* raw, uint64_t raw_bytes,
                                                          uint64_t n_chunks, CodeTable ct,
                                                          const StripeDev* g, const uint32_t* chunk,
                                                          uint8_t* out) {
    __shared__ uint32_t tab[256];
    if (threadIdx.x < 256) tab[threadIdx.x] = ct.e[threadIdx.x];
    __syncthreads();
    const uint64_t c = uint64_t(blockIdx.x) * kChunkThreads + threadIdx.x;
    if (c >= n_chunks) return;
    const uint32_t s = uint32_t(c / kChunksPerStripe);
    const StripeDev G = g[s];
    uint32_t* words = reinterpret_cast<uint32_t*>(out + G.off + G.bits_off);
    const uint32_t local = uint32_t(c % kChunksPerStripe) * K3HUF_LANE_SYMS;   // stripe symbol index
    uint8_t* even = out + G.off + G.even_off + local;
    const uint32_t b0 = chunk[c];
    uint32_t w = b0 >> 5;
    uint64_t acc = 0;            // pending bits, the earliest at bit 63
    uint32_t nacc = b0 & 31u;    // bits of word w before acc's top are a neighbour's (zero here)
    bool first = true;
    auto put = [&](uint32_t sym) {
        const uint32_t e = tab[sym];
        const uint32_t l = e >> 16;
        acc |= uint64_t(e & 0xFFFFu) << (64u - nacc - l);
        nacc += l;
        if (nacc >= 32) {
            const uint32_t v = bswap32(uint32_t(acc >> 32));
            if (first)
                atomicOr(&words[w], v);
            else
                words[w] = v;
            first = false;
            ++w;
            acc <<= 32;
            nacc -= 32;
        }
    };
    const uint64_t r0 = c * 2 * K3HUF_LANE_SYMS;
    const uint64_t r1 = min(r0 + 2 * K3HUF_LANE_SYMS, raw_bytes);
    if (r1 - r0 == 2 * K3HUF_LANE_SYMS) {
        const uint4* p = reinterpret_cast<const uint4*>(raw + r0);
        for (int i = 0; i < 32; ++i) {
            const uint4 v = p[i];
            const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                put((q[k] >> 8) & 0xFFu);
                put(q[k] >> 24);
            }
            // even bytes: bytes 0, 2 of each dword
            const uint2 ev = make_uint2(__builtin_amdgcn_perm(v.y, v.x, 0x06040200u),
                                        __builtin_amdgcn_perm(v.w, v.z, 0x06040200u));
            *reinterpret_cast<uint2*>(even + 8 * i) = ev;
        }
    } else {
        for (uint64_t i = r0; i < r1; i += 2) {
            put(raw[i + 1]);
            even[(i - r0) / 2] = raw[i];
        }
    }
    if (nacc > 0) atomicOr(&words[w], bswap32(uint32_t(acc >> 32)));
}

// a kernel launch's status as a return code
int launched() { return hipGetLastError() == hipSuccess ? K3HUF_OK : K3HUF_E_HIP; }

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
    auto* status = reinterpret_cast<uint32_t*>(work + wl.status);

    // 1. per-stripe histograms (the status word is cleared with them)
    hipLaunchKernelGGL(enc_fill_zero, dim3(64), dim3(256), 0, st, reinterpret_cast<uint4*>(work),
                       wl.total / 16);
    hipLaunchKernelGGL(enc_hist, dim3(kHistBlocksPerStripe, ns), dim3(kHistThreads), 0, st, raw,
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
                       n_chunks, ct, chunk);
    hipLaunchKernelGGL(enc_scan, dim3(ns), dim3(kScanThreads), 0, st, out, geom, chunk, status);
    hipLaunchKernelGGL(enc_pack, dim3(chunk_blocks), dim3(kChunkThreads), 0, st, raw, raw_bytes,
                       n_chunks, ct, geom, chunk, out);
    if (launched()) return K3HUF_E_HIP;
    uint32_t bad = 0;
    if (hipMemcpyAsync(&bad, status, 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return K3HUF_E_HIP;
    return bad ? K3HUF_E_CORRUPT : int64_t(total);
}

}  // extern "C"
