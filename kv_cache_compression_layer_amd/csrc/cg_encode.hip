// Range encoder of the CacheGen codec on gfx950.
//
// LMCache CacheGen page (0539edu.com/news/4720135), section 4: the symbols
// are coded by CDF-driven arithmetic coding on the GPU, in batches of at most
// 256 tokens; every batch yields a byte stream plus one length per stream.
// The page does not define the coder. This library uses a byte-wise range
// coder over a 32-bit window with 16-bit tables:
//
//   r = range >> 16; low += r * cdf[s]; range = r * (cdf[s+1] - cdf[s]);
//   while range < 2^24: shift the top byte of low out, low <<= 8, range <<= 8;
//   finish with the smallest multiple of 2^24 that is >= low (one byte, or
//   none if that byte is zero or the value carries into the bytes before).
//
// A carry out of the 32-bit window must reach the bytes already emitted. The
// device coder never rewrites emitted bytes: it holds back the last byte and
// the run of 0xFF bytes after it (Subbotin/Pavlov "cache + pending" form of
// the byte range coder) and releases them once no carry can reach them. The
// bytes produced are identical to rewriting them on a carry.
//
// Work decomposition: one wave per tile of 64 streams = 64 consecutive
// channels of one (chunk, K|V, layer); lane = stream. The tile's symbols
// (<= 256 tokens x 64 channels) and its 64 tables (packed as
// start | freq << 16, laid out [symbol][lane] so lookups never conflict on
// LDS banks) are staged in LDS. Output bytes are accumulated four at a time
// in a register and stored to LDS words [word][lane], up to kStageWords per
// lane; longer streams are finished by a fix-up kernel.
//
// Streams are concatenated in stream order. The wave scans its 64 lengths,
// then finds the byte offset of the tile with a decoupled look-back over the
// tiles before it (Merrill & Garland, "Single-pass Parallel Prefix Scan with
// Decoupled Look-back", 2016); tiles take their ids from an atomic counter so
// every tile a wave waits on belongs to a wave that is already running.
#include "cg_internal.hpp"

namespace cg {

constexpr int kStageWords = 32;  // 128 bytes of staged output per stream

struct RcEnc {
    uint32_t low, range, carry, cache, nff;
    bool first;  // the held-back byte is still the leading placeholder

    __device__ __forceinline__ void init() {
        low = 0;
        range = 0xFFFFFFFFu;
        carry = 0;
        cache = 0;
        nff = 0;
        first = true;
    }

    template <class Sink>
    __device__ __forceinline__ void shift(Sink &out) {
        const uint32_t top = low >> 24;
        if (top != 0xFFu || carry) {
            if (!first) out.put((cache + carry) & 0xFFu);
            first = false;
            const uint32_t ff = (0xFFu + carry) & 0xFFu;
            for (; nff; --nff) out.put(ff);
            cache = top;
            carry = 0;
        } else {
            ++nff;
        }
        low <<= 8;
    }

    template <class Sink>
    __device__ __forceinline__ void encode(uint32_t start, uint32_t freq, Sink &out) {
        const uint32_t r = range >> 16;
        const uint32_t nl = low + __umul24(r, start);
        carry |= (uint32_t)(nl < low);
        low = nl;
        range = __umul24(r, freq);
        // range >= 2^8 here (r >= 2^8, freq >= 1), so two shifts restore it.
        if (range < kTop) {
            shift(out);
            range <<= 8;
            if (range < kTop) {
                shift(out);
                range <<= 8;
            }
        }
    }

    template <class Sink>
    __device__ __forceinline__ void flush(Sink &out) {
        const uint64_t u = (uint64_t)low + 0xFFFFFFull;
        uint32_t b = (uint32_t)(u >> 24);  // ceil(low / 2^24), 0..256
        uint32_t cc = carry;
        if (b == 256u) {  // the final value carries into the held-back bytes
            cc += 1;
            b = 0;
        }
        if (!first) out.put((cache + cc) & 0xFFu);
        const uint32_t ff = (0xFFu + cc) & 0xFFu;
        for (; nff; --nff) out.put(ff);
        if (b) out.put(b);
    }
};

// Byte sink into LDS words [word][lane]; bytes beyond the stage are counted
// but dropped (the stream is then re-encoded by the fix-up kernel).
struct LdsSink {
    uint32_t *stage;
    int lane;
    uint32_t acc, n;
    __device__ __forceinline__ void put(uint32_t b) {
        acc = (acc >> 8) | (b << 24);  // little-endian: first byte ends in bits 0..7
        ++n;
        if ((n & 3u) == 0) {
            const uint32_t w = (n >> 2) - 1;
            if (w < (uint32_t)kStageWords) stage[w * 64 + lane] = acc;
        }
    }
    __device__ __forceinline__ void finish() {
        const uint32_t k = n & 3u;
        if (k) {
            const uint32_t w = n >> 2;
            if (w < (uint32_t)kStageWords) stage[w * 64 + lane] = acc >> (8 * (4 - k));
        }
    }
};

// Byte sink straight to global memory, bounded by cap.
struct GlobalSink {
    uint8_t *base;
    uint64_t off, cap;
    uint32_t n;
    bool overflow;
    __device__ __forceinline__ void put(uint32_t b) {
        if (off + n < cap) base[off + n] = (uint8_t)b;
        else overflow = true;
        ++n;
    }
};

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o, 64);
        v += ((uint64_t)hi << 32) | lo;
    }
    return v;
}

constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagIncl = 2ull << 62;
constexpr uint64_t kValMask = (1ull << 62) - 1;

// Exclusive byte offset of `tile` in stream order. Publishes the tile's
// aggregate first, then its inclusive prefix.
__device__ uint64_t lookback(uint64_t *state, int64_t tile, uint64_t total, int lane) {
    if (tile == 0) {
        if (lane == 0)
            __hip_atomic_store(&state[0], kFlagIncl | total, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
        return 0;
    }
    if (lane == 0)
        __hip_atomic_store(&state[tile], kFlagAgg | total, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
    uint64_t excl = 0;
    int64_t idx = tile - 1;
    for (;;) {
        const int64_t my = idx - lane;
        const uint64_t v = my >= 0 ? __hip_atomic_load(&state[my], __ATOMIC_ACQUIRE,
                                                       __HIP_MEMORY_SCOPE_AGENT)
                                   : kFlagIncl;  // before tile 0: inclusive prefix 0
        const uint32_t flag = (uint32_t)(v >> 62);
        const uint64_t incl = __ballot(flag == 2);
        const uint64_t none = __ballot(flag == 0);
        const int first_incl = incl ? __ffsll((unsigned long long)incl) - 1 : 64;
        const uint64_t need = first_incl >= 63 ? ~0ull : ((2ull << first_incl) - 1);
        if (none & need) {  // a predecessor has not published yet
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        excl += wave_sum_u64(lane <= first_incl ? (v & kValMask) : 0);
        if (first_incl < 64) break;
        idx -= 64;
    }
    if (lane == 0)
        __hip_atomic_store(&state[tile], kFlagIncl | (excl + total), __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
    return excl;
}

struct EncArgs {
    const uint8_t *sym;
    const int32_t *cdf;
    uint8_t *payload;          // start of the payload
    uint64_t cap;
    uint16_t *lengths;
    uint64_t *chunk_off;
    uint64_t *size_dev;
    uint8_t *header_size;
    uint64_t payload_base;
    WsHeader *hdr;
    uint64_t *tile_state;
    uint32_t *overflow_list;
    int L, T, C, A, NC, CB;
    int64_t tiles;
    int vec16;                 // symbol rows can be staged with 16-byte loads
};

__device__ __forceinline__ void tile_coords(int64_t tile, int L, int CB, int &j, int &slab,
                                            int &cb) {
    const int64_t per_chunk = 2LL * L * CB;
    j = (int)(tile / per_chunk);
    const int64_t rem = tile - (int64_t)j * per_chunk;
    slab = (int)(rem / CB);
    cb = (int)(rem - (int64_t)slab * CB);
}

// Packed table entry of symbol s: start | freq << 16 (start <= 65535 and
// freq <= 65536 - A + 1 both fit in 16 bits).
__device__ __forceinline__ uint32_t packed_entry(const int32_t *tab, int s) {
    const uint32_t a = (uint32_t)tab[s], b = (uint32_t)tab[s + 1];
    return (a & 0xFFFFu) | ((b - a) << 16);
}

__global__ __launch_bounds__(64) void k_encode(EncArgs a) {
    extern __shared__ uint32_t smem[];
    const int lane = threadIdx.x;
    const int A = a.A;
    uint32_t *tab = smem;                                   // [A][64]
    uint8_t *symt = reinterpret_cast<uint8_t *>(tab + A * 64);  // [256][64]
    uint32_t *stage = reinterpret_cast<uint32_t *>(symt + kChunk * 64);  // [kStageWords][64]

    int64_t tile = 0;
    if (lane == 0) tile = atomicAdd(&a.hdr->tile_counter, 1u);
    tile = __shfl((int)tile, 0, 64);
    int j, slab, cb;
    tile_coords(tile, a.L, a.CB, j, slab, cb);
    const int c = cb * 64 + lane;
    const bool active = c < a.C;
    const int t0 = j * kChunk;
    const int n = min(kChunk, a.T - t0);

    // Tables: one per lane, packed, [symbol][lane].
    bool bad_table = false;
    if (active) {
        const int32_t *src = a.cdf + ((int64_t)slab * a.C + c) * (A + 1);
        bad_table = src[0] != 0 || src[A] != (int32_t)kProbOne;
        for (int s = 0; s < A; ++s) {
            const uint32_t e = packed_entry(src, s);
            bad_table |= (e >> 16) == 0;
            tab[s * 64 + lane] = (e >> 16) ? e : (e | (1u << 16));
        }
    } else {
        // Idle lanes code symbol 0 with frequency 65535: they never shift a
        // byte out, so they do not force the wave through the slow path.
        for (int s = 0; s < A; ++s) tab[s * 64 + lane] = 0xFFFFu << 16;
    }

    // Symbols of the tile: rows t0..t0+n-1, channels cb*64..cb*64+63.
    const uint8_t *sbase = a.sym + ((int64_t)slab * a.T + t0) * a.C + cb * 64;
    if (a.vec16 && cb * 64 + 64 <= a.C) {
        // 4 lanes per 64-byte row, 16 rows per instruction.
        const int r = lane >> 2, part = lane & 3;
        for (int t = r; t < n; t += 16)
            *reinterpret_cast<uint4 *>(symt + t * 64 + part * 16) =
                *reinterpret_cast<const uint4 *>(sbase + (int64_t)t * a.C + part * 16);
    } else {
        for (int t = 0; t < n; ++t) symt[t * 64 + lane] = active ? sbase[(int64_t)t * a.C + lane] : 0;
    }
    __syncthreads();

    RcEnc enc;
    enc.init();
    LdsSink sink{stage, lane, 0u, 0u};
    uint32_t bad_sym = 0;
    for (int t = 0; t < n; ++t) {
        uint32_t s = symt[t * 64 + lane];
        bad_sym |= s >= (uint32_t)A;
        s = min(s, (uint32_t)A - 1);
        const uint32_t e = tab[s * 64 + lane];
        enc.encode(e & 0xFFFFu, e >> 16, sink);
    }
    enc.flush(sink);
    sink.finish();
    const uint32_t len = active ? sink.n : 0u;
    if (__ballot((active && (bad_sym || bad_table))) && lane == 0) atomicOr(&a.hdr->status, kStCorrupt);

    if (active) a.lengths[((int64_t)j * 2 * a.L + slab) * a.C + c] = (uint16_t)len;
    const uint32_t incl = wave_incl_scan_u32(len, lane);
    const uint32_t total = (uint32_t)__shfl((int)incl, 63, 64);
    const uint32_t excl = incl - len;
    const uint64_t prefix = lookback(a.tile_state, tile, total, lane);

    // Copy the staged bytes of each lane to its place in the payload.
    const bool spilled = len > (uint32_t)(kStageWords * 4);
    const uint64_t dst = prefix + excl;
    bool over_cap = false;
    if (!spilled) {
        uint32_t w = 0;
        for (uint32_t b = 0; b < len; ++b) {
            if ((b & 3u) == 0) w = stage[(b >> 2) * 64 + lane];
            if (dst + b < a.cap) a.payload[dst + b] = (uint8_t)(w >> (8 * (b & 3u)));
            else over_cap = true;
        }
    }
    if (__ballot(spilled) && lane == 0) {
        const uint32_t slot = atomicAdd(&a.hdr->overflow_count, 1u);
        a.overflow_list[slot] = (uint32_t)tile;
    }
    if (__ballot(over_cap) && lane == 0) atomicOr(&a.hdr->status, kStCapacity);

    if (lane == 0) {
        if (slab == 0 && cb == 0) a.chunk_off[j] = prefix;
        if (tile == a.tiles - 1) {
            const uint64_t end = prefix + total;
            a.chunk_off[a.NC] = end;
            a.hdr->payload_total = end;
            if (end > a.cap) atomicOr(&a.hdr->status, kStCapacity);
            const uint64_t size = a.payload_base + end;
            if (a.size_dev) *a.size_dev = size;
            if (a.header_size)
                for (int i = 0; i < 8; ++i) a.header_size[i] = (uint8_t)(size >> (8 * i));
        }
    }
}

// Streams longer than the LDS stage: re-encode them straight into the
// payload at their final offsets (rare; the tile list comes from k_encode).
__global__ __launch_bounds__(64) void k_encode_overflow(EncArgs a) {
    const int lane = threadIdx.x;
    const uint32_t count = a.hdr->overflow_count;
    for (uint32_t i = blockIdx.x; i < count; i += gridDim.x) {
        const int64_t tile = a.overflow_list[i];
        int j, slab, cb;
        tile_coords(tile, a.L, a.CB, j, slab, cb);
        const int c = cb * 64 + lane;
        const bool active = c < a.C;
        const int t0 = j * kChunk;
        const int n = min(kChunk, a.T - t0);
        const uint32_t len = active ? a.lengths[((int64_t)j * 2 * a.L + slab) * a.C + c] : 0u;
        const uint32_t incl = wave_incl_scan_u32(len, lane);
        const uint32_t total = (uint32_t)__shfl((int)incl, 63, 64);
        const uint64_t prefix = (a.tile_state[tile] & kValMask) - total;
        if (!active || len <= (uint32_t)(kStageWords * 4)) continue;
        const int32_t *tab = a.cdf + ((int64_t)slab * a.C + c) * (a.A + 1);
        const uint8_t *sp = a.sym + ((int64_t)slab * a.T + t0) * a.C + c;
        RcEnc enc;
        enc.init();
        GlobalSink sink{a.payload, prefix + incl - len, a.cap, 0u, false};
        for (int t = 0; t < n; ++t) {
            const uint32_t s = min((uint32_t)sp[(int64_t)t * a.C], (uint32_t)a.A - 1);
            uint32_t e = packed_entry(tab, (int)s);
            if ((e >> 16) == 0) e |= 1u << 16;
            enc.encode(e & 0xFFFFu, e >> 16, sink);
        }
        enc.flush(sink);
        if (sink.overflow) atomicOr(&a.hdr->status, kStCapacity);
    }
}

hipError_t launch_encode(const Dims &d, const uint8_t *sym, const int32_t *cdf, const EncodeOut &o,
                         const EncodeWs &w, hipStream_t s) {
    EncArgs a;
    a.sym = sym;
    a.cdf = cdf;
    a.payload = o.payload;
    a.cap = o.cap;
    a.lengths = o.lengths;
    a.chunk_off = o.chunk_off;
    a.size_dev = o.size_dev;
    a.header_size = o.header_size;
    a.payload_base = o.payload_base;
    a.hdr = w.hdr;
    a.tile_state = w.tile_state;
    a.overflow_list = w.overflow_list;
    a.L = d.L;
    a.T = d.T;
    a.C = d.C;
    a.A = d.A;
    a.NC = d.NC;
    a.CB = d.CB;
    a.tiles = d.tiles;
    a.vec16 = (d.C % 16 == 0) && ((uintptr_t)sym % 16 == 0);
    const size_t lds = (size_t)d.A * 64 * 4 + (size_t)kChunk * 64 + (size_t)kStageWords * 64 * 4;
    hipLaunchKernelGGL(k_encode, dim3((unsigned)d.tiles), dim3(64), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_encode_overflow, dim3(256), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace cg
