// Internal declarations shared by the HIP translation units of
// libcachegen_mi355x.so. Nothing here is part of the C ABI.
//
// Target: gfx950 (CDNA4), wave64. Layout conventions follow include/cachegen.h.
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cachegen.h"

namespace cg {

constexpr int kChunk = CG_CHUNK_TOKENS;   // tokens per coder stream
constexpr int kWave = 64;
constexpr uint32_t kTop = 1u << 24;       // renormalise while range < 2^24
constexpr uint32_t kProbOne = 1u << 16;   // total frequency of every table

// Status bits kept in the first word of every workspace.
constexpr uint32_t kStNonfinite = 1u;
constexpr uint32_t kStCorrupt = 2u;
constexpr uint32_t kStCapacity = 4u;

// Per-(K|V, layer) bins, passed by value to every kernel that needs them
// (2 KiB of kernel arguments): the quantisation constant M = bins//2 - 1 and
// the table width W (the call's alphabet A, or with per-layer tables the
// layer's bins) follow from them.
struct MaxTable {
    uint8_t bins[2][CG_MAX_LAYERS];  // [K|V][layer of a call]
    int32_t per_layer;  // table format: 0 = width A for all tables, 1 = width = the layer's bins
    int32_t A;
};

// l: the layer within its call (SlabLoc::l).
__device__ __forceinline__ int layer_bins(const MaxTable &mt, int kv, int l) { return mt.bins[kv][l]; }
__device__ __forceinline__ int layer_m(const MaxTable &mt, int kv, int l) { return (layer_bins(mt, kv, l) >> 1) - 1; }
__device__ __forceinline__ int layer_w(const MaxTable &mt, int kv, int l) {
    return mt.per_layer ? layer_bins(mt, kv, l) : mt.A;
}

// A batch of B calls of one shape [Lc, 2, T, H, D] runs as one call of
// L = B * Lc layers, whose KV is [B * Lc, 2, T, H, D]. Its (K|V, layer)
// slabs are numbered call by call: slab vs = b * 2Lc + kv * Lc + l is (K|V
// kv, layer l) of call b, which is layer b * Lc + l of the batch's KV. A
// single call is the batch of one (Lc = L: vs = kv * L + l). Workspace
// arrays (symbols, counts, tile sums and offsets, staging) are indexed by
// vs, and the tiles of (chunk j, call b) are contiguous: tile (j * 2L + vs)
// * CB + cb. The blob sections of call b (scales, tables, lengths, chunk
// offsets, payload) lie b * stride bytes after those of call 0 and are
// indexed as in a call of its own (slab ls = vs - b * 2Lc), so each call's
// blob is the blob of that call alone.
struct CallMap {
    int Lc;           // layers per call
    uint64_t stride;  // bytes between the blob sections of consecutive calls (one call: 0)
};
struct SlabLoc {
    int b;   // call
    int ls;  // slab within the call, kv * Lc + l
    int kv;  // 0 = K, 1 = V
    int l;   // layer within the call
    int lv;  // layer within the batch, b * Lc + l
};
__host__ __device__ __forceinline__ SlabLoc slab_loc(const CallMap &m, int vs) {
    SlabLoc s;
    s.b = vs / (2 * m.Lc);
    s.ls = vs - s.b * 2 * m.Lc;
    s.kv = s.ls >= m.Lc ? 1 : 0;
    s.l = s.ls - s.kv * m.Lc;
    s.lv = s.b * m.Lc + s.l;
    return s;
}
// Section pointer of call b (null stays null).
template <class T>
__host__ __device__ __forceinline__ T *call_sec(T *p, const CallMap &m, int b) {
    if (!p) return p;
    return reinterpret_cast<T *>(reinterpret_cast<uintptr_t>(p) + (uint64_t)b * m.stride);
}

// Derived sizes of one call.
struct Dims {
    int L, T, H, D, C, A, NC;
    int Lc;          // layers per call (a batch of L / Lc calls; one call: Lc = L)
    uint64_t cstride;  // bytes between consecutive calls' blob sections (one call: 0)
    int fmt;         // table format (CG_TABLES_*)
    int wmin;        // narrowest table width of the call
    int64_t tab_entries;  // sum of the table widths over the 2L (K|V, layer) slabs
    int CB;          // 64-channel blocks per (kv, layer): ceil(C / 64)
    int64_t N;       // 2*L*T*C symbols
    int64_t NS;      // NC*2*L*C streams
    int64_t tiles;   // NC*2*L*CB coder tiles (64 streams each)
};
inline CallMap call_map(const Dims &d) { return CallMap{d.Lc, d.cstride}; }
inline int ncalls(const Dims &d) { return d.L / d.Lc; }

// Header of every workspace (first 256 bytes).
struct WsHeader {
    uint32_t status;
    uint32_t pad[63];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

// Blob layout (matches cg_blob_info).
struct BlobLayout {
    uint64_t header_bytes, off_scales, off_cdf, off_chunk_off, off_lengths, off_payload;
};

// ---------------------------------------------------------------- launchers
// All return hipSuccess or the launch error. Sizes are validated by the API.

hipError_t launch_fill_u32(uint32_t *p, uint32_t v, int64_t n, hipStream_t s);

hipError_t launch_quantize(const Dims &d, const MaxTable &mt, const uint16_t *kv, uint8_t *sym,
                           uint16_t *scale, uint32_t *status, hipStream_t s);

hipError_t launch_histogram(const Dims &d, const uint8_t *sym, uint32_t *counts, uint32_t *status,
                            hipStream_t s);

// Quantise and histogram in one pass (counts must be zero on entry); only
// for the shapes quantize_hist_fits() accepts. When one block covers a whole
// (K|V, layer) slab (quantize_hist_fuses_cdf), the block builds the slab's
// u16 CDF tables itself: pass `wire` and no counts are written (nor read).
bool quantize_hist_fits(const Dims &d, const void *kv, const void *sym);
bool quantize_hist_fuses_cdf(const Dims &d, const void *wire);
// packed: write the symbols in the encoder's packed layout (T % 8 == 0; see
// k_quantize_hist), as encode_packs() decides; nibbles: the slabs of at most
// 16 symbols as nibbles, as encode_nibbles() decides (else bytes).
hipError_t launch_quantize_hist(const Dims &d, const MaxTable &mt, const uint16_t *kv, uint8_t *sym,
                                uint16_t *scale, uint32_t *counts, uint16_t *wire, const uint32_t *wpre,
                                uint32_t *status, bool packed, bool nibbles, hipStream_t s);

// Table placement: table (slab, c) of width W = layer_w starts at entry
// wpre[slab] * C + c * W of the u16 wire section; wpre[2L] = the section's
// entries / C. With one width A for every table wpre is not needed (null:
// wpre[slab] = slab * A). The int32 tables are [2,L,C,A+1] whatever W
// (entries past W hold 2^16).
hipError_t launch_table_prefix(const Dims &d, const MaxTable &mt, uint32_t *wpre, hipStream_t s);

// counts -> cdf int32 [2,L,C,A+1] and / or the u16 wire form (either may be
// null; the wire form needs wpre).
hipError_t launch_cdf(const Dims &d, const MaxTable &mt, const uint32_t *counts, int32_t *cdf,
                      uint16_t *cdf_wire, const uint32_t *wpre, uint32_t *status, hipStream_t s);

// Tile offsets in stream order (three passes over blocks of 256 tiles). The
// scan runs over segments of 2Lc * CB tiles, one per (chunk j, call b),
// segment j * B + b. The byte count of each tile is tile_sum[t], or, with
// tile_sum null, the sum of its 64 lengths. Offsets are relative to the
// segment, or, with chunk_off set, absolute within the call's payload, each
// segment then checked against the call's chunk offsets (kStCorrupt).
struct TileScan {
    const uint32_t *tile_sum;    // [tiles] or null
    const uint16_t *lengths;     // call 0's [NC,2,Lc,C] when tile_sum is null
    uint64_t *tile_off;          // out [tiles]
    uint64_t *tmp;               // tile_scan_tmp_bytes(d)
    uint64_t *chunk_total;       // out [NC * B] (segment j * B + b), or null
    const uint64_t *chunk_off;   // call 0's [NC+1], or null
    uint64_t payload_bytes;      // bound of chunk_off (with chunk_off)
    // With call_sizes (device, [B]): call b's bound is min(call_sizes[b],
    // stride) - payload_off instead (0 if below).
    const uint64_t *call_sizes;
    uint64_t payload_off;
    uint32_t *status;
    int L, C, CB, NC;
    CallMap cm;
    int j0 = 0, NCr = -1;        // chunks [j0, j0 + NCr) only (NCr < 0: all NC; one call only)
};
size_t tile_scan_tmp_bytes(const Dims &d);
hipError_t launch_tile_scan(const TileScan &a, hipStream_t s);

// The encoder's chunk offsets (call 0's [NC+1]), sizes ([B] or null), the
// header's size field (call 0's or null), the payload's offset in the blob
// and each call's payload capacity.
struct ChunkOut {
    uint64_t *chunk_off = nullptr;
    uint64_t *size_dev = nullptr;
    uint8_t *header_size = nullptr;
    uint64_t payload_base = 0, cap = 0;
};
// One launch for the tile scan of calls of a few chunks (and, with co, the
// encoder's chunk offsets and sizes); call_scan_fits says which calls.
// zero_status (one call only): the kernel zeroes the status word first.
bool call_scan_fits(const TileScan &a);
hipError_t launch_call_scan(const TileScan &a, const ChunkOut *co, hipStream_t s, bool zero_status = false);

// Blob sections of call 0 (call b's lie b * stride bytes further, see
// CallMap); cap is each call's payload capacity.
struct EncodeOut {
    uint8_t *payload;
    uint64_t cap;
    uint16_t *lengths;
    uint64_t *chunk_off;
    uint64_t *size_dev;       // optional: [B], receives payload_base + each call's total
    uint8_t *header_size;     // optional: 8 bytes in the blob header for the size
    uint64_t payload_base;    // offset of the payload within the blob (0 for stage calls)
};

struct EncodeWs {
    WsHeader *hdr;
    uint32_t *tile_sum;       // [tiles] bytes of each 64-stream tile
    uint8_t *tile_mode;       // [tiles] how the tile's bytes were left in its staging slot
    uint64_t *tile_off;       // [tiles] offset of each tile within its chunk
    uint64_t *chunk_total;    // [NC] bytes of each chunk
    uint8_t *staging;         // encode_staging_bytes(d)
    uint64_t *scan_tmp;       // tile_scan_tmp_bytes(d)
};

// Bytes of the staging area k_encode needs (one slot per tile).
size_t encode_staging_bytes(const Dims &d);

// Tables: int32 [2,L,C,A+1] (cdf32) or the u16 wire form [2,L,C,A] (cdf16,
// entry A taken as 2^16); exactly one is set. trusted: the symbols come from
// this library's quantiser (all below A), so the encoder skips its range
// check.
// packed: the symbols are in the quantiser's packed layout (only with
// trusted symbols, and only where encode_packs() holds).
hipError_t launch_encode(const Dims &d, const MaxTable &mt, const uint8_t *sym, const int32_t *cdf32,
                         const uint16_t *cdf16, const uint32_t *wpre, const EncodeOut &o, const EncodeWs &w,
                         bool trusted, bool packed, hipStream_t s);

// Whether the trusted encoder can read packed symbols for this call (T % 8
// == 0), and whether its slabs of at most 16 symbols are read as nibbles:
// only when they have a launch of 16-entry tables of their own (bytes when
// one launch sees both kinds of slabs).
bool encode_packs(const Dims &d, const MaxTable &mt);
bool encode_nibbles(const Dims &d, const MaxTable &mt);

// Decoder table source: int32 [2,L,C,A+1] or the u16 wire form [2,L,C,A].
struct DecodeIn {
    const uint8_t *payload;
    uint64_t payload_bytes;
    const uint16_t *lengths;
    const uint64_t *chunk_off;
    const int32_t *cdf32;      // one of cdf32 / cdf16 is set
    const uint16_t *cdf16;
    uint32_t *wpre;            // with cdf16: table offsets, filled by launch_decode
    int j0 = 0, j1 = -1;       // decode chunks [j0, j1) only (j1 < 0: all); their tokens are written
    // Batches: each call's payload bound from its blob size (see TileScan).
    const uint64_t *call_sizes = nullptr;
    uint64_t payload_off = 0;
    // The status word still has to be zeroed: launch_decode does it before
    // any kernel can set a bit (in the scan kernel when that is one block).
    bool zero_status = false;
};

// Paged output of the fused decoder: element (l, kv, t, c) goes to
// cache[l*layer_stride + kv*kv_stride + (table[t >> log2_bs] << log2_bs |
// (t & (bs-1))) * C + c] (bf16 elements).
struct PagedOut {
    uint16_t *cache;           // null: contiguous output
    int64_t layer_stride, kv_stride;
    int log2_bs;
    const int32_t *table;      // [ceil(T / bs)] physical block of each logical block
    int32_t num_blocks;
};

struct DecodeOut {
    uint8_t *sym;              // stage output, or
    uint16_t *kv;              // fused dequantised bf16 output [L,2,T,C]
    const uint16_t *scale;     // bf16 [2,L,T] (fused only)
    PagedOut paged;            // fused output through a block table (cache != null)
};

hipError_t launch_decode(const Dims &d, const MaxTable &mt, const DecodeIn &in, const DecodeOut &out,
                         uint64_t *tile_off, uint64_t *scan_tmp, uint32_t *status, hipStream_t s);

hipError_t launch_dequantize(const Dims &d, const MaxTable &mt, const uint8_t *sym,
                             const uint16_t *scale, uint16_t *kv_out, hipStream_t s);

// Writes the blob header bytes (passed by value) and zeroes the section gaps.
struct HeaderBytes {
    uint8_t b[2048 + 64];
    uint32_t n;
};
// With status, also zeroes that workspace status word.
hipError_t launch_blob_header(uint8_t *blob, const HeaderBytes &h, const BlobLayout &lay,
                              const Dims &d, hipStream_t s, int nblobs = 1, uint64_t stride = 0,
                              uint32_t *status = nullptr);

// Batch decode: checks each call's blob header (all but the size field)
// against hdr and its size against the header and the stride; a call that
// fails records kStCorrupt.
hipError_t launch_batch_check(const uint8_t *blobs, uint64_t stride, int B, const uint64_t *sizes_dev,
                              const HeaderBytes &hdr, uint64_t off_payload, uint32_t *status, hipStream_t s);

// ----------------------------------------------------------- device helpers

// Buffer resource (V#) over [base, base + bytes) for raw byte-offset loads and
// stores; word 3 is the gfx9-family value for untyped buffer access. With a
// 32-bit row offset in an SGPR and the lane's offset in a VGPR, the access
// needs no per-lane address arithmetic. An access whose lane offset lies
// beyond `bytes` is dropped (stores) or reads 0 (loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2): block b runs on XCD b % 8. This maps block b to a work index such that
// consecutive work indices run on the same XCD, so neighbouring tiles that
// share cache lines share an L2. A bijection on [0, n).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_work_index(int b, int n) {
    const int per = n / kXcds;
    if (b >= per * kXcds) return b;
    return (b % kXcds) * per + b / kXcds;
}

// round_half_even(num / T) for num < 2^48: a double-precision quotient is
// within one of the true quotient; the integer remainder fixes it exactly.
__device__ __forceinline__ uint64_t div_rne(uint64_t num, uint32_t T, double invT) {
    int64_t q = (int64_t)((double)num * invT);
    int64_t r = (int64_t)num - q * (int64_t)T;
    while (r < 0) { --q; r += T; }
    while (r >= (int64_t)T) { ++q; r -= T; }
    if (2 * r > (int64_t)T || (2 * r == (int64_t)T && (q & 1))) ++q;
    return (uint64_t)q;
}

// Start and end of symbol s < W of table (slab, c): from the int32 tables
// [2L, C, A+1], or from the u16 wire tables placed by wpre (or [2L, C, A]
// when wpre is null); exactly one of c32 / c16 set; entry W of a wire table
// is 2^16.
__device__ __forceinline__ void cdf_bounds(const int32_t *c32, const uint16_t *c16, const uint32_t *wpre, int slab,
                                           int C, int c, int A, int W, int s, uint32_t &lo, uint32_t &hi) {
    if (c16) {
        const uint16_t *w = c16 + (wpre ? (int64_t)wpre[slab] : (int64_t)slab * A) * C + (int64_t)c * W;
        lo = w[s];
        hi = s + 1 < W ? (uint32_t)w[s + 1] : kProbOne;
    } else {
        const int32_t *p = c32 + ((int64_t)slab * C + c) * (A + 1);
        lo = (uint32_t)p[s];
        hi = (uint32_t)p[s + 1];
    }
}

// One lane's table, as cdf_bounds reads it: the wire table w (u16, W
// entries, entry W being 2^16) when p is null, else the int32 table p.
struct LaneTable {
    const int32_t *p;
    const uint16_t *w;
    int W;
};

__device__ __forceinline__ LaneTable lane_table(const int32_t *c32, const uint16_t *c16, const uint32_t *wpre,
                                                int slab, int C, int c, int A, int W) {
    LaneTable t;
    t.W = W;
    t.p = c16 ? nullptr : c32 + ((int64_t)slab * C + c) * (A + 1);
    t.w = c16 ? c16 + (wpre ? (int64_t)wpre[slab] : (int64_t)slab * A) * C + (int64_t)c * W : nullptr;
    return t;
}

// Bounds of symbols first + k * step, k < N, with every load issued before
// the first result is used. Indexes are clamped into the table, so symbols
// at or past W get meaningless values that callers must not use.
template <int N>
__device__ __forceinline__ void lane_bounds_n(const LaneTable &t, int first, int step, uint32_t (&lo)[N],
                                              uint32_t (&hi)[N]) {
    const int W = t.W;
    if (!t.p) {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int s = first + k * step;
            lo[k] = t.w[min(s, W - 1)];
            hi[k] = t.w[min(s + 1, W - 1)];
        }
#pragma unroll
        for (int k = 0; k < N; ++k)
            if (first + k * step + 1 >= W) hi[k] = kProbOne;
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int s = first + k * step;
            lo[k] = (uint32_t)t.p[min(s, W)];
            hi[k] = (uint32_t)t.p[min(s + 1, W)];
        }
    }
}

// Calls f(s, lo, hi) for the symbols s = first + k * step < limit, k < N,
// with cdf_bounds' lo and hi (meaningless for s >= W). The loads go out G
// symbols at a time, one memory round trip per group instead of one per
// symbol (which short calls, one wave per SIMD, cannot hide); the compiler
// barrier after each group keeps the next group's loads behind this one's
// uses, so no more than G symbols' values are live. limit is wave-uniform.
constexpr int kTabGroup = 8;  // table symbols per load group

template <int N, int G, class F>
__device__ __forceinline__ void for_lane_bounds(const LaneTable &t, int first, int step, int limit, F &&f) {
#pragma unroll
    for (int k0 = 0; k0 < N; k0 += G) {
        if (first + k0 * step < limit) {
            uint32_t lo[G], hi[G];
            lane_bounds_n<G>(t, first + k0 * step, step, lo, hi);
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const int s = first + (k0 + k) * step;
                if (k0 + k < N && s < limit) f(s, lo[k], hi[k]);
            }
            __asm__ volatile("" ::: "memory");
        }
    }
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

// Inclusive prefix sum across the wave.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t t = (uint32_t)__shfl_up((int)v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

}  // namespace cg
