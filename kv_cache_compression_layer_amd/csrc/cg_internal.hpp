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

// Per-(K|V, layer) quantisation constant M = bins//2 - 1, passed by value to
// every kernel that needs it (2 KiB of kernel arguments).
struct MaxTable {
    uint8_t m[2][CG_MAX_LAYERS];
};

// Derived sizes of one call.
struct Dims {
    int L, T, H, D, C, A, NC;
    int CB;          // 64-channel blocks per (kv, layer): ceil(C / 64)
    int64_t N;       // 2*L*T*C symbols
    int64_t NS;      // NC*2*L*C streams
    int64_t tiles;   // NC*2*L*CB coder tiles (64 streams each)
};

// Header of every workspace (first 256 bytes).
struct WsHeader {
    uint32_t status;
    uint32_t reserved0;
    uint32_t overflow_count;   // tiles whose streams did not fit in LDS
    uint32_t pad0;
    uint64_t payload_total;    // sum of all stream lengths (encode)
    uint32_t pad[58];
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
// for the shapes quantize_hist_fits() accepts.
bool quantize_hist_fits(const Dims &d, const void *kv, const void *sym);
hipError_t launch_quantize_hist(const Dims &d, const MaxTable &mt, const uint16_t *kv, uint8_t *sym,
                                uint16_t *scale, uint32_t *counts, uint32_t *status, hipStream_t s);

// counts -> cdf int32 [2,L,C,A+1]; optionally the u16 wire form [2,L,C,A].
hipError_t launch_cdf(const Dims &d, const uint32_t *counts, int32_t *cdf, uint16_t *cdf_wire,
                      uint32_t *status, hipStream_t s);

struct EncodeOut {
    uint8_t *payload;
    uint64_t cap;
    uint16_t *lengths;
    uint64_t *chunk_off;
    uint64_t *size_dev;       // optional: receives payload_base + total
    uint8_t *header_size;     // optional: 8 bytes in the blob header for the size
    uint64_t payload_base;    // offset of the payload within the blob (0 for stage calls)
};

struct EncodeWs {
    WsHeader *hdr;
    uint32_t *tile_sum;       // [tiles] bytes of each 64-stream tile
    uint64_t *tile_off;       // [tiles] offset of each tile within its chunk
    uint64_t *chunk_total;    // [NC] bytes of each chunk
    uint32_t *overflow_list;  // [tiles] tiles with a stream beyond the LDS stage
    uint8_t *staging;         // encode_staging_bytes(d)
};

// Bytes of the staging area k_encode needs (one slot per tile).
size_t encode_staging_bytes(const Dims &d);

// trusted: the symbols come from this library's quantiser (all below A), so
// the encoder skips its range check.
hipError_t launch_encode(const Dims &d, const uint8_t *sym, const int32_t *cdf, const EncodeOut &o,
                         const EncodeWs &w, bool trusted, hipStream_t s);

// Decoder table source: int32 [2,L,C,A+1] or the u16 wire form [2,L,C,A].
struct DecodeIn {
    const uint8_t *payload;
    uint64_t payload_bytes;
    const uint16_t *lengths;
    const uint64_t *chunk_off;
    const int32_t *cdf32;      // one of cdf32 / cdf16 is set
    const uint16_t *cdf16;
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
                         uint64_t *tile_off, uint32_t *status, hipStream_t s);

hipError_t launch_dequantize(const Dims &d, const MaxTable &mt, const uint8_t *sym,
                             const uint16_t *scale, uint16_t *kv_out, hipStream_t s);

// Writes the blob header bytes (passed by value) and zeroes the section gaps.
struct HeaderBytes {
    uint8_t b[2048 + 64];
    uint32_t n;
};
hipError_t launch_blob_header(uint8_t *blob, const HeaderBytes &h, const BlobLayout &lay,
                              const Dims &d, hipStream_t s);

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
