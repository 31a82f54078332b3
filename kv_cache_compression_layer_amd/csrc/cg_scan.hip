// Byte offset of every 64-stream coder tile within the payload, on gfx950.
//
// LMCache CacheGen page (0539edu.com/news/4720135), sections 4 and 5: the
// streams of a chunk are concatenated in (K|V, layer, channel) order, and a
// stream is found again from the prefix sum of the uint16 lengths before it.
// A tile's offset is the exclusive prefix sum of the tile byte counts of its
// chunk. There are 2 * L * ceil(C / 64) tiles per chunk: few for one long
// call, very many for a batch of short calls run as one call, so the scan is
// spread over blocks of 256 tiles in three passes:
//
//   1. k_scan_local (block per 256 tiles of a segment): each tile's byte count
//      (given, or summed from its 64 lengths), the exclusive scan within the
//      block, and the block's total;
//   2. k_scan_blocks (block per segment): the exclusive scan of the block
//      totals of the segment, its total, and, for the decoder, the check of
//      the chunk against the stored chunk offsets;
//   3. k_scan_add (as pass 1): adds the block's offset (and, for the
//      decoder, the chunk offset) to every tile of the block.
//
// A batch of calls scans one segment per (chunk j, call b), whose tiles are
// contiguous (slabs are numbered call by call), and checks and offsets it
// against call b's own chunk offsets and payload.
//
// A range of chunks [j0, j0 + NCr) of one call can be scanned alone (the
// decoder of a blob whose payload has arrived up to some chunk): only those
// chunks' tiles are written and only those chunks are checked.
//
// Segments of at most 1024 tiles (2L * ceil(C / 64) of them per chunk of a
// call: 32 layers of 1024 channels, or fewer) take one launch instead,
// k_scan_seg, a block of 1024 threads per segment.
//
// Calls of at most 1024 tiles per chunk and few chunks (the 256-token
// calls LMCache makes, alone or batched: one chunk; the encoder takes up to
// four) use k_call_scan instead: one launch, one block per call, which does
// the three passes (and the encoder's chunk pass) in order within the block.
// Each of those kernels costs a few microseconds however little it does, a
// large share of a short call.
#include "cg_internal.hpp"

namespace cg {

namespace {

constexpr int kScanBlock = 256;

int64_t tiles_per_seg(const TileScan &a) { return 2LL * a.cm.Lc * a.CB; }
int64_t blocks_per_seg(const TileScan &a) { return (tiles_per_seg(a) + kScanBlock - 1) / kScanBlock; }
int segs_in_range(const TileScan &a) { return a.NCr < 0 ? a.NC * (a.L / a.cm.Lc) : a.NCr; }

// Call b of segment js and its chunk j.
__device__ __forceinline__ void seg_call(const TileScan &a, int64_t js, int &j, int &b) {
    const int B = a.L / a.cm.Lc;
    j = (int)(js / B);
    b = (int)(js - (int64_t)j * B);
}

// Payload bytes of call b (the bound of its chunk offsets).
__device__ __forceinline__ uint64_t call_payload_bytes(const TileScan &a, int b) {
    if (!a.call_sizes) return a.payload_bytes;
    uint64_t sz = a.call_sizes[b];
    if (a.cm.stride && sz > a.cm.stride) sz = a.cm.stride;
    return sz > a.payload_off ? sz - a.payload_off : 0ull;
}

// Byte count of tile tl of segment js: given (tile_sum), or the sum of its
// 64 stream lengths.
__device__ __forceinline__ uint32_t tile_bytes(const TileScan &a, int64_t js, int64_t tps, int64_t tl) {
    if (a.tile_sum) return a.tile_sum[js * tps + tl];
    int j, b;
    seg_call(a, js, j, b);
    const int64_t ls = tl / a.CB;
    const int cb = (int)(tl - ls * a.CB);
    const uint16_t *lb = call_sec(a.lengths, a.cm, b);
    const uint16_t *p = lb + ((int64_t)j * 2 * a.cm.Lc + ls) * a.C + cb * 64;
    const int nch = min(64, a.C - cb * 64);
    uint32_t v = 0;
    if (nch == 64 && a.C % 8 == 0 && ((uintptr_t)lb & 15) == 0) {
        // A full tile's 64 lengths are 128 aligned bytes: eight 16-byte
        // loads, each word holding two lengths.
        const uint4 *p4 = reinterpret_cast<const uint4 *>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint4 w = p4[i];
            v += (w.x & 0xFFFFu) + (w.x >> 16) + (w.y & 0xFFFFu) + (w.y >> 16) + (w.z & 0xFFFFu) + (w.z >> 16) +
                 (w.w & 0xFFFFu) + (w.w >> 16);
        }
    } else {
        for (int i = 0; i < nch; ++i) v += p[i];
    }
    return v;
}

// Checks chunk j of call b (decoder): its stored offsets against the bytes
// of its tiles and the call's payload.
__device__ __forceinline__ void check_chunk(const TileScan &a, int j, int b, uint64_t bytes) {
    const uint64_t *co = call_sec(a.chunk_off, a.cm, b);
    const uint64_t c0 = co[j], c1 = co[j + 1];
    const bool bad = (j == 0 && c0 != 0) || c1 < c0 || c1 - c0 != bytes || c1 > call_payload_bytes(a, b);
    if (bad) atomicOr(a.status, kStCorrupt);
}

}  // namespace

size_t tile_scan_tmp_bytes(const Dims &d) {
    const int64_t tps = 2LL * d.Lc * d.CB;
    return (size_t)(8 * (int64_t)d.NC * ncalls(d) * ((tps + kScanBlock - 1) / kScanBlock));
}

__global__ __launch_bounds__(kScanBlock) void k_scan_local(TileScan a, int64_t tps, int64_t nbps) {
    __shared__ uint32_t wsum[kScanBlock / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t bid = blockIdx.x;
    const int64_t jr = bid / nbps, blk = bid - jr * nbps, js = a.j0 + jr;
    const int64_t tl = blk * kScanBlock + tid;
    const uint32_t v = tl < tps ? tile_bytes(a, js, tps, tl) : 0u;
    const uint32_t incl = wave_incl_scan_u32(v, lane);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < kScanBlock / 64; ++k) {
        if (k < wv) before += wsum[k];
        total += wsum[k];
    }
    if (tl < tps) a.tile_off[js * tps + tl] = before + incl - v;
    if (tid == 0) a.tmp[bid] = total;
}

__global__ __launch_bounds__(kScanBlock) void k_scan_blocks(TileScan a, int64_t nbps) {
    __shared__ uint64_t wsum[kScanBlock / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t js = a.j0 + (int64_t)blockIdx.x;
    uint64_t *t = a.tmp + (int64_t)blockIdx.x * nbps;
    uint64_t run = 0;
    for (int64_t seg = 0; seg < nbps; seg += kScanBlock) {
        const int64_t i = seg + tid;
        const uint64_t v = i < nbps ? t[i] : 0ull;
        uint64_t incl = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)incl, o, 64);
            const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(incl >> 32), o, 64);
            if (lane >= o) incl += ((uint64_t)hi << 32) | lo;
        }
        if (lane == 63) wsum[wv] = incl;
        __syncthreads();
        uint64_t before = 0, total = 0;
#pragma unroll
        for (int k = 0; k < kScanBlock / 64; ++k) {
            if (k < wv) before += wsum[k];
            total += wsum[k];
        }
        if (i < nbps) t[i] = run + before + incl - v;
        run += total;
        __syncthreads();
    }
    if (tid == 0) {
        if (a.chunk_total) a.chunk_total[js] = run;
        if (a.chunk_off) {
            int j, b;
            seg_call(a, js, j, b);
            check_chunk(a, j, b, run);
        }
    }
}

__global__ __launch_bounds__(kScanBlock) void k_scan_add(TileScan a, int64_t tps, int64_t nbps) {
    const int64_t bid = blockIdx.x;
    const int64_t jr = bid / nbps, blk = bid - jr * nbps, js = a.j0 + jr;
    const int64_t tl = blk * kScanBlock + threadIdx.x;
    if (tl >= tps) return;
    uint64_t add = a.tmp[bid];
    if (a.chunk_off) {
        int j, b;
        seg_call(a, js, j, b);
        add += call_sec(a.chunk_off, a.cm, b)[j];
    }
    a.tile_off[js * tps + tl] += add;
}

// Segments of at most kSegThreads tiles: one block per segment does the
// three passes at once (its block scan is the segment's scan), as their
// last two would for a segment of one block.
constexpr int kSegThreads = 1024;

__global__ __launch_bounds__(kSegThreads) void k_scan_seg(TileScan a, int64_t tps) {
    __shared__ uint32_t wsum[kSegThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t js = a.j0 + (int64_t)blockIdx.x;
    int j, b;
    seg_call(a, js, j, b);
    const uint32_t v = tid < tps ? tile_bytes(a, js, tps, tid) : 0u;
    const uint64_t add = a.chunk_off ? call_sec(a.chunk_off, a.cm, b)[j] : 0ull;
    const uint32_t incl = wave_incl_scan_u32(v, lane);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < kSegThreads / 64; ++k) {
        if (k < wv) before += wsum[k];
        total += wsum[k];
    }
    if (tid < tps) a.tile_off[js * tps + tid] = add + before + incl - v;
    if (tid == 0) {
        if (a.chunk_total) a.chunk_total[js] = total;
        if (a.chunk_off) check_chunk(a, j, b, total);
    }
}

hipError_t launch_tile_scan(const TileScan &a, hipStream_t s) {
    if (a.NCr >= 0 && a.cm.Lc != a.L) return hipErrorInvalidValue;  // chunk ranges: one call only
    const int64_t tps = tiles_per_seg(a), nbps = blocks_per_seg(a);
    const int nseg = segs_in_range(a);
    if (tps <= kSegThreads) {
        hipLaunchKernelGGL(k_scan_seg, dim3((unsigned)nseg), dim3(kSegThreads), 0, s, a, tps);
        return hipGetLastError();
    }
    const unsigned nblk = (unsigned)(nseg * nbps);
    hipLaunchKernelGGL(k_scan_local, dim3(nblk), dim3(kScanBlock), 0, s, a, tps, nbps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_scan_blocks, dim3((unsigned)nseg), dim3(kScanBlock), 0, s, a, nbps);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_scan_add, dim3(nblk), dim3(kScanBlock), 0, s, a, tps, nbps);
    return hipGetLastError();
}

// ------------------------------------------------------ one block per call

// Calls of a few chunks, and batches of such calls, scan in one launch
// instead of three (or four, with the encoder's chunk pass): block b takes
// call b's chunks in order, kCallScanThreads tiles at a time, loads all of
// their byte counts up front (one round trip), and carries the chunk
// offsets from one chunk to the next. The decoder's form adds the stored
// chunk offset to every tile and checks each chunk, as k_scan_add and
// k_scan_blocks do; the encoder's form leaves the tile offsets relative to
// their chunk and writes what k_chunk_scan would: the chunk offsets, the
// size and the capacity check. Sums within a step fit 32 bits: 1024 tiles
// of 64 lengths below 2^16.
constexpr int kCallScanThreads = 1024, kCallScanSteps = 4;

template <bool ENC>
__global__ __launch_bounds__(kCallScanThreads) void k_call_scan(TileScan a, ChunkOut co, int64_t tps, int parts,
                                                                int nch, bool zero_status) {
    __shared__ uint32_t wsum[kCallScanThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // A one-block launch that runs before anything else sets a status bit
    // zeroes the word itself (thread 0, which alone sets bits here, and by an
    // atomic, so its later atomicOr is ordered after it).
    if (zero_status && tid == 0) atomicExch(a.status, 0u);
    const int b = blockIdx.x;
    const int B = a.L / a.cm.Lc;
    const int steps = nch * parts;
    uint32_t v[kCallScanSteps];
#pragma unroll
    for (int i = 0; i < kCallScanSteps; ++i) {
        v[i] = 0;
        const int64_t tl = (int64_t)(i % parts) * kCallScanThreads + tid;
        if (i < steps && tl < tps) v[i] = tile_bytes(a, (int64_t)(a.j0 + i / parts) * B + b, tps, tl);
    }
    uint64_t run = 0, chunk = 0;  // bytes of the call's earlier chunks; of this chunk's earlier steps
#pragma unroll
    for (int i = 0; i < kCallScanSteps; ++i) {
        if (i >= steps) break;
        const int j = a.j0 + i / parts, part = i % parts;
        const int64_t tl = (int64_t)part * kCallScanThreads + tid;
        const uint32_t incl = wave_incl_scan_u32(v[i], lane);
        if (lane == 63) wsum[wv] = incl;
        __syncthreads();
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int k = 0; k < kCallScanThreads / 64; ++k) {
            if (k < wv) before += wsum[k];
            total += wsum[k];
        }
        __syncthreads();
        if (part == 0) chunk = 0;
        if (tl < tps) {
            uint64_t off = chunk + before + incl - v[i];
            if (!ENC) off += call_sec(a.chunk_off, a.cm, b)[j];
            a.tile_off[((int64_t)j * B + b) * tps + tl] = off;
        }
        chunk += total;
        if (part == parts - 1) {
            if (tid == 0) {
                if (ENC) call_sec(co.chunk_off, a.cm, b)[j] = run;
                else check_chunk(a, j, b, chunk);
            }
            run += chunk;
        }
    }
    if (ENC && tid == 0) {
        call_sec(co.chunk_off, a.cm, b)[a.j0 + nch] = run;
        if (run > co.cap) atomicOr(a.status, kStCapacity);
        const uint64_t size = co.payload_base + run;
        if (co.size_dev) co.size_dev[b] = size;
        if (co.header_size) {
            uint8_t *h = call_sec(co.header_size, a.cm, b);
            for (int i = 0; i < 8; ++i) h[i] = (uint8_t)(size >> (8 * i));
        }
    }
}

// The decoder's form reads each tile's 64 lengths (128 bytes), so it takes
// one step: a block summing more is slower than the three passes spread
// over the chip (3 x 1024 tiles: +5 us on a 768-token call).
bool call_scan_fits(const TileScan &a) {
    const int64_t parts = (tiles_per_seg(a) + kCallScanThreads - 1) / kCallScanThreads;
    const int64_t nch = a.NCr < 0 ? a.NC : a.NCr;
    return nch * parts <= (a.tile_sum ? kCallScanSteps : 1);
}

hipError_t launch_call_scan(const TileScan &a, const ChunkOut *co, hipStream_t s, bool zero_status) {
    if (!call_scan_fits(a) || (a.NCr >= 0 && a.cm.Lc != a.L)) return hipErrorInvalidValue;
    if (zero_status && a.cm.Lc != a.L) return hipErrorInvalidValue;  // one block only
    if (co && (a.j0 != 0 || a.NCr >= 0)) return hipErrorInvalidValue;  // the encoder scans every chunk
    const int64_t tps = tiles_per_seg(a);
    const int parts = (int)((tps + kCallScanThreads - 1) / kCallScanThreads);
    const int nch = a.NCr < 0 ? a.NC : a.NCr;
    const unsigned B = (unsigned)(a.L / a.cm.Lc);
    if (co)
        hipLaunchKernelGGL(k_call_scan<true>, dim3(B), dim3(kCallScanThreads), 0, s, a, *co, tps, parts, nch,
                           zero_status);
    else
        hipLaunchKernelGGL(k_call_scan<false>, dim3(B), dim3(kCallScanThreads), 0, s, a, ChunkOut{}, tps, parts, nch,
                           zero_status);
    return hipGetLastError();
}

}  // namespace cg
