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
    uint32_t v = 0;
    if (tl < tps) {
        if (a.tile_sum) {
            v = a.tile_sum[js * tps + tl];
        } else {
            int j, b;
            seg_call(a, js, j, b);
            const int64_t ls = tl / a.CB;
            const int cb = (int)(tl - ls * a.CB);
            const uint16_t *lb = call_sec(a.lengths, a.cm, b);
            const uint16_t *p = lb + ((int64_t)j * 2 * a.cm.Lc + ls) * a.C + cb * 64;
            const int nch = min(64, a.C - cb * 64);
            if (nch == 64 && a.C % 8 == 0 && ((uintptr_t)lb & 15) == 0) {
                // A full tile's 64 lengths are 128 aligned bytes: eight
                // 16-byte loads, each word holding two lengths.
                const uint4 *p4 = reinterpret_cast<const uint4 *>(p);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint4 w = p4[i];
                    v += (w.x & 0xFFFFu) + (w.x >> 16) + (w.y & 0xFFFFu) + (w.y >> 16) + (w.z & 0xFFFFu) +
                         (w.z >> 16) + (w.w & 0xFFFFu) + (w.w >> 16);
                }
            } else {
                for (int i = 0; i < nch; ++i) v += p[i];
            }
        }
    }
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
            const uint64_t *co = call_sec(a.chunk_off, a.cm, b);
            const uint64_t c0 = co[j], c1 = co[j + 1];
            const bool bad =
                (j == 0 && c0 != 0) || c1 < c0 || c1 - c0 != run || c1 > call_payload_bytes(a, b);
            if (bad) atomicOr(a.status, kStCorrupt);
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

hipError_t launch_tile_scan(const TileScan &a, hipStream_t s) {
    if (a.NCr >= 0 && a.cm.Lc != a.L) return hipErrorInvalidValue;  // chunk ranges: one call only
    const int64_t tps = tiles_per_seg(a), nbps = blocks_per_seg(a);
    const int nseg = segs_in_range(a);
    const unsigned nblk = (unsigned)(nseg * nbps);
    hipLaunchKernelGGL(k_scan_local, dim3(nblk), dim3(kScanBlock), 0, s, a, tps, nbps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_scan_blocks, dim3((unsigned)nseg), dim3(kScanBlock), 0, s, a, nbps);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_scan_add, dim3(nblk), dim3(kScanBlock), 0, s, a, tps, nbps);
    return hipGetLastError();
}

}  // namespace cg
