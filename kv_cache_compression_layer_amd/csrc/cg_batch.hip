// Batches of to_bytes / from_bytes calls of one shape on gfx950.
//
// LMCache CacheGen page (0539edu.com/news/4720135), end-to-end benchmark:
// KV is encoded per LMCache chunk (64..768 tokens), each call with its own
// tables. B such calls of one shape [L,2,T,H,D] are laid out as [B*L,2,T,H,D]
// and coded as one virtual call of B*L layers: layer b*L + l of the virtual
// call is layer l of call b, so its scales, histograms, CDFs and streams are
// exactly those of call b alone (the per-layer constants repeat with period
// L), and only the order of the sections differs. Every per-call section
// piece is contiguous in both layouts:
//
//   piece 0, 1          scales of K, V          L*T bf16
//   piece 2, 3          CDF tables of K, V      C * (sum of the K (V) table widths) u16
//   piece 4 + 2j + kv   lengths of (chunk j, K|V)   L*C u16
//   piece 4+2NC+2j+kv   payload of (chunk j, K|V)   the streams' bytes
//
// so a batch costs one virtual call plus a plan and a copy of the blob bytes.
#include "cg_internal.hpp"

namespace cg {

namespace {

// Piece source that means "write zeros".
constexpr uint64_t kZeroFill = ~0ull;

// Offsets of the fixed pieces of call b in the virtual blob (v) and in the
// call's blob (c).
__device__ void fixed_piece(const BatchGeom &g, int b, int p, uint64_t &v, uint64_t &c, uint64_t &len) {
    const Dims &d = g.d;
    const int64_t Lv = g.vd.L;
    if (p < 2) {
        const int kv = p;
        v = g.vlay.off_scales + (uint64_t)((kv * Lv + (int64_t)b * d.L) * d.T) * 2;
        c = g.lay.off_scales + (uint64_t)((int64_t)kv * d.L * d.T) * 2;
        len = (uint64_t)d.L * d.T * 2;
    } else if (p < 4) {
        // The tables of call b's K (V) layers: in the virtual call they
        // follow the K tables of every call (for V) and those of calls < b.
        const int kv = p - 2;
        const uint64_t before = (kv ? (uint64_t)g.B * g.wsum[0] : 0) + (uint64_t)b * g.wsum[kv];
        v = g.vlay.off_cdf + before * d.C * 2;
        c = g.lay.off_cdf + (kv ? g.wsum[0] : 0) * d.C * 2;
        len = g.wsum[kv] * d.C * 2;
    } else {
        const int q = p - 4, j = q >> 1, kv = q & 1;
        v = g.vlay.off_lengths + (uint64_t)(((int64_t)j * 2 * Lv + kv * Lv + (int64_t)b * d.L) * d.C) * 2;
        c = g.lay.off_lengths + (uint64_t)(((int64_t)j * 2 * d.L + (int64_t)kv * d.L) * d.C) * 2;
        len = (uint64_t)d.L * d.C * 2;
    }
}

// Exclusive scan of one uint64 per thread over a 256-thread block.
__device__ uint64_t block_excl_scan_u64(uint64_t v, uint64_t *tmp, uint64_t &total) {
    const int tid = threadIdx.x;
    tmp[tid] = v;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const uint64_t add = tid >= o ? tmp[tid - o] : 0;
        __syncthreads();
        tmp[tid] += add;
        __syncthreads();
    }
    total = tmp[255];
    const uint64_t incl = tmp[tid];
    __syncthreads();
    return incl - v;
}

}  // namespace

// Split plan: one block per call.
__global__ __launch_bounds__(256) void k_split_plan(BatchGeom g, const uint8_t *__restrict__ vblob,
                                                    const uint64_t *__restrict__ vtile_off,
                                                    uint8_t *__restrict__ blobs, uint64_t *__restrict__ sizes_dev,
                                                    Piece *__restrict__ pieces, uint32_t *__restrict__ status) {
    __shared__ uint64_t tmp[256];
    const int b = blockIdx.x, tid = threadIdx.x;
    const Dims &d = g.d;
    const int64_t Lv = g.vd.L;
    const int NC = d.NC;
    Piece *pc = pieces + (int64_t)b * g.npieces;
    uint8_t *blob = blobs + (uint64_t)b * g.stride;
    const uint64_t *vchunk = reinterpret_cast<const uint64_t *>(vblob + g.vlay.off_chunk_off);
    const uint64_t cap = g.stride - g.lay.off_payload;
    const uint64_t vcap = (uint64_t)g.B * cap;
    for (int p = tid; p < 4 + 2 * NC; p += 256) {
        uint64_t v, c, len;
        fixed_piece(g, b, p, v, c, len);
        pc[p] = Piece{v, c, len};
    }
    // Payload pieces in the call's order (chunk j, then K, V).
    uint64_t run = 0;
    for (int base = 0; base < 2 * NC; base += 256) {
        const int i = base + tid;
        uint64_t start = 0, len = 0;
        if (i < 2 * NC) {
            const int j = i >> 1, kv = i & 1;
            const int64_t t = ((int64_t)j * 2 * Lv + kv * Lv + (int64_t)b * d.L) * d.CB;
            start = vchunk[j] + vtile_off[t];
            const bool last = kv == 1 && b == g.B - 1;
            const uint64_t end = last ? vchunk[j + 1] : vchunk[j] + vtile_off[t + (int64_t)d.L * d.CB];
            len = end - start;
        }
        uint64_t total;
        const uint64_t off = run + block_excl_scan_u64(len, tmp, total);
        if (i < 2 * NC) {
            const int j = i >> 1, kv = i & 1;
            if (kv == 0) reinterpret_cast<uint64_t *>(blob + g.lay.off_chunk_off)[j] = off;
            uint64_t n = len;
            if (off + len > cap) {
                n = off < cap ? cap - off : 0;  // the blob is too small: keep inside it
                atomicOr(status, kStCapacity);
            }
            // A call beyond the virtual payload's capacity (set by the encoder's
            // own capacity check) copies only what was written.
            if (start + n > vcap) n = start < vcap ? vcap - start : 0;
            pc[4 + 2 * NC + i] = Piece{g.vlay.off_payload + start, g.lay.off_payload + off, n};
        }
        run += total;
    }
    if (tid == 0) {
        reinterpret_cast<uint64_t *>(blob + g.lay.off_chunk_off)[NC] = run;
        const uint64_t size = g.lay.off_payload + run;
        if (size > g.stride) atomicOr(status, kStCapacity);
        sizes_dev[b] = size;
        for (int i = 0; i < 8; ++i) blob[40 + i] = (uint8_t)(size >> (8 * i));
    }
}

hipError_t launch_split_plan(const BatchGeom &g, const uint8_t *vblob, const uint64_t *vtile_off,
                             uint8_t *blobs, uint64_t *sizes_dev, Piece *pieces, uint32_t *status,
                             hipStream_t s) {
    hipLaunchKernelGGL(k_split_plan, dim3((unsigned)g.B), dim3(256), 0, s, g, vblob, vtile_off, blobs, sizes_dev,
                       pieces, status);
    return hipGetLastError();
}

// Merge, step 1 (block b per call): the bytes of the K and V streams of
// every chunk of call b, from its lengths; the check of its header, size and
// chunk offsets against them; its fixed pieces. A call whose blob does not
// check out is decoded from nothing: its length pieces are zero-filled and
// its payload pieces empty, so the other calls' streams keep their places.
__global__ __launch_bounds__(256) void k_merge_check(BatchGeom g, const uint8_t *__restrict__ blobs,
                                                     const uint64_t *__restrict__ sizes_dev, HeaderBytes hdr,
                                                     uint64_t *__restrict__ piece_len, Piece *__restrict__ pieces,
                                                     uint32_t *__restrict__ status) {
    __shared__ uint64_t tmp[256];
    __shared__ int bad_call;
    const int b = blockIdx.x, tid = threadIdx.x;
    const Dims &d = g.d;
    const int NC = d.NC;
    const uint8_t *blob = blobs + (uint64_t)b * g.stride;
    if (tid == 0) bad_call = 0;
    __syncthreads();
    const uint64_t size = sizes_dev[b];
    bool bad = size < g.lay.off_payload || size > g.stride;
    for (uint32_t i = tid; i < hdr.n; i += 256)
        if ((i < 40 || i >= 48) && blob[i] != hdr.b[i]) bad = true;
    if (tid < 8 && blob[40 + tid] != (uint8_t)(size >> (8 * tid))) bad = true;
    const uint64_t *coff = reinterpret_cast<const uint64_t *>(blob + g.lay.off_chunk_off);
    if (tid == 0 && (coff[0] != 0 || g.lay.off_payload + coff[NC] > size)) bad = true;
    const int64_t n = (int64_t)d.L * d.C;
    uint64_t *pl = piece_len + (int64_t)b * NC * 2;
    for (int j = 0; j < NC; ++j) {
        const uint16_t *len = reinterpret_cast<const uint16_t *>(blob + g.lay.off_lengths) + (int64_t)j * 2 * n;
        uint64_t sk = 0, sv = 0;
        for (int64_t i = tid; i < n; i += 256) {
            sk += len[i];
            sv += len[n + i];
        }
        uint64_t tk, tv;
        block_excl_scan_u64(sk, tmp, tk);
        block_excl_scan_u64(sv, tmp, tv);
        if (tid == 0) {
            pl[2 * j] = tk;
            pl[2 * j + 1] = tv;
            if (coff[j + 1] < coff[j] || coff[j + 1] - coff[j] != tk + tv) bad = true;
        }
    }
    if (bad) atomicOr(&bad_call, 1);
    __syncthreads();
    const bool drop = bad_call != 0;
    if (drop) {
        if (tid == 0) atomicOr(status, kStCorrupt);
        for (int i = tid; i < 2 * NC; i += 256) pl[i] = 0;
    }
    Piece *pc = pieces + (int64_t)b * g.npieces;
    for (int p = tid; p < 4 + 2 * NC; p += 256) {
        uint64_t v, c, len;
        fixed_piece(g, b, p, v, c, len);
        pc[p] = Piece{drop && p >= 4 ? kZeroFill : c, v, len};
    }
}

// Merge, step 2 (one block): the payload pieces in the virtual order (chunk
// j, K|V, call b) and the virtual chunk offsets.
__global__ __launch_bounds__(256) void k_merge_scan(BatchGeom g, const uint8_t *__restrict__ blobs,
                                                    uint8_t *__restrict__ vblob,
                                                    const uint64_t *__restrict__ piece_len,
                                                    Piece *__restrict__ pieces) {
    __shared__ uint64_t tmp[256];
    const int tid = threadIdx.x;
    const int NC = g.d.NC;
    uint64_t *vchunk = reinterpret_cast<uint64_t *>(vblob + g.vlay.off_chunk_off);
    const int64_t total_pieces = (int64_t)NC * 2 * g.B;
    uint64_t run = 0;
    for (int64_t base = 0; base < total_pieces; base += 256) {
        const int64_t i = base + tid;
        int j = 0, kv = 0, b = 0;
        uint64_t len = 0;
        if (i < total_pieces) {
            j = (int)(i / (2 * g.B));
            const int r = (int)(i - (int64_t)j * 2 * g.B);
            kv = r / g.B;
            b = r - kv * g.B;
            len = piece_len[((int64_t)b * NC + j) * 2 + kv];
        }
        uint64_t total;
        const uint64_t off = run + block_excl_scan_u64(len, tmp, total);
        if (i < total_pieces) {
            if (kv == 0 && b == 0) vchunk[j] = off;
            uint64_t src = 0;
            if (len) {
                const uint64_t *coff =
                    reinterpret_cast<const uint64_t *>(blobs + (uint64_t)b * g.stride + g.lay.off_chunk_off);
                src = g.lay.off_payload + coff[j] + (kv ? piece_len[((int64_t)b * NC + j) * 2] : 0);
            }
            pieces[(int64_t)b * g.npieces + 4 + 2 * NC + 2 * j + kv] = Piece{src, g.vlay.off_payload + off, len};
        }
        run += total;
    }
    if (tid == 0) vchunk[NC] = run;
}

hipError_t launch_merge_plan(const BatchGeom &g, const uint8_t *blobs, const uint64_t *sizes_dev,
                             const HeaderBytes &hdr, uint8_t *vblob, uint64_t *piece_len, Piece *pieces,
                             uint32_t *status, hipStream_t s) {
    hipLaunchKernelGGL(k_merge_check, dim3((unsigned)g.B), dim3(256), 0, s, g, blobs, sizes_dev, hdr, piece_len,
                       pieces, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_merge_scan, dim3(1), dim3(256), 0, s, g, blobs, vblob, piece_len, pieces);
    return hipGetLastError();
}

// Copy of every piece; blockIdx = (piece * kSlices + slice, call). The
// destination is written in aligned dwords; a source dword at any byte
// offset is joined from the two aligned dwords that hold it (the second is
// read only when the offset is not a multiple of 4, so no read leaves a
// dword that holds a byte of the piece).
constexpr int kSlices = 8;

__device__ __forceinline__ uint32_t load_u32_any(const uint8_t *p) {
    const uintptr_t a = (uintptr_t)p;
    const uint32_t *w = reinterpret_cast<const uint32_t *>(a & ~(uintptr_t)3);
    const uint32_t sh = (uint32_t)(a & 3);
    const uint32_t w0 = w[0];
    if (sh == 0) return w0;
    return __builtin_amdgcn_alignbyte(w[1], w0, sh);
}

__global__ __launch_bounds__(256) void k_copy_pieces(const Piece *__restrict__ pieces, int npieces,
                                                     const uint8_t *__restrict__ src_base, uint64_t src_stride,
                                                     uint8_t *__restrict__ dst_base, uint64_t dst_stride) {
    const int b = blockIdx.y;
    const int p = blockIdx.x / kSlices, sl = blockIdx.x - p * kSlices;
    const Piece pc = pieces[(int64_t)b * npieces + p];
    if (pc.len == 0) return;
    uint8_t *dst = dst_base + (uint64_t)b * dst_stride + pc.dst;
    const bool zero = pc.src == kZeroFill;
    const uint8_t *src = zero ? nullptr : src_base + (uint64_t)b * src_stride + pc.src;
    // Head bytes up to a 4-byte aligned destination, then dwords, then tail.
    const uint64_t mis = (4 - ((uintptr_t)dst & 3)) & 3;
    const uint64_t head = mis < pc.len ? mis : pc.len;
    const uint64_t nw = (pc.len - head) / 4;
    const uint64_t per = (nw + kSlices - 1) / kSlices;
    const uint64_t lo = (uint64_t)sl * per, hi = min(nw, lo + per);
    const int tid = threadIdx.x;
    uint32_t *dw = reinterpret_cast<uint32_t *>(dst + head);
    const uint8_t *sw = zero ? nullptr : src + head;
    uint64_t i = lo + tid;
    if (zero) {
        for (; i < hi; i += 256) dw[i] = 0;
    } else {
        for (; i + 3 * 256 < hi; i += 4 * 256) {
            uint32_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = load_u32_any(sw + 4 * (i + u * 256));
#pragma unroll
            for (int u = 0; u < 4; ++u) dw[i + u * 256] = v[u];
        }
        for (; i < hi; i += 256) dw[i] = load_u32_any(sw + 4 * i);
    }
    if (sl == kSlices - 1) {
        const uint64_t t0 = head + 4 * nw;
        for (uint64_t k = (uint64_t)tid; k < pc.len - t0; k += 256) dst[t0 + k] = zero ? 0 : src[t0 + k];
    }
    if (sl == 0 && (uint64_t)tid < head) dst[tid] = zero ? 0 : src[tid];
}

hipError_t launch_copy_pieces(const BatchGeom &g, const Piece *pieces, const uint8_t *src_base,
                              uint64_t src_stride, uint8_t *dst_base, uint64_t dst_stride, hipStream_t s) {
    hipLaunchKernelGGL(k_copy_pieces, dim3((unsigned)(g.npieces * kSlices), (unsigned)g.B), dim3(256), 0, s, pieces,
                       g.npieces, src_base, src_stride, dst_base, dst_stride);
    return hipGetLastError();
}

}  // namespace cg
