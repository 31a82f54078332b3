// Range decoder (and fused dequantisation) of the CacheGen codec on gfx950.
//
// LMCache CacheGen page (0539edu.com/news/4720135), section 5: every
// (layer, channel) stream is restored from the CDF and the prefix sums of the
// stream lengths, the symbols are reshaped to [2, L, T, C], and dequantised
// as t = (t - M) / M * scale before being stacked back to [L, 2, T, H, D] in
// the input dtype.
//
// Pass 1 (k_lenscan, one block per 256-token chunk) turns the uint16 lengths
// into the byte offset of every 64-stream tile: the chunk offset plus the
// prefix sum of the lengths before it, and checks that the chunk's lengths
// add up to the next chunk offset.
//
// Pass 2 (k_decode, one wave per tile, lane = stream) copies the tile's
// bytes (contiguous in the payload) into LDS with the 64 lanes reading
// consecutive words, stages the 64 tables as start | freq << 16 [symbol][lane]
// and decodes. The symbol is the largest s with r * cdf[s] <= code, found by
// a branch-free binary search over the LDS table; comparing r * cdf[s] with
// code is the same test as cdf[s] <= floor(code / r), so no division is
// needed. Renormalisation is two predicated steps (the window never needs
// more). The fused variant multiplies by the per-token scale and writes bf16
// directly, so the symbols never reach memory.
#include "cg_internal.hpp"

namespace cg {

constexpr int kStageBytes = 8192;  // LDS bytes for a tile's payload

// Block-wide exclusive scan of one uint32 per thread (256 threads).
__device__ __forceinline__ uint32_t block_excl_scan_256(uint32_t v, uint32_t *tmp,
                                                        uint32_t &total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan_u32(v, lane);
    if (lane == 63) tmp[wv] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int i = 0; i < wv; ++i) before += tmp[i];
    total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
    __syncthreads();
    return before + incl - v;
}

__global__ __launch_bounds__(256) void k_lenscan(const uint16_t *__restrict__ lengths,
                                                 const uint64_t *__restrict__ chunk_off,
                                                 uint64_t *__restrict__ tile_off,
                                                 uint32_t *__restrict__ status, int L, int C,
                                                 int CB, int NC, uint64_t payload_bytes) {
    __shared__ uint32_t tmp[4];
    const int j = blockIdx.x;
    const int ntc = 2 * L * CB;
    uint64_t base = chunk_off[j];
    for (int seg = 0; seg < ntc; seg += 256) {
        const int tl = seg + threadIdx.x;
        uint32_t sum = 0;
        if (tl < ntc) {
            const int slab = tl / CB, cb = tl - slab * CB;
            const uint16_t *p = lengths + ((int64_t)j * 2 * L + slab) * C + cb * 64;
            const int nch = min(64, C - cb * 64);
            for (int i = 0; i < nch; ++i) sum += p[i];
        }
        uint32_t total;
        const uint32_t excl = block_excl_scan_256(sum, tmp, total);
        if (tl < ntc) tile_off[(int64_t)j * ntc + tl] = base + excl;
        base += total;
    }
    if (threadIdx.x == 0) {
        const bool bad = (j == 0 && chunk_off[0] != 0) || base != chunk_off[j + 1] ||
                         chunk_off[j + 1] > payload_bytes;
        if (bad) atomicOr(status, kStCorrupt);
    }
}

struct DecArgs {
    const uint8_t *payload;
    uint64_t payload_bytes;
    const uint16_t *lengths;
    const uint64_t *tile_off;
    const int32_t *cdf32;
    const uint16_t *cdf16;
    uint8_t *sym;
    uint16_t *kv;
    const uint16_t *scale;
    uint32_t *status;
    MaxTable mt;
    int L, T, C, A, CB;
};

template <int LOGA, bool FUSED>
__global__ __launch_bounds__(64) void k_decode(DecArgs a) {
    extern __shared__ uint32_t smem[];
    const int lane = threadIdx.x;
    const int A = a.A;
    uint32_t *tab = smem;                                            // [A][64]
    uint32_t *bytes_w = tab + A * 64;                                // kStageBytes/4 words
    float *sc = reinterpret_cast<float *>(bytes_w + kStageBytes / 4);  // [256]
    float *dq = sc + kChunk;                                          // [128]
    const uint8_t *bytes = reinterpret_cast<const uint8_t *>(bytes_w);

    const int64_t tile = blockIdx.x;
    const int64_t per_chunk = 2LL * a.L * a.CB;
    const int j = (int)(tile / per_chunk);
    const int rem = (int)(tile - (int64_t)j * per_chunk);
    const int slab = rem / a.CB, cb = rem - slab * a.CB;
    const int kv = slab / a.L, l = slab - kv * a.L;
    const int c = cb * 64 + lane;
    const bool active = c < a.C;
    const int t0 = j * kChunk;
    const int n = min(kChunk, a.T - t0);

    uint32_t len = active ? a.lengths[((int64_t)j * 2 * a.L + slab) * a.C + c] : 0u;
    const uint32_t incl = wave_incl_scan_u32(len, lane);
    uint32_t total = (uint32_t)__shfl((int)incl, 63, 64);
    uint32_t excl = incl - len;
    const uint64_t base = a.tile_off[tile];
    bool corrupt = false;
    if (base > a.payload_bytes || total > a.payload_bytes - base) {
        corrupt = true;  // offsets point outside the payload: decode from nothing
        len = 0;
        excl = 0;
        total = 0;
    }

    // Stage the tile's bytes: words from the aligned start, bounded by the payload.
    const bool staged = total <= (uint32_t)(kStageBytes - 8);
    const uint64_t abase = base & ~3ull;
    const uint32_t head = (uint32_t)(base - abase);
    if (staged && total) {
        const uint32_t nw = (head + total + 3) >> 2;
        for (uint32_t w = lane; w < nw; w += 64) {
            const uint64_t g = abase + 4ull * w;
            uint32_t v;
            if (g + 4 <= a.payload_bytes) {
                v = *reinterpret_cast<const uint32_t *>(a.payload + g);
            } else {
                v = 0;
                for (int i = 0; i < 4; ++i)
                    if (g + i < a.payload_bytes) v |= (uint32_t)a.payload[g + i] << (8 * i);
            }
            bytes_w[w] = v;
        }
    }

    // Tables.
    bool bad_table = false;
    if (active) {
        const int64_t row = (int64_t)slab * a.C + c;
        uint32_t prev = 0;
        for (int s = 0; s < A; ++s) {
            uint32_t nxt;
            if (a.cdf32) {
                if (s == 0) prev = (uint32_t)a.cdf32[row * (A + 1)];
                nxt = (uint32_t)a.cdf32[row * (A + 1) + s + 1];
            } else {
                if (s == 0) prev = a.cdf16[row * A];
                nxt = s + 1 < A ? (uint32_t)a.cdf16[row * A + s + 1] : kProbOne;
            }
            if (s == 0) bad_table |= prev != 0;
            uint32_t f = nxt - prev;
            if (nxt <= prev || nxt > kProbOne) {
                bad_table = true;
                f = 1;
            }
            tab[s * 64 + lane] = (prev & 0xFFFFu) | (f << 16);
            prev = nxt;
        }
        if (a.cdf32) bad_table |= (uint32_t)a.cdf32[row * (A + 1) + A] != kProbOne;
    } else {
        // Idle lanes: code stays 0, so they always decode symbol 0, whose
        // frequency 65535 never forces a renormalisation.
        tab[lane] = 0xFFFFu << 16;
        for (int s = 1; s < A; ++s) tab[s * 64 + lane] = (uint32_t)s | (1u << 16);
    }
    if (FUSED) {
        const uint16_t *sp = a.scale + (int64_t)slab * a.T + t0;
        for (int t = lane; t < n; t += 64) sc[t] = bf16_to_f32(sp[t]);
        const int M = a.mt.m[kv][l];
        dq[lane] = __fdiv_rn((float)(lane - M), (float)M);
        dq[lane + 64] = __fdiv_rn((float)(lane + 64 - M), (float)M);
    }
    __syncthreads();

    const uint8_t *gsrc = a.payload + base + excl;  // unstaged path
    const uint32_t loff = head + excl;
    uint32_t pos = 0;
    auto next_byte = [&]() -> uint32_t {
        uint32_t b = 0;
        if (pos < len) b = staged ? (uint32_t)bytes[loff + pos] : (uint32_t)gsrc[pos];
        ++pos;
        return b;
    };
    uint32_t code = 0;
    for (int i = 0; i < 4; ++i) code = (code << 8) | next_byte();
    uint32_t range = 0xFFFFFFFFu;

    uint8_t *sym_out = FUSED ? nullptr : a.sym + ((int64_t)slab * a.T + t0) * a.C + c;
    uint16_t *kv_out = FUSED ? a.kv + (((int64_t)l * 2 + kv) * a.T + t0) * a.C + c : nullptr;
    for (int t = 0; t < n; ++t) {
        const uint32_t r = range >> 16;
        uint32_t s = 0;
#pragma unroll
        for (int step = 1 << (LOGA - 1); step > 0; step >>= 1) {
            const uint32_t cand = s + step;
            if (cand < (uint32_t)A) {
                const uint32_t st = tab[cand * 64 + lane] & 0xFFFFu;
                if (__umul24(r, st) <= code) s = cand;
            }
        }
        const uint32_t e = tab[s * 64 + lane];
        code -= __umul24(r, e & 0xFFFFu);
        range = __umul24(r, e >> 16);
        if (range < kTop) {
            code = (code << 8) | next_byte();
            range <<= 8;
            if (range < kTop) {
                code = (code << 8) | next_byte();
                range <<= 8;
            }
        }
        corrupt |= code >= range;
        if (active) {
            if (FUSED) {
                kv_out[(int64_t)t * a.C] = (uint16_t)f32_to_bf16_rne(__fmul_rn(dq[s & 0x7F], sc[t]));
            } else {
                sym_out[(int64_t)t * a.C] = (uint8_t)s;
            }
        }
    }
    if (__ballot(active && (corrupt || bad_table)) && lane == 0) atomicOr(a.status, kStCorrupt);
}

template <int LOGA>
static hipError_t launch_decode_t(const Dims &d, const DecArgs &a, bool fused, hipStream_t s) {
    const size_t lds = (size_t)d.A * 64 * 4 + kStageBytes + kChunk * 4 + 128 * 4;
    if (fused)
        hipLaunchKernelGGL((k_decode<LOGA, true>), dim3((unsigned)d.tiles), dim3(64), lds, s, a);
    else
        hipLaunchKernelGGL((k_decode<LOGA, false>), dim3((unsigned)d.tiles), dim3(64), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_decode(const Dims &d, const MaxTable &mt, const DecodeIn &in, const DecodeOut &out,
                         uint64_t *tile_off, uint32_t *status, hipStream_t s) {
    hipLaunchKernelGGL(k_lenscan, dim3((unsigned)d.NC), dim3(256), 0, s, in.lengths, in.chunk_off,
                       tile_off, status, d.L, d.C, d.CB, d.NC, in.payload_bytes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    DecArgs a;
    a.payload = in.payload;
    a.payload_bytes = in.payload_bytes;
    a.lengths = in.lengths;
    a.tile_off = tile_off;
    a.cdf32 = in.cdf32;
    a.cdf16 = in.cdf16;
    a.sym = out.sym;
    a.kv = out.kv;
    a.scale = out.scale;
    a.status = status;
    a.mt = mt;
    a.L = d.L;
    a.T = d.T;
    a.C = d.C;
    a.A = d.A;
    a.CB = d.CB;
    const bool fused = out.kv != nullptr;
    if (d.A <= 32) return launch_decode_t<5>(d, a, fused, s);
    if (d.A <= 64) return launch_decode_t<6>(d, a, fused, s);
    return launch_decode_t<7>(d, a, fused, s);
}

}  // namespace cg
