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
// Pass 2 (k_decode): one wave per group of S tiles that share 64 channels
// (lane = channel) and differ only in the chunk, so each lane decodes S
// streams of its channel interleaved (independent dependency chains) with
// one table. The tiles' bytes (contiguous in the payload) are copied into LDS
// with the 64 lanes reading consecutive words; the tables are staged as
// start | freq << 16 [symbol][lane]. The symbol is the largest s with
// r * cdf[s] <= code, found by a branch-free binary search over the whole
// alphabet (depth fixed at compile time, the S searches interleaved);
// comparing r * cdf[s] with code is the same test as cdf[s] <= floor(code / r), so no
// division is needed. Renormalisation is two predicated steps. The fused
// variant multiplies by the per-token scale and converts to bf16 with the
// hardware round-to-nearest-even conversion, so the symbols never reach
// memory.
#include "cg_internal.hpp"

namespace cg {

constexpr int kStageTile = 1536;  // LDS bytes per staged tile payload (larger tiles read global memory)

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
    int L, T, C, A, NC, CB;
};

// One stream's decoder state and byte source.
struct DecStream {
    uint32_t code, range;
    uint32_t ptr, end;    // LDS byte address of the next byte / of the stream's end
    uint32_t pos, len;    // the same, counted in the stream (unstaged path)
    const uint8_t *gsrc;  // unstaged source (payload + stream offset)
};

// The per-token loop of k_decode.
//
// Latency: the first two levels of the binary search compare against CDF
// values held in registers (the same candidates every token); the byte the
// next renormalisation shifts in is read one renormalisation ahead; each
// token's dequantisation and store run one token later, so their LDS reads
// overlap the next search. A stream whose tile did not fit the LDS stage
// reads its bytes from global memory instead (staged[s] is wave-uniform).
template <int S, bool FUSED, int LOGA, bool CLAMP>
__device__ __forceinline__ void decode_loop(const DecArgs &a, DecStream (&st)[S], const int (&n)[S],
                                            const bool (&staged)[S], const uint32_t (&rowoff)[S],
                                            const uint32_t *tab, const float *dq, const uint16_t *sc,
                                            const uint8_t *stage, __amdgpu_buffer_rsrc_t out_rsrc,
                                            uint32_t out_voff, int lane, uint64_t &bad_mask) {
    const uint32_t zero_at = S * kStageTile;
    auto fetch = [&](int s) -> uint32_t {
        const DecStream &d = st[s];
        if (staged[s]) return stage[d.ptr < d.end ? d.ptr : zero_at];
        return d.pos < d.len ? (uint32_t)d.gsrc[d.pos] : 0u;
    };
    auto advance = [&](int s) {
        ++st[s].ptr;
        ++st[s].pos;
    };
    uint32_t nxt[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        for (int i = 0; i < 4; ++i) {
            st[s].code = (st[s].code << 8) | fetch(s);
            advance(s);
        }
        nxt[s] = fetch(s);
    }

    // Byte address in tab of (symbol s, this lane) is s * 256 + lane * 4.
    const uint8_t *tabb = reinterpret_cast<const uint8_t *>(tab);
    const uint32_t lane4 = (uint32_t)lane * 4;
    const uint32_t amax4 = ((uint32_t)a.A - 1) * 256 + lane4;
    constexpr uint32_t H1 = 1u << (LOGA - 1), H2 = 1u << (LOGA - 2);
    // Candidates of the first two levels (clamped to the alphabet).
    const uint32_t sa = CLAMP ? min(H1, (uint32_t)a.A - 1) : H1;
    const uint32_t sb = CLAMP ? min(H2, (uint32_t)a.A - 1) : H2;
    const uint32_t sc3 = CLAMP ? min(H1 + H2, (uint32_t)a.A - 1) : H1 + H2;
    const uint32_t cdf_a = tab[sa * 64 + lane] & 0xFFFFu;
    const uint32_t cdf_b = tab[sb * 64 + lane] & 0xFFFFu;
    const uint32_t cdf_c = tab[sc3 * 64 + lane] & 0xFFFFu;
    const uint32_t ad_a = sa * 256 + lane4, ad_b = sb * 256 + lane4, ad_c = sc3 * 256 + lane4;
    const int nmax = n[0];

    // Output of the previous token, written one step late.
    uint32_t p_sy[S], p_sc[S];
    float p_dq[S];
    int p_t = -1;
    auto store = [&](int s, int t) {
        if (t < n[s]) {
            const uint32_t off = rowoff[s] + (uint32_t)t * (uint32_t)a.C * (FUSED ? 2u : 1u);
            if (FUSED) {
                const float x = __fmul_rn(p_dq[s], __uint_as_float(p_sc[s] << 16));
                const __hip_bfloat16 h = __float2bfloat16(x);
                __builtin_amdgcn_raw_buffer_store_b16(*reinterpret_cast<const uint16_t *>(&h), out_rsrc,
                                                      (int)out_voff, (int)off, 0);
            } else {
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)p_sy[s], out_rsrc, (int)out_voff, (int)off, 0);
            }
        }
    };

    for (int t = 0; t < nmax; ++t) {
        uint32_t r[S], ad[S];
        // Levels 1 and 2 from registers.
#pragma unroll
        for (int s = 0; s < S; ++s) {
            r[s] = st[s].range >> 16;
            const bool hi = __umul24(r[s], cdf_a) <= st[s].code;
            const uint32_t c2 = hi ? cdf_c : cdf_b;
            const bool hi2 = __umul24(r[s], c2) <= st[s].code;
            ad[s] = hi ? (hi2 ? ad_c : ad_a) : (hi2 ? ad_b : lane4);
        }
        // Remaining levels: interleaved branch-free binary searches over LDS.
#pragma unroll
        for (int i = LOGA - 3; i >= 0; --i) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                uint32_t cand = ad[s] + (256u << i);
                if (CLAMP) cand = min(cand, amax4);
                const uint32_t ec = *reinterpret_cast<const uint32_t *>(tabb + cand);
                ad[s] = __umul24(r[s], ec & 0xFFFFu) <= st[s].code ? cand : ad[s];
            }
        }
        // The previous token's output, now that its LDS reads have landed.
        if (p_t >= 0) {
#pragma unroll
            for (int s = 0; s < S; ++s) store(s, p_t);
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
            // Every stream steps every token (a finished stream keeps decoding
            // zeros); only its output and its checks are guarded.
            DecStream &d = st[s];
            const uint32_t e = *reinterpret_cast<const uint32_t *>(tabb + ad[s]);
            const uint32_t sy = (ad[s] - lane4) >> 8;
            d.code -= __umul24(r[s], e & 0xFFFFu);
            d.range = __umul24(r[s], e >> 16);
            if (d.range < kTop) {
                d.code = (d.code << 8) | nxt[s];
                d.range <<= 8;
                advance(s);
                if (d.range < kTop) {
                    d.code = (d.code << 8) | fetch(s);
                    d.range <<= 8;
                    advance(s);
                }
                nxt[s] = fetch(s);
            }
            if (t < n[s]) bad_mask |= __ballot(d.code >= d.range);
            p_sy[s] = sy;
            if (FUSED) {
                p_dq[s] = dq[sy];
                p_sc[s] = sc[s * kChunk + t];
            }
        }
        p_t = t;
    }
    if (p_t >= 0) {
#pragma unroll
        for (int s = 0; s < S; ++s) store(s, p_t);
    }
}

template <int S, bool FUSED, int LOGA, bool CLAMP>
__global__ __launch_bounds__(64) void k_decode(DecArgs a) {
    // Static LDS sized by the template, so every address folds to an immediate.
    __shared__ float dq[128];
    __shared__ uint32_t tab[(1 << LOGA) * 64];                                   // [symbol][lane]
    __shared__ __attribute__((aligned(16))) uint8_t stage[S * kStageTile + 8];  // tiles' bytes, then zeros
    __shared__ uint16_t sc[FUSED ? S * kChunk : 1];                             // per-token scales (bf16)
    const int lane = threadIdx.x;
    const int A = a.A;

    const int bid = blockIdx.x;
    const int cb = bid % a.CB;
    const int slab = (bid / a.CB) % (2 * a.L);
    const int g = bid / (a.CB * 2 * a.L);
    const int kv = slab / a.L, l = slab - kv * a.L;
    const int c = cb * 64 + lane;
    const bool active = c < a.C;
    const int M = a.mt.m[kv][l];

    int n[S], t0[S];
    bool staged[S];
    DecStream st[S];
    bool corrupt = false;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int j = g * S + s;
        n[s] = j < a.NC ? min(kChunk, a.T - j * kChunk) : 0;
        t0[s] = min(j, a.NC - 1) * kChunk;
        uint32_t len = 0, excl = 0, total = 0;
        uint64_t base = 0;
        if (n[s]) {
            len = active ? a.lengths[((int64_t)j * 2 * a.L + slab) * a.C + c] : 0u;
            const uint32_t incl = wave_incl_scan_u32(len, lane);
            total = (uint32_t)__shfl((int)incl, 63, 64);
            excl = incl - len;
            base = a.tile_off[((int64_t)j * 2 * a.L + slab) * a.CB + cb];
            if (base > a.payload_bytes || total > a.payload_bytes - base) {
                corrupt = true;  // offsets point outside the payload: decode from nothing
                len = excl = total = 0;
                base = 0;
            }
        }
        // Stage the tile's bytes: words from the aligned start, bounded by the payload.
        const uint64_t abase = base & ~3ull;
        const uint32_t head = (uint32_t)(base - abase);
        staged[s] = total + head <= (uint32_t)kStageTile;
        if (staged[s] && total) {
            uint32_t *w = reinterpret_cast<uint32_t *>(stage + s * kStageTile);
            const uint32_t nw = (head + total + 3) >> 2;
            for (uint32_t i = lane; i < nw; i += 64) {
                const uint64_t gaddr = abase + 4ull * i;
                uint32_t v;
                if (gaddr + 4 <= a.payload_bytes) {
                    v = *reinterpret_cast<const uint32_t *>(a.payload + gaddr);
                } else {
                    v = 0;
                    for (int k = 0; k < 4; ++k)
                        if (gaddr + k < a.payload_bytes) v |= (uint32_t)a.payload[gaddr + k] << (8 * k);
                }
                w[i] = v;
            }
        }
        st[s].len = len;
        st[s].pos = 0;
        st[s].ptr = s * kStageTile + head + excl;
        st[s].end = st[s].ptr + len;
        st[s].gsrc = a.payload + base + excl;
        st[s].range = 0xFFFFFFFFu;
        st[s].code = 0;
    }

    // Tables.
    bool bad_table = false;
    if (active) {
        const int64_t row = (int64_t)slab * a.C + c;
        uint32_t prev = a.cdf32 ? (uint32_t)a.cdf32[row * (A + 1)] : (uint32_t)a.cdf16[row * A];
        bad_table = prev != 0;
        for (int s = 0; s < A; ++s) {
            uint32_t nxtv;
            if (a.cdf32)
                nxtv = (uint32_t)a.cdf32[row * (A + 1) + s + 1];
            else
                nxtv = s + 1 < A ? (uint32_t)a.cdf16[row * A + s + 1] : kProbOne;
            uint32_t f = nxtv - prev;
            if (nxtv <= prev || nxtv > kProbOne) {
                bad_table = true;
                f = 1;
            }
            tab[s * 64 + lane] = (prev & 0xFFFFu) | (f << 16);
            prev = nxtv;
        }
        if (a.cdf32) bad_table |= (uint32_t)a.cdf32[row * (A + 1) + A] != kProbOne;
    } else {
        // Idle lanes: code stays 0, so they always decode symbol 0, whose
        // frequency 65535 never forces a renormalisation.
        tab[lane] = 0xFFFFu << 16;
        for (int s = 1; s < A; ++s) tab[s * 64 + lane] = (uint32_t)s | (1u << 16);
    }
    if (lane < 8) stage[S * kStageTile + lane] = 0;  // the byte read past every stream
    if (FUSED) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const uint16_t *sp = a.scale + (int64_t)slab * a.T + t0[s];
            for (int t = lane; t < n[s]; t += 64) sc[s * kChunk + t] = sp[t];
        }
        dq[lane] = __fdiv_rn((float)(lane - M), (float)M);
        dq[lane + 64] = __fdiv_rn((float)(lane + 64 - M), (float)M);
    }
    __syncthreads();

    // Output rows: a buffer over this (K|V, layer) slab; the row offset is
    // wave-uniform, the lane offset constant; idle lanes point past the end.
    const uint32_t esz = FUSED ? 2u : 1u;
    const uint64_t slab_elems = (uint64_t)a.T * a.C;
    const void *obase = FUSED ? (const void *)(a.kv + ((int64_t)l * 2 + kv) * (int64_t)slab_elems)
                              : (const void *)(a.sym + (int64_t)slab * (int64_t)slab_elems);
    const __amdgpu_buffer_rsrc_t out_rsrc = make_rsrc(obase, (uint32_t)(slab_elems * esz));
    const uint32_t out_voff = active ? (uint32_t)(cb * 64 + lane) * esz : 0x7FFFFFF0u;
    uint32_t rowoff[S];
#pragma unroll
    for (int s = 0; s < S; ++s) rowoff[s] = (uint32_t)t0[s] * (uint32_t)a.C * esz;

    uint64_t bad_mask = 0;
    decode_loop<S, FUSED, LOGA, CLAMP>(a, st, n, staged, rowoff, tab, dq, sc, stage, out_rsrc, out_voff,
                                       lane, bad_mask);
    if ((__ballot(active && (corrupt || bad_table)) | (bad_mask & __ballot(active))) && lane == 0)
        atomicOr(a.status, kStCorrupt);
}

template <int S, bool FUSED, int LOGA>
static hipError_t launch_decode_s(const Dims &d, const DecArgs &a, hipStream_t s) {
    static_assert(kStageTile % 4 == 0, "stage holds whole words");
    const size_t lds = 0;  // all LDS is static
    const int ngroups = (d.NC + S - 1) / S;
    const dim3 grid((unsigned)((int64_t)ngroups * 2 * d.L * d.CB));
    if (d.A == (1 << LOGA))
        hipLaunchKernelGGL((k_decode<S, FUSED, LOGA, false>), grid, dim3(64), lds, s, a);
    else
        hipLaunchKernelGGL((k_decode<S, FUSED, LOGA, true>), grid, dim3(64), lds, s, a);
    return hipGetLastError();
}

template <int S, bool FUSED>
static hipError_t launch_decode_f(const Dims &d, const DecArgs &a, hipStream_t s) {
    if (d.A <= 4) return launch_decode_s<S, FUSED, 2>(d, a, s);
    if (d.A <= 8) return launch_decode_s<S, FUSED, 3>(d, a, s);
    if (d.A <= 16) return launch_decode_s<S, FUSED, 4>(d, a, s);
    if (d.A <= 32) return launch_decode_s<S, FUSED, 5>(d, a, s);
    if (d.A <= 64) return launch_decode_s<S, FUSED, 6>(d, a, s);
    return launch_decode_s<S, FUSED, 7>(d, a, s);
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
    a.NC = d.NC;
    a.CB = d.CB;
    const bool fused = out.kv != nullptr;
    if (d.NC >= 2) return fused ? launch_decode_f<2, true>(d, a, s) : launch_decode_f<2, false>(d, a, s);
    return fused ? launch_decode_f<1, true>(d, a, s) : launch_decode_f<1, false>(d, a, s);
}

}  // namespace cg
