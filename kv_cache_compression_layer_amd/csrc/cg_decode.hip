// Range decoder (and fused dequantisation) of the CacheGen codec on gfx950.
//
// LMCache CacheGen page (0539edu.com/news/4720135), section 5: every
// (layer, channel) stream is restored from the CDF and the prefix sums of the
// stream lengths, the symbols are reshaped to [2, L, T, C], and dequantised
// as t = (t - M) / M * scale before being stacked back to [L, 2, T, H, D] in
// the input dtype.
//
// Pass 1 (launch_tile_scan) turns the uint16 lengths into the byte offset of
// every 64-stream tile: the chunk offset plus the prefix sum of the lengths
// before it, and checks that the chunk's lengths add up to the next chunk
// offset.
//
// Pass 2 (k_decode): a block of NW waves owns 64 channels of one (K|V,
// layer) (lane = channel) and NW * S chunks; each wave decodes S streams per
// lane interleaved (independent dependency chains) with the one table of its
// channel. The waves share the tables, staged as start | freq << 16
// [symbol][lane] (blocks of one or two waves, which short calls use and
// whose residency the LDS decides, keep 16-bit starts instead), and an LDS
// pool for their tiles' payload: every lane copies
// its own stream there, followed by four zero bytes (the bytes past a
// stream's end read as zero), so the byte fetch needs no bounds check. A
// wave whose tiles do not fit the pool reads global memory instead. The
// symbol is the largest s with r * cdf[s] <= code, found by a branch-free
// binary search over the whole alphabet (depth fixed at compile time, the S
// searches interleaved); comparing r * cdf[s] with code is the same test as
// cdf[s] <= floor(code / r), so no division is needed. Renormalisation is
// two predicated steps. The fused variant multiplies by the per-token scale
// and converts to bf16 with the hardware round-to-nearest-even conversion,
// so the symbols never reach memory.
#include "cg_internal.hpp"

namespace cg {

struct DecArgs {
    const uint8_t *payload;
    uint64_t payload_bytes;
    const uint16_t *lengths;
    const uint64_t *tile_off;
    const int32_t *cdf32;
    const uint16_t *cdf16;
    const uint32_t *wpre;
    uint8_t *sym;
    uint16_t *kv;
    const uint16_t *scale;
    uint32_t *status;
    PagedOut paged;
    MaxTable mt;
    CallMap cm;    // calls of a batch: blob sections per call
    // Batches: call b's payload bound is min(call_sizes[b], stride) -
    // payload_off (0 if below) instead of payload_bytes.
    const uint64_t *call_sizes;
    uint64_t payload_off;
    int L, T, C, A, NC, CB;
    int j0, NCr;   // the chunks decoded: [j0, j0 + NCr)
    int nsym_lo, nsym_hi;
};

// Payload of the call that slab location sl belongs to, and its size.
__device__ __forceinline__ const uint8_t *call_payload(const DecArgs &a, const SlabLoc &sl, uint64_t &bytes) {
    bytes = a.payload_bytes;
    if (a.call_sizes) {
        uint64_t sz = a.call_sizes[sl.b];
        if (sz > a.cm.stride) sz = a.cm.stride;
        bytes = sz > a.payload_off ? sz - a.payload_off : 0ull;
    }
    return call_sec(a.payload, a.cm, sl.b);
}

// Bytes of the LDS pool a block of NW waves shares for its tiles' payload,
// and the slack after it: a stream is never read more than 4 + 2 * 256 + 2
// bytes past its first byte (two renormalisations per symbol at most, two
// bytes of look-ahead), so reads of a malformed stream stay inside the
// block's LDS.
// Residency beats pool size: with eight waves per block and 3840 bytes per
// wave (~39 KiB per block) four blocks, 32 waves, fit a CU; the few tiles
// that do not fit read global memory.
constexpr uint32_t kPoolPerWave = 3840;
constexpr uint32_t kPoolPerWaveSmall = 1536;  // blocks of one or two waves
constexpr uint32_t kPoolPerWaveLat = 12288;   // the same, in a launch of few waves (LAT 1)
constexpr uint32_t kPoolPerWaveLat2 = 6144;   // ... of somewhat more waves (LAT 2)
constexpr uint32_t kPoolSlack = 528;

// One stream's decoder state. Staged streams read pool bytes at `ptr` (each
// stream is followed by at least four zero bytes, the bytes past its end);
// unstaged streams read global memory at gsrc[pos] while pos < len.
struct DecStream {
    uint32_t code, range;
    uint32_t ptr;
    uint32_t pos, len;
    const uint8_t *gsrc;
};

// The per-token loop of k_decode.
//
// The table holds 2^LOGA entries per lane; entries past the table's width W
// have start 0xFFFF, so the search can only land on them when the symbol is
// the last one, W - 1, and one clamp at the end maps them back (CLAMP).
//
// Latency: the first two levels of the binary search compare against CDF
// values held in registers (the same candidates every token); the two bytes
// the next renormalisations shift in are read ahead; each token's
// dequantisation and store run one token later, so their LDS reads overlap
// the next search. The per-token scale is wave-uniform: lane i of sc_v[s][k]
// holds the scale of token 64k + i of stream s, read out with readlane.
// Row offsets through the block table (PAGED): lane i of pv[s] holds the
// physical block of logical block b0[s] + i, for the blocks stream s spans.
template <int S>
struct PagedRows {
    uint32_t pv[S];
    int t0[S], b0[S];
};

// T16: the table holds 16-bit starts [symbol][lane] (2^LOGA + 1 of them:
// 0xFFFF past the width W, or the true start of symbol 2^LOGA when the table
// is wider than the LDS part), and a symbol's frequency is the difference of
// two starts, plus one for the last symbol W - 1 (whose upper bound 2^16 is
// stored as 0xFFFF so that the search never passes it).
// BL: renormalise without a branch (launches of few waves, where a wave's
// branches and exec-mask updates sit on its chain with nothing to hide them).
template <int S, bool FUSED, int LOGA, bool CLAMP, bool STAGED, bool HALF, bool PAGED, bool TAIL, bool T16, bool BL>
__device__ __forceinline__ void decode_loop(const DecArgs &a, DecStream (&st)[S], const int (&n)[S],
                                            const uint32_t (&rowoff)[S], const PagedRows<S> &pg,
                                            const uint32_t *tab,
                                            const float *dq, uint32_t (&sc_v)[S][4], const uint8_t *pool,
                                            __amdgpu_buffer_rsrc_t out_rsrc, uint32_t out_voff,
                                            int lane, int W, const uint16_t *c16, int slab, int c,
                                            uint64_t &bad_mask) {
    auto fetch = [&](int s) -> uint32_t {
        DecStream &d = st[s];
        if (STAGED) return pool[d.ptr++];
        const uint32_t v = d.pos < d.len ? (uint32_t)d.gsrc[d.pos] : 0u;
        ++d.pos;
        return v;
    };
    uint32_t nx0[S], nx1[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        for (int i = 0; i < 4; ++i) st[s].code = (st[s].code << 8) | fetch(s);
        nx0[s] = fetch(s);
        nx1[s] = fetch(s);
        if (STAGED) st[s].ptr -= 2;
        else st[s].pos -= 2;
    }

    // Byte address in tab of (symbol s, this lane) is s * RB + lane * EB.
    constexpr uint32_t EB = T16 ? 2u : 4u, RB = 64u * EB;
    const uint8_t *tabb = reinterpret_cast<const uint8_t *>(tab);
    const uint32_t lane4 = (uint32_t)lane * EB;
    auto start_at = [&](uint32_t a) -> uint32_t {
        if constexpr (T16) return *reinterpret_cast<const uint16_t *>(tabb + a);
        return *reinterpret_cast<const uint32_t *>(tabb + a) & 0xFFFFu;
    };
    // The LDS table holds min(W, 2^LOGA) entries; with TAIL and a wider
    // table, symbols from 2^LOGA up are found in the table in global memory.
    const int WL = W < (1 << LOGA) ? W : (1 << LOGA);
    const uint32_t amax4 = ((uint32_t)WL - 1) * RB + lane4;
    // The last symbol's row (T16: its frequency takes the +1), if in LDS.
    const uint32_t wlast = W <= (1 << LOGA) ? amax4 : 0xFFFFFFFFu;
    const bool tail_on = TAIL && W > (1 << LOGA);
    const uint32_t ltop4 = ((1u << LOGA) - 1) * RB + lane4;
    // Search depth: the whole table, or (HALF) its lower half when the layer's
    // symbols all lie below the half's top entry; landing on that top entry
    // then means a symbol at or above it (only in corrupt streams), and a
    // rare wave-uniform path continues the search upwards.
    constexpr int SD = HALF ? LOGA - 1 : LOGA;
    constexpr uint32_t H1 = 1u << (SD - 1), H2 = 1u << (SD - 2);
    const uint32_t top4 = ((1u << SD) - 1) * RB + lane4;
    const uint32_t cdf_a = start_at(H1 * RB + lane4);
    const uint32_t cdf_b = start_at(H2 * RB + lane4);
    const uint32_t cdf_c = start_at((H1 + H2) * RB + lane4);
    const int nmax = n[0];

    // Output of the previous token, written one step late.
    uint32_t p_sy[S], p_sc[S];
    float p_dq[S];
    int p_t = -1;
    auto row_off = [&](int s, int t) -> uint32_t {
        if constexpr (PAGED) {
            const int tt = pg.t0[s] + t;
            const uint32_t blk =
                (uint32_t)__builtin_amdgcn_readlane((int)pg.pv[s], (tt >> a.paged.log2_bs) - pg.b0[s]);
            const uint32_t row = (blk << a.paged.log2_bs) | (uint32_t)(tt & ((1 << a.paged.log2_bs) - 1));
            return row * (uint32_t)a.C * 2u;
        } else {
            return rowoff[s] + (uint32_t)t * (uint32_t)a.C * (FUSED ? 2u : 1u);
        }
    };
    auto store = [&](int s, int t) {
        if (t < n[s]) {
            const uint32_t off = row_off(s, t);
            // The output is written once and not read back here: stores carry
            // the non-temporal hint (cache policy 2), measured ~5% faster.
            if (FUSED) {
                const float x = __fmul_rn(p_dq[s], __uint_as_float(p_sc[s] << 16));
                const __hip_bfloat16 h = __float2bfloat16(x);
                __builtin_amdgcn_raw_buffer_store_b16(*reinterpret_cast<const uint16_t *>(&h), out_rsrc,
                                                      (int)out_voff, (int)off, 2);
            } else {
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)p_sy[s], out_rsrc, (int)out_voff, (int)off, 2);
            }
        }
    };

    auto store_all = [&](int t) {
#pragma unroll
        for (int s = 0; s < S; ++s) store(s, t);
    };

    // Tokens in blocks of 64: the scale register of a block is loop-invariant.
    for (int tb = 0; tb < nmax; tb += 64) {
    uint32_t cur_sc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) cur_sc[s] = sc_v[s][0];
    const int tend = min(nmax, tb + 64);
    for (int t = tb; t < tend; ++t) {
        uint32_t r[S], ad[S];
        // Levels 1 and 2 from registers.
#pragma unroll
        for (int s = 0; s < S; ++s) {
            r[s] = st[s].range >> 16;
            const bool hi = __umul24(r[s], cdf_a) <= st[s].code;
            const uint32_t c2 = hi ? cdf_c : cdf_b;
            const bool hi2 = __umul24(r[s], c2) <= st[s].code;
            ad[s] = lane4 | (hi ? H1 * RB : 0u) | (hi2 ? H2 * RB : 0u);
        }
        // Remaining levels: interleaved branch-free binary searches over LDS.
#pragma unroll
        for (int i = SD - 3; i >= 0; --i) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const uint32_t cand = ad[s] | (RB << i);
                ad[s] = __umul24(r[s], start_at(cand)) <= st[s].code ? cand : ad[s];
            }
        }
        // The previous token's output, now that its LDS reads have landed.
        if (p_t >= 0) store_all(p_t);
#pragma unroll
        for (int s = 0; s < S; ++s) {
            // Every stream steps every token (a finished stream keeps decoding
            // zeros); only its output and its checks are guarded.
            DecStream &d = st[s];
            if (HALF && __builtin_amdgcn_ballot_w64(ad[s] == top4)) {
                __asm__ volatile("" ::: "memory");
                if (ad[s] == top4) {
                    for (uint32_t cand = top4 + RB; cand < (1u << LOGA) * RB; cand += RB) {
                        if (__umul24(r[s], start_at(cand)) > st[s].code) break;
                        ad[s] = cand;
                    }
                }
            }
            if (CLAMP) ad[s] = min(ad[s], amax4);
            uint32_t e;
            if constexpr (T16) {
                const uint32_t lo = start_at(ad[s]), hi = start_at(ad[s] + RB);
                e = lo | ((hi - lo + (ad[s] == wlast ? 1u : 0u)) << 16);
            } else {
                e = *reinterpret_cast<const uint32_t *>(tabb + ad[s]);
            }
            if (tail_on && __builtin_amdgcn_ballot_w64(ad[s] == ltop4)) {
                // The search stopped at the last LDS entry: the symbol may lie
                // above it (never for the quantiser's symbols, which stay below
                // 2M + 1 <= 2^LOGA). Continue upwards in global memory.
                __asm__ volatile("" ::: "memory");
                if (ad[s] == ltop4) {
                    bool bad = false;
                    for (int sy = 1 << LOGA; sy < W; ++sy) {
                        uint32_t lo, hi;
                        cdf_bounds(a.cdf32, c16, a.wpre, slab, a.C, c, a.A, W, sy, lo, hi);
                        if (__umul24(r[s], lo & 0xFFFFu) > st[s].code) break;
                        bad |= hi <= lo || hi > kProbOne;
                        ad[s] = (uint32_t)sy * RB + lane4;
                        e = (lo & 0xFFFFu) | ((hi - lo) << 16);
                    }
                    if (bad) e = (e & 0xFFFFu) | (1u << 16);
                    bad_mask |= __ballot(bad);
                }
            }
            d.code -= __umul24(r[s], e & 0xFFFFu);
            d.range = __umul24(r[s], e >> 16);
            if (BL && STAGED) {
                // The same renormalisation without a branch: selects, and the
                // look-ahead bytes read again at the same place when nothing
                // shifted.
                const bool one = d.range < kTop, two = d.range < (1u << 16);
                d.code = one ? (d.code << 8) | nx0[s] : d.code;
                d.range = two ? d.range << 16 : one ? d.range << 8 : d.range;
                d.ptr += (uint32_t)one + (uint32_t)two;
                if (__builtin_amdgcn_ballot_w64(two)) {
                    __asm__ volatile("" ::: "memory");
                    if (two) d.code = (d.code << 8) | nx1[s];
                }
                nx0[s] = pool[d.ptr];
                nx1[s] = pool[d.ptr + 1];
            } else if (d.range < kTop) {
                // A second shift (range < 2^16) needs a rare symbol (freq <
                // 2^16 / r); the wave-uniform test keeps its code out of the
                // common path.
                const bool two = d.range < (1u << 16);
                d.code = (d.code << 8) | nx0[s];
                d.range <<= two ? 16 : 8;
                if (STAGED) d.ptr += 1u + (uint32_t)two;
                else d.pos += 1u + (uint32_t)two;
                if (__builtin_amdgcn_ballot_w64(two)) {
                    __asm__ volatile("" ::: "memory");  // a real branch, not selects
                    if (two) d.code = (d.code << 8) | nx1[s];
                }
                if (STAGED) {
                    nx0[s] = pool[d.ptr];
                    nx1[s] = pool[d.ptr + 1];
                } else {
                    nx0[s] = d.pos < d.len ? (uint32_t)d.gsrc[d.pos] : 0u;
                    nx1[s] = d.pos + 1 < d.len ? (uint32_t)d.gsrc[d.pos + 1] : 0u;
                }
            }
            if (t < n[s]) bad_mask |= __ballot(d.code >= d.range);
            if (FUSED) {
                p_dq[s] = *reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(dq) +
                                                           ((ad[s] >> (T16 ? 5 : 6)) & ~3u));
                p_sc[s] = (uint32_t)__builtin_amdgcn_readlane((int)cur_sc[s], t & 63);
            } else {
                p_sy[s] = ad[s] >> (T16 ? 7 : 8);
            }
        }
        p_t = t;
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        sc_v[s][0] = sc_v[s][1];
        sc_v[s][1] = sc_v[s][2];
        sc_v[s][2] = sc_v[s][3];
    }
    }
    if (p_t >= 0) store_all(p_t);
}

// Reads the aligned 32-bit word at payload offset g (g % 4 == 0), with the
// bytes at or beyond payload_bytes read as zero.
__device__ __forceinline__ uint32_t load_word(const uint8_t *payload, uint64_t payload_bytes, uint64_t g) {
    if (g + 4 <= payload_bytes) return *reinterpret_cast<const uint32_t *>(payload + g);
    uint32_t v = 0;
    for (int k = 0; k < 4; ++k)
        if (g + k < payload_bytes) v |= (uint32_t)payload[g + k] << (8 * k);
    return v;
}

// Block of NW waves for one (K|V, layer, 64-channel block): wave w decodes
// the S chunks (group * NW + w) * S + s, lane = channel. The waves share the
// channel tables, the dequantisation table and an LDS pool for the payload.
// LAT (1, 2): a launch of few waves (a short call alone), whose time is one
// stream's latency; see kPoolBytes.
template <int S, bool FUSED, int LOGA, bool CLAMP, int NW, bool PAGED, bool TAIL, int LAT>
__global__ __launch_bounds__(64 * NW) void k_decode(DecArgs a) {
    // Static LDS sized by the template, so every address folds to an immediate.
    // Blocks of one or two waves (short calls) are as many per CU as their
    // LDS allows: they keep 16-bit starts (see decode_loop's T16).
    constexpr bool T16 = NW <= 2;
    __shared__ uint32_t tab[T16 ? ((1 << LOGA) + 1) * 32 : (1 << LOGA) * 64];  // [symbol][lane]
    __shared__ float dq[128];
    // Blocks of one or two waves (calls of fewer than eight chunks) keep a
    // small pool: what limits them is residency, so it holds only the tiles
    // of short streams (a 16-bin slab's 64 streams of a 256-token chunk at
    // about 12 bytes each), whose bytes then come from LDS instead of
    // bounds-checked global reads (128 calls of 256 tokens: 2.55 ms with no
    // pool, 2.42 / 2.39 / 2.49 ms with 1024 / 1536 / 2560 bytes per wave).
    // Larger blocks share their tables across more waves and a full pool
    // pays for itself (measured: 1.79 vs 2.14 ms on 32K tokens). A launch of
    // few waves (LAT) is not held back by residency at all: with a pool
    // that holds whole tiles of long streams (a 32-bin slab's 64 streams of a
    // 256-token chunk take about 5 KB) no renormalisation waits for a
    // global read; 12 KiB per wave up to 8 waves per CU (LAT 1), 6 KiB up
    // to 16 (LAT 2), which still fit the CU's LDS.
    constexpr uint32_t kPoolBytes =
        NW * (LAT == 1 ? kPoolPerWaveLat : LAT == 2 ? kPoolPerWaveLat2 : NW <= 2 ? kPoolPerWaveSmall : kPoolPerWave);
    __shared__ uint32_t pool_w[(kPoolBytes + kPoolSlack) / 4];  // staged payload
    __shared__ uint32_t need_w[NW];
    const int lane = threadIdx.x & 63;
    // The wave index is uniform across the wave; readfirstlane tells the compiler so,
    // which keeps everything derived from it in scalar registers.
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int A = a.A;

    const int bid = blockIdx.x;
    const int cb = bid % a.CB;
    const int slab = (bid / a.CB) % (2 * a.L);
    const int g = bid / (a.CB * 2 * a.L);
    const SlabLoc sl = slab_loc(a.cm, slab);
    const int kv = sl.kv, l = sl.l;
    const int c = cb * 64 + lane;
    const bool active = c < a.C;
    const int M = layer_m(a.mt, kv, l);
    const int W = layer_w(a.mt, kv, l);  // symbols of this slab's tables
    // This launch decodes only the slabs whose quantiser symbol count 2M+1
    // lies in [nsym_lo, nsym_hi]; the other blocks return at once.
    if (2 * M + 1 < a.nsym_lo || 2 * M + 1 > a.nsym_hi) return;  // block-uniform
    uint64_t payload_bytes;
    const uint8_t *payload = call_payload(a, sl, payload_bytes);
    const uint16_t *lengths = call_sec(a.lengths, a.cm, sl.b);
    const uint16_t *cdf16 = call_sec(a.cdf16, a.cm, sl.b);

    // This wave's streams: lengths, offsets and the pool bytes they need
    // (alignment head + bytes + four zero bytes after each of the 64 streams).
    int n[S], t0[S];
    uint32_t len[S], excl[S], need[S];
    uint64_t base[S];
    bool corrupt = false;
    uint32_t need_total = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int jr = (g * NW + wv) * S + s, j = a.j0 + jr;
        n[s] = jr < a.NCr ? min(kChunk, a.T - j * kChunk) : 0;
        t0[s] = (a.j0 + min(jr, a.NCr - 1)) * kChunk;
        uint32_t total = 0;
        len[s] = excl[s] = 0;
        base[s] = 0;
        if (n[s]) {
            len[s] = active ? lengths[((int64_t)j * 2 * a.cm.Lc + sl.ls) * a.C + c] : 0u;
            const uint32_t incl = wave_incl_scan_u32(len[s], lane);
            total = (uint32_t)__shfl((int)incl, 63, 64);
            excl[s] = incl - len[s];
            base[s] = a.tile_off[((int64_t)j * 2 * a.L + slab) * a.CB + cb];
            if (base[s] > payload_bytes || total > payload_bytes - base[s]) {
                corrupt = true;  // offsets point outside the payload: decode from nothing
                len[s] = excl[s] = total = 0;
                base[s] = 0;
            }
        }
        need[s] = ((uint32_t)(base[s] & 3u) + total + 4u * 64u + 4u + 3u) & ~3u;
        need_total += need[s];
    }
    if (lane == 0) need_w[wv] = need_total;
    __syncthreads();
    uint32_t woff = 0;
    for (int i = 0; i < wv; ++i) woff += need_w[i];
    const bool staged = kPoolBytes != 0 && woff + need_total <= kPoolBytes;

    DecStream st[S];
    uint8_t *pool = reinterpret_cast<uint8_t *>(pool_w);
    if (staged) {
        for (uint32_t i = lane; i < need_total / 4; i += 64) pool_w[woff / 4 + i] = 0;
        uint32_t soff = woff;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            // LDS start of this lane's stream: congruent to its payload offset mod 4.
            const uint64_t g0 = base[s] + excl[s];
            const uint32_t ls = soff + (uint32_t)(base[s] & 3u) + excl[s] + 4u * (uint32_t)lane;
            st[s].ptr = ls;
            if (len[s]) {
                const uint64_t gend = g0 + len[s];
                const uint64_t ga = g0 & ~3ull, ge = (gend + 3) & ~3ull;
                uint32_t la = ls - (uint32_t)(g0 - ga);
                // LAT: the copy is on the call's critical path: more loads in flight.
                constexpr int kCopyUnroll = LAT ? 16 : 4;
#pragma unroll kCopyUnroll
                for (uint64_t gw = ga; gw < ge; gw += 4, la += 4) {
                    uint32_t v = load_word(payload, payload_bytes, gw);
                    if (gw < g0) v &= 0xFFFFFFFFu << (8 * (uint32_t)(g0 - gw));
                    if (gw + 4 > gend) v &= 0xFFFFFFFFu >> (8 * (uint32_t)(gw + 4 - gend));
                    pool_w[la >> 2] = v;
                }
            }
            soff += need[s];
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        st[s].len = len[s];
        st[s].pos = 0;
        st[s].gsrc = payload + base[s] + excl[s];
        st[s].range = 0xFFFFFFFFu;
        st[s].code = 0;
        if (!staged) st[s].ptr = 0;
    }

    // Tables, built by the block's waves together: wave w writes symbols w,
    // w + NW, ...; entries past the table's width W (up to 2^LOGA) have start
    // 0xFFFF.
    bool bad_table = false;
    // Loads read an in-bounds column (the lane's own for active lanes).
    const LaneTable lt = lane_table(a.cdf32, cdf16, a.wpre, sl.ls, a.C, min(c, a.C - 1), A, W);
    if constexpr (T16) {
        // Starts 0..2^LOGA: the symbol's lower bound below W, 0xFFFF from W
        // on; idle lanes: 0 then 0xFFFF (code 0 always decodes symbol 0 with
        // frequency 0xFFFF, which never forces a renormalisation).
        uint16_t *tab16 = reinterpret_cast<uint16_t *>(tab);
        for_lane_bounds<((1 << LOGA) + NW) / NW, kTabGroup>(lt, wv, NW, (1 << LOGA) + 1,
                                                            [&](int s, uint32_t lo, uint32_t hi) {
            uint32_t v = 0xFFFFu;
            if (s < W && active) {
                if (s < (1 << LOGA) &&
                    (hi <= lo || hi > kProbOne || (s == 0 && lo != 0) || (s == W - 1 && hi != kProbOne)))
                    bad_table = true;
                v = lo & 0xFFFFu;
            } else if (s == 0) {
                v = 0;
            }
            tab16[s * 64 + lane] = (uint16_t)v;
        });
    } else {
        for_lane_bounds<((1 << LOGA) + NW - 1) / NW, kTabGroup>(lt, wv, NW, 1 << LOGA, [&](int s, uint32_t lo, uint32_t hi) {
            uint32_t entry = 0xFFFFu;
            if (s < W && active) {
                uint32_t f = hi - lo;
                if (hi <= lo || hi > kProbOne || (s == 0 && lo != 0) || (s == W - 1 && hi != kProbOne)) {
                    bad_table = true;
                    f = 1;
                }
                entry = (lo & 0xFFFFu) | (f << 16);
            } else if (s < W) {
                // Idle lanes: code stays 0, so they always decode symbol 0,
                // whose frequency 65535 never forces a renormalisation.
                entry = s == 0 ? 0xFFFFu << 16 : (uint32_t)s | (1u << 16);
            }
            tab[s * 64 + lane] = entry;
        });
    }
    uint32_t sc_v[S][4];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint16_t *sp = call_sec(a.scale, a.cm, sl.b) + (int64_t)sl.ls * a.T + t0[s];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t = 64 * k + lane;
            sc_v[s][k] = FUSED && t < n[s] ? (uint32_t)sp[t] : 0u;
        }
    }
    if (FUSED && wv == 0) {
        dq[lane] = __fdiv_rn((float)(lane - M), (float)M);
        dq[lane + 64] = __fdiv_rn((float)(lane + 64 - M), (float)M);
    }
    __syncthreads();

    // Output rows: a buffer over this (K|V, layer) slab; the row offset is
    // wave-uniform, the lane offset constant; idle lanes point past the end.
    const uint32_t esz = FUSED ? 2u : 1u;
    const uint64_t slab_elems = (uint64_t)a.T * a.C;
    const void *obase = FUSED ? (const void *)(a.kv + ((int64_t)sl.lv * 2 + kv) * (int64_t)slab_elems)
                              : (const void *)(a.sym + (int64_t)slab * (int64_t)slab_elems);
    __amdgpu_buffer_rsrc_t out_rsrc = make_rsrc(obase, (uint32_t)(slab_elems * esz));
    PagedRows<S> pg;
    if constexpr (PAGED) {
        // The (l, kv) region of the cache; block table entries outside
        // [0, num_blocks) become num_blocks, whose rows lie past the buffer,
        // so their stores are dropped (and the call reports corruption).
        const uint32_t bs_log = (uint32_t)a.paged.log2_bs;
        const uint32_t region = ((uint32_t)a.paged.num_blocks << bs_log) * (uint32_t)a.C * 2u;
        out_rsrc = make_rsrc(a.paged.cache + (int64_t)sl.lv * a.paged.layer_stride + (int64_t)kv * a.paged.kv_stride,
                             region);
        const int nblk_total = (a.T + (1 << bs_log) - 1) >> bs_log;
        bool bad_block = false;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            pg.t0[s] = t0[s];
            pg.b0[s] = t0[s] >> bs_log;
            const int bi = pg.b0[s] + lane;
            uint32_t v = 0;
            if (n[s] && bi < nblk_total && bi <= ((t0[s] + n[s] - 1) >> bs_log)) {
                const int32_t e = a.paged.table[bi];
                if (e < 0 || e >= a.paged.num_blocks) {
                    bad_block = true;
                    v = (uint32_t)a.paged.num_blocks;
                } else {
                    v = (uint32_t)e;
                }
            }
            pg.pv[s] = v;
        }
        if (__ballot(bad_block) && lane == 0) atomicOr(a.status, kStCorrupt);
    }
    const uint32_t out_voff = active ? (uint32_t)(cb * 64 + lane) * esz : 0x7FFFFFF0u;
    uint32_t rowoff[S];
#pragma unroll
    for (int s = 0; s < S; ++s) rowoff[s] = (uint32_t)t0[s] * (uint32_t)a.C * esz;

    uint64_t bad_mask = 0;
    // The lower half of the table suffices when every symbol of the layer,
    // 0..2M, lies below its top entry 2^(LOGA-1) - 1.
    const bool half = LOGA >= 3 && M + 1 <= (1 << (LOGA - 2));
    if (half) {
        if (staged)
            decode_loop<S, FUSED, LOGA, CLAMP, true, LOGA >= 3, PAGED, TAIL, T16, (LAT == 1)>(a, st, n, rowoff, pg, tab, dq, sc_v, pool, out_rsrc,
                                                               out_voff, lane, W, cdf16, sl.ls, c, bad_mask);
        else
            decode_loop<S, FUSED, LOGA, CLAMP, false, LOGA >= 3, PAGED, TAIL, T16, (LAT == 1)>(a, st, n, rowoff, pg, tab, dq, sc_v, pool, out_rsrc,
                                                                out_voff, lane, W, cdf16, sl.ls, c, bad_mask);
    } else {
        if (staged)
            decode_loop<S, FUSED, LOGA, CLAMP, true, false, PAGED, TAIL, T16, (LAT == 1)>(a, st, n, rowoff, pg, tab, dq, sc_v, pool, out_rsrc,
                                                            out_voff, lane, W, cdf16, sl.ls, c, bad_mask);
        else
            decode_loop<S, FUSED, LOGA, CLAMP, false, false, PAGED, TAIL, T16, (LAT == 1)>(a, st, n, rowoff, pg, tab, dq, sc_v, pool, out_rsrc,
                                                             out_voff, lane, W, cdf16, sl.ls, c, bad_mask);
    }
    if ((__ballot(active && (corrupt || bad_table)) | (bad_mask & __ballot(active))) && lane == 0)
        atomicOr(a.status, kStCorrupt);
}

// ------------------------------------------------------------------------
// Two adjacent channels per lane (calls of eight chunks or more).
//
// A block of NW waves owns 128 consecutive channels of one (K|V, layer) and
// NW chunks, one per wave; lane i decodes the streams of channels
// 128 * cb2 + 2i and 2i + 1 of its wave's chunk, interleaved. Both streams of
// a lane are at the same token, so one per-token scale serves both, their two
// bf16 results leave in one 32-bit store, and the row address (of a paged
// cache too) is computed once. The wave's 128 streams are the two adjacent
// 64-stream tiles 2 * cb2 and 2 * cb2 + 1 of the chunk, one contiguous run of
// payload bytes starting at the first tile's offset. Tables [symbol][stream]
// [lane], start | freq << 16, shared by the block's waves.
// Pool bytes per wave: four blocks of eight waves (32 waves) per CU fit the
// 160 KiB of LDS with 16-entry tables (8 KiB per block) and 3840 bytes per
// wave, or with 32-entry tables (16 KiB) and 2928 bytes per wave.
__host__ __device__ constexpr uint32_t pool_per_wave2(int loga) { return loga <= 4 ? 3840u : 2928u; }
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <bool FUSED, int LOGA, bool CLAMP, bool STAGED, bool HALF, bool PAGED, bool TAIL, bool FULL>
__device__ __forceinline__ void decode_loop2(const DecArgs &a, DecStream (&st)[2], int n, uint32_t rowoff,
                                             int pg_t0, int pg_b0, uint32_t pg_v, const uint32_t *tab,
                                             const float *dq, uint32_t (&sc_v)[4], const uint8_t *pool,
                                             __amdgpu_buffer_rsrc_t out_rsrc, uint32_t out_voff, int lane, int W,
                                             const uint16_t *c16, int slab, const int (&cch)[2],
                                             uint64_t &bad_mask) {
    constexpr int S = 2;
    auto fetch = [&](int s) -> uint32_t {
        DecStream &d = st[s];
        if (STAGED) return pool[d.ptr++];
        const uint32_t v = d.pos < d.len ? (uint32_t)d.gsrc[d.pos] : 0u;
        ++d.pos;
        return v;
    };
    uint32_t nx0[S], nx1[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        for (int i = 0; i < 4; ++i) st[s].code = (st[s].code << 8) | fetch(s);
        nx0[s] = fetch(s);
        nx1[s] = fetch(s);
        if (STAGED) st[s].ptr -= 2;
        else st[s].pos -= 2;
    }

    // Byte address in tab of (symbol q, stream s, this lane): q * RB + s * 256 + lane * 4.
    constexpr uint32_t RB = 512u;
    const uint8_t *tabb = reinterpret_cast<const uint8_t *>(tab);
    uint32_t lane4[S];
#pragma unroll
    for (int s = 0; s < S; ++s) lane4[s] = (uint32_t)s * 256u + (uint32_t)lane * 4u;
    auto start_at = [&](uint32_t ad) -> uint32_t { return *reinterpret_cast<const uint32_t *>(tabb + ad) & 0xFFFFu; };
    const int WL = W < (1 << LOGA) ? W : (1 << LOGA);
    constexpr int SD = HALF ? LOGA - 1 : LOGA;
    constexpr uint32_t H1 = 1u << (SD - 1), H2 = 1u << (SD - 2);
    uint32_t amax4[S], ltop4[S], top4[S], cdf_a[S], cdf_b[S], cdf_c[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        amax4[s] = ((uint32_t)WL - 1) * RB + lane4[s];
        ltop4[s] = ((1u << LOGA) - 1) * RB + lane4[s];
        top4[s] = ((1u << SD) - 1) * RB + lane4[s];
        cdf_a[s] = start_at(H1 * RB + lane4[s]);
        cdf_b[s] = start_at(H2 * RB + lane4[s]);
        cdf_c[s] = start_at((H1 + H2) * RB + lane4[s]);
    }
    const bool tail_on = TAIL && W > (1 << LOGA);

    // Output of the previous token, written one step late (token t - 1 while
    // token t is searched; t is the wave-uniform loop counter).
    float p_dq[S];
    uint32_t p_sy[S], p_sc = 0;
    auto row_off = [&](int t) -> uint32_t {
        if constexpr (PAGED) {
            const int tt = pg_t0 + t;
            const uint32_t blk = (uint32_t)__builtin_amdgcn_readlane((int)pg_v, (tt >> a.paged.log2_bs) - pg_b0);
            const uint32_t row = (blk << a.paged.log2_bs) | (uint32_t)(tt & ((1 << a.paged.log2_bs) - 1));
            return row * (uint32_t)a.C * 2u;
        } else {
            return rowoff + (uint32_t)t * (uint32_t)a.C * (FUSED ? 2u : 1u);
        }
    };
    auto store_all = [&](int t) {
        // The token is wave-uniform; readfirstlane keeps its row offset in a
        // scalar register (the buffer store's offset operand).
        t = __builtin_amdgcn_readfirstlane(t);
        if (t >= n) return;
        const uint32_t off = row_off(t);
        // Written once and not read back here: non-temporal stores (cache policy 2).
        if constexpr (FUSED) {
            const float sc = __uint_as_float(p_sc << 16);
            // Both products rounded to bf16 (nearest even) by one packed
            // conversion: channel c0 in the low half, c0 + 1 in the high.
            const f32x2_t x = {__fmul_rn(p_dq[0], sc), __fmul_rn(p_dq[1], sc)};
            const uint32_t hv = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
            if constexpr (FULL) {
                __builtin_amdgcn_raw_buffer_store_b32(hv, out_rsrc, (int)out_voff, (int)off, 2);
            } else {
                // Channel counts that are not a multiple of 128: stores per
                // channel, those of idle channels past the buffer (dropped).
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hv, out_rsrc, (int)out_voff, (int)off, 2);
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(hv >> 16), out_rsrc,
                                                      (int)(cch[1] < a.C ? out_voff + 2u : 0x7FFFFFF0u), (int)off, 2);
            }
        } else {
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)p_sy[0], out_rsrc, (int)out_voff, (int)off, 2);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)p_sy[1], out_rsrc,
                                                 (int)(cch[1] < a.C ? out_voff + 1u : 0x7FFFFFF0u), (int)off, 2);
        }
    };

    for (int tb = 0; tb < n; tb += 64) {
        const uint32_t cur_sc = sc_v[0];
        const int tend = min(n, tb + 64);
        for (int t = tb; t < tend; ++t) {
            uint32_t r[S], ad[S];
            // Levels 1 and 2 from registers.
#pragma unroll
            for (int s = 0; s < S; ++s) {
                r[s] = st[s].range >> 16;
                const bool hi = __umul24(r[s], cdf_a[s]) <= st[s].code;
                const uint32_t c2 = hi ? cdf_c[s] : cdf_b[s];
                const bool hi2 = __umul24(r[s], c2) <= st[s].code;
                ad[s] = lane4[s] | (hi ? H1 * RB : 0u) | (hi2 ? H2 * RB : 0u);
            }
            // Remaining levels: interleaved branch-free binary searches over LDS.
#pragma unroll
            for (int i = SD - 3; i >= 0; --i) {
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const uint32_t cand = ad[s] | (RB << i);
                    ad[s] = __umul24(r[s], start_at(cand)) <= st[s].code ? cand : ad[s];
                }
            }
            // The previous token's output, now that its LDS reads have landed.
            if (t > 0) store_all(t - 1);
#pragma unroll
            for (int s = 0; s < S; ++s) {
                DecStream &d = st[s];
                if (HALF && __builtin_amdgcn_ballot_w64(ad[s] == top4[s])) {
                    __asm__ volatile("" ::: "memory");
                    if (ad[s] == top4[s]) {
                        for (uint32_t cand = top4[s] + RB; cand < (1u << LOGA) * RB; cand += RB) {
                            if (__umul24(r[s], start_at(cand)) > d.code) break;
                            ad[s] = cand;
                        }
                    }
                }
                if (CLAMP) ad[s] = min(ad[s], amax4[s]);
                uint32_t e = *reinterpret_cast<const uint32_t *>(tabb + ad[s]);
                if (tail_on && __builtin_amdgcn_ballot_w64(ad[s] == ltop4[s])) {
                    // The search stopped at the last LDS entry: the symbol may lie
                    // above it (only in streams the quantiser did not make).
                    // Continue upwards in global memory, every lane the same
                    // number of steps (a per-lane exit from this loop would make
                    // the token counter of the whole loop divergent).
                    __asm__ volatile("" ::: "memory");
                    bool bad = false;
                    if (ad[s] == ltop4[s]) {
                        bool up = true;
                        for (int sy = 1 << LOGA; sy < W; ++sy) {
                            uint32_t lo, hi;
                            cdf_bounds(a.cdf32, c16, a.wpre, slab, a.C, min(cch[s], a.C - 1), a.A, W, sy, lo,
                                       hi);
                            up = up && __umul24(r[s], lo & 0xFFFFu) <= d.code;
                            if (up) {
                                bad |= hi <= lo || hi > kProbOne;
                                ad[s] = (uint32_t)sy * RB + lane4[s];
                                e = (lo & 0xFFFFu) | ((hi - lo) << 16);
                            }
                        }
                        if (bad) e = (e & 0xFFFFu) | (1u << 16);
                    }
                    bad_mask |= __ballot(bad);
                }
                d.code -= __umul24(r[s], e & 0xFFFFu);
                d.range = __umul24(r[s], e >> 16);
                if (d.range < kTop) {
                    // One byte in; a second one (range < 2^16 before: a rare
                    // symbol) behind a wave-uniform test.
                    d.code = (d.code << 8) | nx0[s];
                    d.range <<= 8;
                    if (STAGED) d.ptr += 1u;
                    else d.pos += 1u;
                    // Keep the shifted state in its registers: otherwise the
                    // second shift is rebuilt from the unshifted values
                    // (range << 16, ptr + 2) and both paths merge through
                    // register copies on every step.
                    if (STAGED) __asm__ volatile("" : "+v"(d.code), "+v"(d.range), "+v"(d.ptr));
                    else __asm__ volatile("" : "+v"(d.code), "+v"(d.range), "+v"(d.pos));
                    if (__builtin_amdgcn_ballot_w64(d.range < kTop)) {
                        __asm__ volatile("" ::: "memory");  // a real branch, not selects
                        if (d.range < kTop) {
                            d.code = (d.code << 8) | nx1[s];
                            d.range <<= 8;
                            if (STAGED) d.ptr += 1u;
                            else d.pos += 1u;
                        }
                    }
                    if (STAGED) {
                        nx0[s] = pool[d.ptr];
                        nx1[s] = pool[d.ptr + 1];
                    } else {
                        nx0[s] = d.pos < d.len ? (uint32_t)d.gsrc[d.pos] : 0u;
                        nx1[s] = d.pos + 1 < d.len ? (uint32_t)d.gsrc[d.pos + 1] : 0u;
                    }
                }
                bad_mask |= __ballot(d.code >= d.range);
                if (FUSED) {
                    p_dq[s] = *reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(dq) +
                                                               ((ad[s] >> 7) & ~3u));
                } else {
                    p_sy[s] = ad[s] >> 9;
                }
            }
            if (FUSED) p_sc = (uint32_t)__builtin_amdgcn_readlane((int)cur_sc, t & 63);
        }
        sc_v[0] = sc_v[1];
        sc_v[1] = sc_v[2];
        sc_v[2] = sc_v[3];
    }
    if (n > 0) store_all(n - 1);
}

// Waves per SIMD that the LDS of a block allows (160 KiB per CU, four
// SIMDs), at most eight: the register budget is set to match, so the
// registers never hold residency below what the LDS allows (eight waves
// means at most 64 VGPRs): residency decides the decoder's speed more than
// anything the registers would save.
__host__ __device__ constexpr uint32_t dec2_lds_bytes(int loga, int nw) {
    return (1u << loga) * 128u * 4u + 128u * 4u + (uint32_t)nw * pool_per_wave2(loga) + kPoolSlack + 4u * nw;
}
__host__ __device__ constexpr int dec2_waves_per_simd(int loga, int nw) {
    return (int)(163840u / dec2_lds_bytes(loga, nw)) * nw / 4 > 8 ? 8 : (int)(163840u / dec2_lds_bytes(loga, nw)) * nw / 4;
}
static_assert(dec2_waves_per_simd(5, 8) == 8 && dec2_waves_per_simd(4, 8) == 8, "32-wave residency of the 32K path");

template <bool FUSED, int LOGA, bool CLAMP, int NW, bool PAGED, bool TAIL>
__global__ __launch_bounds__(64 * NW, dec2_waves_per_simd(LOGA, NW)) void k_decode2(DecArgs a) {
    constexpr int S = 2;
    __shared__ uint32_t tab[(1 << LOGA) * 128];  // [symbol][stream][lane]
    __shared__ float dq[128];
    constexpr uint32_t kPoolBytes = NW * pool_per_wave2(LOGA);
    __shared__ uint32_t pool_w[(kPoolBytes + kPoolSlack) / 4];  // staged payload
    __shared__ uint32_t need_w[NW];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int A = a.A;
    const int CB2 = (a.C + 127) >> 7;

    // Block -> (slab, chunk group g, 128-channel block cb2), slab slowest.
    // Blocks start in roughly this order, slabs K then V by layer, so the K
    // slabs of the first layers, which the default per-layer bins make the
    // widest and slowest to decode, start first and finish among the later
    // slabs' rounds instead of in the tail (with the chunk group slowest:
    // the 32K-token call 1.66 -> 1.57 ms, the GLM-4-9B shape 0.41 -> 0.36
    // ms); a slab's chunk groups, which share its tables, run together.
    const int bid = blockIdx.x;
    const int ngr = (a.NCr + NW - 1) / NW;
    const int cb2 = bid % CB2;
    const int g = (bid / CB2) % ngr;
    const int slab = bid / (CB2 * ngr);
    const SlabLoc sl = slab_loc(a.cm, slab);
    const int kv = sl.kv, l = sl.l;
    int cch[S];
    bool act[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        cch[s] = cb2 * 128 + 2 * lane + s;
        act[s] = cch[s] < a.C;
    }
    const int M = layer_m(a.mt, kv, l);
    const int W = layer_w(a.mt, kv, l);
    if (2 * M + 1 < a.nsym_lo || 2 * M + 1 > a.nsym_hi) return;  // block-uniform
    uint64_t payload_bytes;
    const uint8_t *payload = call_payload(a, sl, payload_bytes);
    const uint16_t *cdf16 = call_sec(a.cdf16, a.cm, sl.b);

    // This wave's chunk and its 128 streams: lengths, offsets (the two tiles
    // 2 cb2, 2 cb2 + 1 are adjacent in the payload) and the pool bytes they
    // need (alignment head + bytes + four zero bytes after each stream).
    const int jr = g * NW + wv, j = a.j0 + jr;
    const int n = jr < a.NCr ? min(kChunk, a.T - j * kChunk) : 0;
    const int t0 = (a.j0 + min(jr, a.NCr - 1)) * kChunk;
    uint32_t len[S] = {0u, 0u}, excl = 0, total = 0;
    uint64_t base = 0;
    bool corrupt = false;
    if (n) {
        const uint16_t *lp = call_sec(a.lengths, a.cm, sl.b) + ((int64_t)j * 2 * a.cm.Lc + sl.ls) * a.C;
#pragma unroll
        for (int s = 0; s < S; ++s) len[s] = act[s] ? lp[cch[s]] : 0u;
        const uint32_t pr = len[0] + len[1];
        const uint32_t incl = wave_incl_scan_u32(pr, lane);
        total = (uint32_t)__shfl((int)incl, 63, 64);
        excl = incl - pr;
        base = a.tile_off[((int64_t)j * 2 * a.L + slab) * a.CB + 2 * cb2];
        if (base > payload_bytes || total > payload_bytes - base) {
            corrupt = true;  // offsets point outside the payload: decode from nothing
            len[0] = len[1] = excl = total = 0;
            base = 0;
        }
    }
    const uint32_t need_total = ((uint32_t)(base & 3u) + total + 4u * 128u + 4u + 3u) & ~3u;
    if (lane == 0) need_w[wv] = need_total;
    __syncthreads();
    uint32_t woff = 0;
    for (int i = 0; i < wv; ++i) woff += need_w[i];
    const bool staged = woff + need_total <= kPoolBytes;

    DecStream st[S];
    uint8_t *pool = reinterpret_cast<uint8_t *>(pool_w);
    uint32_t soff[S];  // offset of each stream from the wave's first payload byte
    soff[0] = excl;
    soff[1] = excl + len[0];
    if (staged) {
        for (uint32_t i = lane; i < need_total / 4; i += 64) pool_w[woff / 4 + i] = 0;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            // LDS start of this stream: congruent to its payload offset mod 4.
            const uint64_t g0 = base + soff[s];
            const uint32_t ls = woff + (uint32_t)(base & 3u) + soff[s] + 4u * (uint32_t)(2 * lane + s);
            st[s].ptr = ls;
            if (len[s]) {
                const uint64_t gend = g0 + len[s];
                const uint64_t ga = g0 & ~3ull, ge = (gend + 3) & ~3ull;
                uint32_t la = ls - (uint32_t)(g0 - ga);
#pragma unroll 4
                for (uint64_t gw = ga; gw < ge; gw += 4, la += 4) {
                    uint32_t v = load_word(payload, payload_bytes, gw);
                    if (gw < g0) v &= 0xFFFFFFFFu << (8 * (uint32_t)(g0 - gw));
                    if (gw + 4 > gend) v &= 0xFFFFFFFFu >> (8 * (uint32_t)(gw + 4 - gend));
                    pool_w[la >> 2] = v;
                }
            }
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        st[s].len = len[s];
        st[s].pos = 0;
        st[s].gsrc = payload + base + soff[s];
        st[s].range = 0xFFFFFFFFu;
        st[s].code = 0;
        if (!staged) st[s].ptr = 0;
    }

    // Tables, built by the block's waves together: wave w writes symbols w,
    // w + NW, ...; entries past the table's width W (up to 2^LOGA) have start
    // 0xFFFF. Idle channels: code stays 0, so they always decode symbol 0,
    // whose frequency 65535 never forces a renormalisation.
    bool bad_table = false;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const LaneTable lt = lane_table(a.cdf32, cdf16, a.wpre, sl.ls, a.C, min(cch[s], a.C - 1), A, W);
        for_lane_bounds<((1 << LOGA) + NW - 1) / NW, kTabGroup>(lt, wv, NW, 1 << LOGA, [&](int q, uint32_t lo, uint32_t hi) {
            uint32_t entry = 0xFFFFu;
            if (q < W && act[s]) {
                uint32_t f = hi - lo;
                if (hi <= lo || hi > kProbOne || (q == 0 && lo != 0) || (q == W - 1 && hi != kProbOne)) {
                    bad_table = true;
                    f = 1;
                }
                entry = (lo & 0xFFFFu) | (f << 16);
            } else if (q < W) {
                entry = q == 0 ? 0xFFFFu << 16 : (uint32_t)q | (1u << 16);
            }
            tab[(q * 2 + s) * 64 + lane] = entry;
        });
    }
    // Per-token scales of the chunk: lane i of sc_v[k] holds token 64k + i.
    uint32_t sc_v[4];
    {
        const uint16_t *sp = call_sec(a.scale, a.cm, sl.b) + (int64_t)sl.ls * a.T + t0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t = 64 * k + lane;
            sc_v[k] = FUSED && t < n ? (uint32_t)sp[t] : 0u;
        }
    }
    if (FUSED && wv == 0) {
        dq[lane] = __fdiv_rn((float)(lane - M), (float)M);
        dq[lane + 64] = __fdiv_rn((float)(lane + 64 - M), (float)M);
    }
    __syncthreads();

    // Output rows: a buffer over this (K|V, layer) slab; the row offset is
    // wave-uniform, the lane offset constant; idle lanes point past the end.
    const uint32_t esz = FUSED ? 2u : 1u;
    const uint64_t slab_elems = (uint64_t)a.T * a.C;
    const void *obase = FUSED ? (const void *)(a.kv + ((int64_t)sl.lv * 2 + kv) * (int64_t)slab_elems)
                              : (const void *)(a.sym + (int64_t)slab * (int64_t)slab_elems);
    __amdgpu_buffer_rsrc_t out_rsrc = make_rsrc(obase, (uint32_t)(slab_elems * esz));
    int pg_t0 = 0, pg_b0 = 0;
    uint32_t pg_v = 0;
    if constexpr (PAGED) {
        const uint32_t bs_log = (uint32_t)a.paged.log2_bs;
        const uint32_t region = ((uint32_t)a.paged.num_blocks << bs_log) * (uint32_t)a.C * 2u;
        out_rsrc = make_rsrc(a.paged.cache + (int64_t)sl.lv * a.paged.layer_stride + (int64_t)kv * a.paged.kv_stride,
                             region);
        const int nblk_total = (a.T + (1 << bs_log) - 1) >> bs_log;
        bool bad_block = false;
        pg_t0 = t0;
        pg_b0 = t0 >> bs_log;
        const int bi = pg_b0 + lane;
        if (n && bi < nblk_total && bi <= ((t0 + n - 1) >> bs_log)) {
            const int32_t e = a.paged.table[bi];
            if (e < 0 || e >= a.paged.num_blocks) {
                bad_block = true;
                pg_v = (uint32_t)a.paged.num_blocks;
            } else {
                pg_v = (uint32_t)e;
            }
        }
        if (__ballot(bad_block) && lane == 0) atomicOr(a.status, kStCorrupt);
    }
    const uint32_t out_voff = act[0] ? (uint32_t)cch[0] * esz : 0x7FFFFFF0u;
    const uint32_t rowoff = (uint32_t)t0 * (uint32_t)a.C * esz;

    uint64_t bad_mask = 0;
    // The lower half of the table suffices when every symbol of the layer,
    // 0..2M, lies below its top entry 2^(LOGA-1) - 1.
    const bool half = LOGA >= 3 && M + 1 <= (1 << (LOGA - 2));
    // Every lane's two channels exist and their bf16 pair is 4-byte aligned.
    const bool full = FUSED && (a.C & 127) == 0;
#define CG_DL2(ST, HF, FL)                                                                                        \
    decode_loop2<FUSED, LOGA, CLAMP, ST, HF, PAGED, TAIL, FL>(a, st, n, rowoff, pg_t0, pg_b0, pg_v, tab, dq, sc_v, \
                                                              pool, out_rsrc, out_voff, lane, W, cdf16, sl.ls, cch, \
                                                              bad_mask)
    if (full) {
        if (half) {
            if (staged) CG_DL2(true, LOGA >= 3, true);
            else CG_DL2(false, LOGA >= 3, true);
        } else {
            if (staged) CG_DL2(true, false, true);
            else CG_DL2(false, false, true);
        }
    } else {
        if (half) {
            if (staged) CG_DL2(true, LOGA >= 3, false);
            else CG_DL2(false, LOGA >= 3, false);
        } else {
            if (staged) CG_DL2(true, false, false);
            else CG_DL2(false, false, false);
        }
    }
#undef CG_DL2
    const uint64_t act_mask = __ballot(act[0]) | __ballot(act[1]);
    if ((__ballot((act[0] || act[1]) && (corrupt || bad_table)) | (bad_mask & act_mask)) && lane == 0)
        atomicOr(a.status, kStCorrupt);
}

template <bool FUSED, int LOGA, int NW, bool PAGED, bool TAIL>
static hipError_t launch_decode2_s(const Dims &d, const DecArgs &a, bool clamp, hipStream_t s) {
    const int ngroups = (a.NCr + NW - 1) / NW;
    const int CB2 = (d.C + 127) / 128;
    const dim3 grid((unsigned)((int64_t)ngroups * 2 * d.L * CB2));
    if (!clamp)
        hipLaunchKernelGGL((k_decode2<FUSED, LOGA, false, NW, PAGED, TAIL>), grid, dim3(64 * NW), 0, s, a);
    else
        hipLaunchKernelGGL((k_decode2<FUSED, LOGA, true, NW, PAGED, TAIL>), grid, dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

// One launch of the paired decoder over every slab, with tables of the
// call's width; the 16-bin slabs search the lower half. (A 16-entry launch
// for those slabs needs the global-memory tail search for symbols above the
// table, whose registers cost a quarter of the residency.)
template <bool FUSED, int NW, bool PAGED>
static hipError_t launch_decode2_f(const Dims &d, DecArgs a, hipStream_t s) {
    int loga = 2;
    while ((1 << loga) < d.A) ++loga;
    a.nsym_lo = 0;
    a.nsym_hi = 1 << 30;
    const bool clamp = !(d.A == (1 << loga) && d.wmin == d.A);
    switch (loga) {
    case 2: return launch_decode2_s<FUSED, 2, NW, PAGED, false>(d, a, clamp, s);
    case 3: return launch_decode2_s<FUSED, 3, NW, PAGED, false>(d, a, clamp, s);
    case 4: return launch_decode2_s<FUSED, 4, NW, PAGED, false>(d, a, clamp, s);
    case 5: return launch_decode2_s<FUSED, 5, NW, PAGED, false>(d, a, clamp, s);
    case 6: return launch_decode2_s<FUSED, 6, NW, PAGED, false>(d, a, clamp, s);
    default: return launch_decode2_s<FUSED, 7, NW, PAGED, false>(d, a, clamp, s);
    }
}

// Waves (over the chip) up to which a launch of one- or two-wave blocks
// takes a large pool: eight per CU (LAT 1), sixteen (LAT 2).
constexpr int64_t kLatWaves = 8 * 256, kLat2Waves = 16 * 256;

template <int S, bool FUSED, int LOGA, int NW, bool PAGED, bool TAIL>
static hipError_t launch_decode_s(const Dims &d, const DecArgs &a, bool clamp, hipStream_t s) {
    const int ngroups = (a.NCr + S * NW - 1) / (S * NW);
    const dim3 grid((unsigned)((int64_t)ngroups * 2 * d.L * d.CB));
    constexpr bool kLat = NW <= 2;
    const int64_t waves = (int64_t)grid.x * NW;
    const int lat = !kLat ? 0 : waves <= kLatWaves ? 1 : waves <= kLat2Waves ? 2 : 0;
#define CG_DEC(CL, LT) hipLaunchKernelGGL((k_decode<S, FUSED, LOGA, CL, NW, PAGED, TAIL, LT>), grid, dim3(64 * NW), 0, s, a)
    // clamp: some table is narrower than the 2^LOGA entries.
    if (lat == 1) {
        if constexpr (kLat) {
            if (!clamp) CG_DEC(false, 1);
            else CG_DEC(true, 1);
        }
    } else if (lat == 2) {
        if constexpr (kLat) {
            if (!clamp) CG_DEC(false, 2);
            else CG_DEC(true, 2);
        }
    } else {
        if (!clamp) CG_DEC(false, 0);
        else CG_DEC(true, 0);
    }
#undef CG_DEC
    return hipGetLastError();
}

template <int S, bool FUSED, int NW, bool PAGED = false>
static hipError_t launch_decode_f(const Dims &d, const MaxTable &mt, DecArgs a, hipStream_t s) {
    int loga = 2;
    while ((1 << loga) < d.A) ++loga;
    a.nsym_lo = 0;
    a.nsym_hi = 1 << 30;
    if constexpr (NW <= 2) {
        // Blocks of one or two waves are held back by their LDS table. The
        // slabs whose quantiser symbols fit 16 entries (2M + 1 <= 16, the
        // 16-bin layers) take a launch with 16-entry tables (a rare symbol
        // above them is looked up in global memory); the others take the
        // full width in a second launch. A call too small to fill the GPU
        // (a single short call) runs both kinds in one launch instead: its
        // time is one stream's latency, which two launches in a row double.
        const int64_t blocks = (int64_t)((a.NCr + S * NW - 1) / (S * NW)) * 2 * d.L * d.CB;
        if (loga > 4) {
            bool small = false, large = false, small_narrow = false;
            for (int kv = 0; kv < 2; ++kv)
                for (int l = 0; l < d.Lc; ++l) {
                    const int b = mt.bins[kv][l], w = mt.per_layer ? b : d.A;
                    if (2 * (b / 2 - 1) + 1 <= 16) {
                        small = true;
                        small_narrow |= w < 16;
                    } else {
                        large = true;
                    }
                }
            if (small && (!large || blocks >= 16384)) {
                a.nsym_hi = 16;
                hipError_t e = launch_decode_s<S, FUSED, 4, NW, PAGED, true>(d, a, small_narrow, s);
                if (e != hipSuccess || !large) return e;
                a.nsym_lo = 17;
                a.nsym_hi = 1 << 30;
            }
        }
    }
    const bool clamp = !(d.A == (1 << loga) && d.wmin == d.A);
    switch (loga) {
    case 2: return launch_decode_s<S, FUSED, 2, NW, PAGED, false>(d, a, clamp, s);
    case 3: return launch_decode_s<S, FUSED, 3, NW, PAGED, false>(d, a, clamp, s);
    case 4: return launch_decode_s<S, FUSED, 4, NW, PAGED, false>(d, a, clamp, s);
    case 5: return launch_decode_s<S, FUSED, 5, NW, PAGED, false>(d, a, clamp, s);
    case 6: return launch_decode_s<S, FUSED, 6, NW, PAGED, false>(d, a, clamp, s);
    default: return launch_decode_s<S, FUSED, 7, NW, PAGED, false>(d, a, clamp, s);
    }
}

hipError_t launch_decode(const Dims &d, const MaxTable &mt, const DecodeIn &in, const DecodeOut &out,
                         uint64_t *tile_off, uint64_t *scan_tmp, uint32_t *status, hipStream_t s) {
    const int j0 = in.j0, j1 = in.j1 < 0 ? d.NC : in.j1;
    // Table offsets: only the per-layer format needs them computed.
    uint32_t *wpre = in.cdf16 && d.fmt == CG_TABLES_PER_LAYER ? in.wpre : nullptr;
    if (wpre) {
        hipError_t e0 = launch_table_prefix(d, mt, wpre, s);
        if (e0 != hipSuccess) return e0;
    }
    if ((j0 != 0 || j1 != d.NC || out.paged.cache) && d.Lc != d.L) return hipErrorInvalidValue;  // one call only
    TileScan ts{nullptr, in.lengths, tile_off, scan_tmp, nullptr, in.chunk_off, in.payload_bytes, in.call_sizes,
                in.payload_off, status, d.L, d.C, d.CB, d.NC, call_map(d), j0, d.Lc == d.L ? j1 - j0 : -1};
    const bool one_block = call_scan_fits(ts) && d.Lc == d.L;
    hipError_t e;
    if (in.zero_status && !one_block && (e = launch_fill_u32(status, 0u, 1, s)) != hipSuccess) return e;
    e = call_scan_fits(ts) ? launch_call_scan(ts, nullptr, s, in.zero_status && one_block) : launch_tile_scan(ts, s);
    if (e != hipSuccess) return e;
    DecArgs a;
    a.cm = call_map(d);
    a.call_sizes = in.call_sizes;
    a.payload_off = in.payload_off;
    a.payload = in.payload;
    a.payload_bytes = in.payload_bytes;
    a.lengths = in.lengths;
    a.tile_off = tile_off;
    a.cdf32 = in.cdf32;
    a.cdf16 = in.cdf16;
    a.wpre = wpre;
    a.sym = out.sym;
    a.kv = out.kv;
    a.scale = out.scale;
    a.status = status;
    a.paged = out.paged;
    a.mt = mt;
    a.L = d.L;
    a.T = d.T;
    a.C = d.C;
    a.A = d.A;
    a.NC = d.NC;
    a.j0 = j0;
    a.NCr = j1 - j0;
    const int ncr = a.NCr;
    a.CB = d.CB;
    // Two streams per lane and eight (or four) waves per block when there are
    // enough chunks; otherwise one stream per lane and as few waves as chunks.
    if (out.paged.cache) {
        if (ncr >= 16) return launch_decode2_f<true, 8, true>(d, a, s);
        if (ncr >= 8) return launch_decode2_f<true, 4, true>(d, a, s);
        if (ncr >= 2) return launch_decode_f<1, true, 2, true>(d, mt, a, s);
        return launch_decode_f<1, true, 1, true>(d, mt, a, s);
    }
    const bool fused = out.kv != nullptr;
    if (ncr >= 16)
        return fused ? launch_decode2_f<true, 8, false>(d, a, s) : launch_decode2_f<false, 8, false>(d, a, s);
    if (ncr >= 8)
        return fused ? launch_decode2_f<true, 4, false>(d, a, s) : launch_decode2_f<false, 4, false>(d, a, s);
    if (ncr >= 2)
        return fused ? launch_decode_f<1, true, 2>(d, mt, a, s) : launch_decode_f<1, false, 2>(d, mt, a, s);
    return fused ? launch_decode_f<1, true, 1>(d, mt, a, s) : launch_decode_f<1, false, 1>(d, mt, a, s);
}

}  // namespace cg
