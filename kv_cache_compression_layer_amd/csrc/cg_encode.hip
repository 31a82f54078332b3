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
// Kernels:
//
// k_encode: a block of NW waves (four for calls of eight 256-token chunks
// or more, else one) owns 64 consecutive channels (lane = channel) of one
// (K|V, layer) and NW * S chunks; each wave codes S chunks per lane: two
// interleaved (independent dependency chains), or one (calls of one chunk;
// grids small enough that a wave has its SIMD nearly to itself; the wider
// launch of a split, see enc_plan and launch_encode). The
// waves share one table per lane in LDS, start | freq << 16 laid out
// [symbol][lane] (no bank conflicts whatever the symbols). Symbols come
// straight from global memory into a register ring of prefetches, so the
// loop never waits on them: from [T][C] byte rows (64 lanes read one 64-byte
// row per load), or, in cg_to_bytes, from the quantiser's packed layout (one
// dword per lane per 8 tokens as nibbles, or per 4 tokens as bytes). Bytes
// are written as soon as they are shifted out into an LDS stage per stream
// ([row][lane]); rows past the stage spill to the tile's 16 KiB staging slot
// in global memory. At the end the wave gathers the tile's streams in
// stream order into the slot, contiguously, and writes the stream lengths
// and the tile's byte total. A stream longer than the slot (256 bytes)
// marks the tile as an overflow tile.
//
// launch_call_scan, or launch_tile_scan + k_chunk_scan: exclusive scan of
// the tile totals in stream order (per chunk, then over the chunk totals)
// -> tile offsets, chunk offsets and the payload size.
//
// k_compact: one wave per tile copies the gathered tile to its offset (a
// tile too large for the LDS gather is gathered here from the slot's rows),
// and re-encodes every stream of an overflow tile straight to its final
// offset with a byte-at-a-time coder that holds back the last byte and the
// run of 0xFF after it until no carry can reach them (fixup_tile).
#include "cg_internal.hpp"

namespace cg {

constexpr int kStageBytes = 256;  // staging slot bytes per stream (5 bits/symbol fit)
constexpr int kRing = 16;         // symbol prefetch depth

// What k_encode left in a tile's staging slot: the tile's bytes in stream
// order at slot bytes [0, total) (gathered), each stream's bytes in slot rows
// [row][lane] (rows), or a stream too long for the slot, re-coded by fixup_tile
// (overflow).
constexpr uint8_t kTileGathered = 0, kTileRows = 1, kTileOverflow = 2;

// ----------------------------------------------------------- fix-up coder

struct RcEncHold {
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
        while (range < kTop) {
            shift(out);
            range <<= 8;
        }
    }

    template <class Sink>
    __device__ __forceinline__ void flush(Sink &out) {
        uint32_t b = (low >> 24) + ((low & 0xFFFFFFu) != 0);  // ceil(low / 2^24), 0..256
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

// ------------------------------------------------------------ main coder

struct EncArgs {
    const uint8_t *sym;
    const int32_t *cdf;        // int32 tables, or
    const uint16_t *cdf16;     // u16 wire tables, placed by wpre
    const uint32_t *wpre;
    uint8_t *staging;          // [tiles][kStageBytes][64] bytes
    uint32_t *tile_sum;        // [tiles]
    uint8_t *tile_mode;        // [tiles] kTileGathered / kTileRows / kTileOverflow
    uint16_t *lengths;         // [NC, 2L, C]
    WsHeader *hdr;
    int L, T, C, A, NC, CB;
    MaxTable mt;               // table width of each (K|V, layer)
    CallMap cm;                // calls of a batch (tables and lengths per call)
    // This launch codes only the slabs whose symbol count 2M+1 lies in
    // [nsym_lo, nsym_hi]; the other blocks return at once.
    int nsym_lo, nsym_hi;
};

// Tile = (chunk j, slab = kv*L + l, 64-channel block cb); tile index in
// stream order: (j * 2L + slab) * CB + cb.
__device__ __forceinline__ int64_t tile_index(int j, int slab, int cb, int L, int CB) {
    return ((int64_t)j * 2 * L + slab) * CB + cb;
}

// Range coder. Every byte is written as soon as it is shifted out, except the
// last one, `pend`, which still takes the carry of the next step. A carry
// that lifts pend past 0xFF is added to the bytes already written, walking
// back through the run of 0xFF bytes (rare: the written prefix must end in
// 0xFF). Bytes go to an LDS stage of R + 2 rows ([row][lane], rows kRowPitch
// bytes apart; a wider pitch that spreads a column over the banks costs a
// block of residency per CU, which is worth more; row 0 holds the
// placeholder in front of the stream, which no carry ever reaches; row R + 1
// is a spare that takes the LDS writes of rows past R); bytes past row R also
// go to the tile's staging slot in global memory, row pos - 1, through a
// buffer whose range is the slot (bytes past the slot are dropped; such a
// stream is re-coded by fixup_tile).
// The coder tracks the LDS address of its next row, `la`, rather than the row
// number (row = (la - lrow0) / kRowPitch), so a byte costs one min (clamp to
// the spare row) and one compare (spill test) besides the write.
constexpr int kRowPitch = 64;  // LDS stage row pitch in bytes

template <int R>
struct Coder {
    uint32_t low, range, pend;
    uint32_t la;      // LDS byte address of the next byte's row for this lane
    uint32_t lrow0;   // LDS byte address of this lane's row 0
    uint32_t llast;   // LDS byte address of row R (the last row of the stage)
    uint32_t sbase;   // LDS byte address of the stream's stage (lrow0 - lane), wave-uniform
    __device__ __forceinline__ void init(uint32_t stream_base, int lane) {
        low = 0;
        range = 0xFFFFFFFFu;
        pend = 0;
        sbase = stream_base;
        lrow0 = stream_base + (uint32_t)lane;
        la = lrow0;
        llast = lrow0 + (uint32_t)R * kRowPitch;
    }
    __device__ __forceinline__ int pos() const { return (int)((la - lrow0) / kRowPitch); }
    // Writes byte b at the next row: the LDS stage (rows past R land in the
    // spare row R + 1), and the global slot for rows past the stage (row
    // p goes to slot row p - 1), behind a wave-uniform test since few lanes
    // get there.
    __device__ __forceinline__ void put(uint8_t *lds, __amdgpu_buffer_rsrc_t slot, uint32_t b) {
        lds[min(la, llast + kRowPitch)] = (uint8_t)b;
        if (__builtin_amdgcn_ballot_w64(la > llast)) {
            __asm__ volatile("" ::: "memory");
            if (la > llast)
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b, slot, (int)(la - sbase - kRowPitch), 0, 0);
        }
        la += kRowPitch;
    }
    __device__ __forceinline__ void carry_back(uint8_t *lds, __amdgpu_buffer_rsrc_t slot, int lane) {
        uint32_t c = pend >> 8;
        for (int k = min(pos(), kStageBytes + 1) - 1; k >= 1 && c; --k) {
            uint32_t v;
            if (k <= R) {
                v = lds[lrow0 + k * kRowPitch] + c;
                lds[lrow0 + k * kRowPitch] = (uint8_t)v;
            } else {
                v = __builtin_amdgcn_raw_buffer_load_b8(slot, (k - 1) * 64 + lane, 0, 0) + c;
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, slot, (k - 1) * 64 + lane, 0, 0);
            }
            c = v >> 8;
        }
    }
    // pend past 0xFF: add its carry to the bytes already written. Rare, so it
    // sits behind a wave-uniform test (and a real branch).
    __device__ __forceinline__ void settle(uint8_t *lds, __amdgpu_buffer_rsrc_t slot, int lane) {
        if (__builtin_amdgcn_ballot_w64(pend > 0xFFu)) {
            __asm__ volatile("" ::: "memory");
            if (pend > 0xFFu) carry_back(lds, slot, lane);
        }
    }
    // One byte shift: pend goes out, the top byte of low becomes pend.
    __device__ __forceinline__ void shift(uint8_t *lds, __amdgpu_buffer_rsrc_t slot, int lane) {
        settle(lds, slot, lane);
        put(lds, slot, pend);
        pend = low >> 24;
        low <<= 8;
        range <<= 8;
    }
    __device__ __forceinline__ void step(uint32_t e, uint8_t *lds, __amdgpu_buffer_rsrc_t slot, int lane) {
        const uint32_t r = range >> 16;
        uint32_t nl;
        const bool c = __builtin_add_overflow(low, (uint32_t)__umul24(r, e & 0xFFFFu), &nl);
        low = nl;
        pend += (uint32_t)c;  // at most one wrap between two shifts
        range = __umul24(r, e >> 16);
        // range >= 2^8 here (r >= 2^8, freq >= 1): one shift, or two when
        // range < 2^16 (a rare symbol), the second behind a wave-uniform
        // branch. pend is at most 0xFF before the second, so it settles
        // nothing.
        if (range < kTop) {
            shift(lds, slot, lane);
            // Keep the shifted state in its registers: otherwise the second
            // shift is rebuilt from the unshifted values (low << 16 ...) and
            // the two paths merge through register copies.
            __asm__ volatile("" : "+v"(low), "+v"(range), "+v"(pend), "+v"(la));
            if (__builtin_amdgcn_ballot_w64(range < kTop)) {
                __asm__ volatile("" ::: "memory");
                if (range < kTop) shift(lds, slot, lane);
            }
        }
    }
    // Final value: the smallest multiple of 2^24 >= low; returns the length.
    __device__ __forceinline__ uint32_t flush(uint8_t *lds, __amdgpu_buffer_rsrc_t slot, int lane) {
        uint32_t b = (low >> 24) + ((low & 0xFFFFFFu) != 0);  // 0..256
        if (b == 256u) {
            pend += 1;
            b = 0;
        }
        if (pend > 0xFFu) carry_back(lds, slot, lane);
        put(lds, slot, pend);
        if (b) put(lds, slot, b);
        return (uint32_t)(pos() - 1);
    }
};

// LDS stage rows per stream: 44 in four-wave blocks with tables wider than
// 16 entries (longer streams, which would otherwise spill to the slot), 28
// elsewhere (the 16-bin slabs' short streams, and one-wave blocks of short
// calls, whose residency the LDS decides).
constexpr int kLdsRows = 28;
constexpr int kLdsRowsWide = 44;
__host__ __device__ constexpr int enc_rows(int loga, int nw) { return loga >= 5 && nw >= 4 ? kLdsRowsWide : kLdsRows; }

// Block of NW waves for one (K|V, layer, 64-channel block); wave w codes the
// S chunks (group * NW + w) * S + s, lane = channel, with the table the
// waves share.
// TRUSTED: the symbols come from this library's quantiser, so every symbol
// is at most 2M < bins <= W (the table width) and neither the clamp of the
// table index nor the range check is needed.
// PK: symbol layout. 0 = u8 [T][C] rows; 1 = nibble dwords of 8-token groups
// and 2 = byte dwords of 4-token groups, as k_quantize_hist writes them for
// slabs of at most 16 symbols and for the others (trusted symbols only).
template <int S, int LOGA, int NW, bool TRUSTED, int PK>
__global__ __launch_bounds__(64 * NW) void k_encode(EncArgs a) {
    static_assert(PK == 0 || TRUSTED, "packed symbols come from the quantiser");
    constexpr int R = enc_rows(LOGA, NW);
    // One-wave blocks (calls of fewer than eight chunks) are as many per CU as
    // their LDS allows, so they keep 16-bit starts, [symbol][lane], W + 1 of
    // them (2^16 stored as 0), and take a symbol's frequency as the
    // difference of two starts; larger blocks keep start | freq << 16.
    constexpr bool T16 = NW == 1;
    __shared__ uint32_t tab[T16 ? ((1 << LOGA) + 1) * 32 : (1 << LOGA) * 64];  // [symbol][lane]
    __shared__ __attribute__((aligned(16))) uint8_t stage[NW * S * (R + 2) * kRowPitch];  // [wave][stream][row][lane]
    const int lane = threadIdx.x & 63;
    // Wave index, uniform across the wave (readfirstlane keeps what derives
    // from it in scalar registers).
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int A = a.A;

    // Block -> (chunk group g, slab, cb); all wave-uniform. Neighbouring
    // channel blocks read the two halves of the same 128-byte symbol lines,
    // so they are kept on one XCD.
    const int bid = xcd_work_index(blockIdx.x, gridDim.x);
    const int cb = bid % a.CB;
    const int slab = (bid / a.CB) % (2 * a.L);
    const int g = bid / (a.CB * 2 * a.L);
    const int c = cb * 64 + lane;
    const bool active = c < a.C;
    const int lane_off = active ? lane : (a.C - 1 - cb * 64);  // in-bounds column for idle lanes
    const SlabLoc sl = slab_loc(a.cm, slab);
    const int nsym = 2 * layer_m(a.mt, sl.kv, sl.l) + 1;
    if (nsym < a.nsym_lo || nsym > a.nsym_hi) return;  // block-uniform
    const uint16_t *cdf16 = call_sec(a.cdf16, a.cm, sl.b);  // the call's wire tables

    // Symbols are read through a buffer over this (K|V, layer) slab: the row
    // offset is wave-uniform (scalar), the column the lane's constant offset.
    const __amdgpu_buffer_rsrc_t srsrc = make_rsrc(a.sym + (int64_t)slab * a.T * a.C, (uint32_t)((int64_t)a.T * a.C));
    const int col = cb * 64 + lane_off;
    int n[S], row0[S];
    __amdgpu_buffer_rsrc_t slot[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int j = (g * NW + wv) * S + s;
        n[s] = j < a.NC ? min(kChunk, a.T - j * kChunk) : 0;
        row0[s] = min(j, a.NC - 1) * kChunk;
        slot[s] = make_rsrc(a.staging + tile_index(min(j, a.NC - 1), slab, cb, a.L, a.CB) * (kStageBytes * 64),
                            kStageBytes * 64);
    }
    const int nmax = n[0];  // the first chunk of a wave is never the short one

    // Prefetch ring: symbol of token t of stream s sits in ring[s][t % kRing]
    // from kRing tokens before it is coded. Loads are unconditional (rows are
    // clamped into the stream) so their waits are exact.
    uint32_t ring[S][kRing];
    // Packed symbols: a ring of RD dwords of TPD tokens each (KR tokens),
    // group gb[s] + m in slot m; the stream's groups are gb[s] .. gb[s] + gl[s].
    constexpr int TPD = PK == 1 ? 8 : 4;
    constexpr int KR = PK == 1 ? 32 : 16;
    constexpr int RD = KR / TPD;
    uint32_t rd[S][RD];
    int gb[S], gl[S];
    if constexpr (PK == 0) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int last = max(n[s] - 1, 0);
#pragma unroll
            for (int k = 0; k < kRing; ++k) {
                ring[s][k] = __builtin_amdgcn_raw_buffer_load_b8(srsrc, col, (row0[s] + min(k, last)) * a.C, 0);
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            gb[s] = row0[s] / TPD;
            gl[s] = max(n[s] / TPD - 1, 0);
#pragma unroll
            for (int m = 0; m < RD; ++m)
                rd[s][m] = __builtin_amdgcn_raw_buffer_load_b32(srsrc, col * 4, (gb[s] + min(m, gl[s])) * a.C * 4, 0);
        }
    }

    // Tables, built by the block's waves together: one per lane, packed
    // start | freq << 16, [symbol][lane]; W symbols (the slab's table width).
    const int W = layer_w(a.mt, sl.kv, sl.l);
    bool bad = false;
    // A launch for slabs of at most 2^LOGA symbols holds only that many
    // entries of a wider table: the quantiser's symbols never reach the rest.
    const int WT = min(W, 1 << LOGA);
    // Loads use the in-bounds column col (the lane's own for active lanes).
    const LaneTable lt = lane_table(a.cdf, cdf16, a.wpre, sl.ls, a.C, col, A, W);
    if constexpr (T16) {
        // Starts 0..WT (start WT is 2^16, stored as 0, when WT == W). Idle
        // lanes write nothing and read the table of an active column.
        uint16_t *tab16 = reinterpret_cast<uint16_t *>(tab);
        for_lane_bounds<(1 << LOGA) + 1, kTabGroup>(lt, 0, 1, WT + 1, [&](int s, uint32_t lo, uint32_t hi) {
            if (!active) return;
            uint32_t v = 0;
            if (s < W) {
                v = lo;
                if (s < WT) bad |= hi <= lo || hi > kProbOne || (s == 0 && lo != 0) || (s == W - 1 && hi != kProbOne);
            }
            tab16[s * 64 + lane] = (uint16_t)v;
        });
    } else {
        // Wave wv writes symbols wv, wv + NW, ...
        for_lane_bounds<((1 << LOGA) + NW - 1) / NW, kTabGroup>(lt, wv, NW, WT, [&](int s, uint32_t lo, uint32_t hi) {
            uint32_t entry;
            if (active) {
                uint32_t f = hi - lo;
                if (hi <= lo || hi > kProbOne || (s == 0 && lo != 0) || (s == W - 1 && hi != kProbOne)) {
                    bad = true;
                    f = 1;
                }
                entry = (lo & 0xFFFFu) | (f << 16);
            } else {
                // Idle lanes code with frequency 65535 whatever their symbol:
                // they never shift a byte out.
                entry = 0xFFFFu << 16;
            }
            tab[s * 64 + lane] = entry;
        });
    }
    __syncthreads();

    Coder<R> cd[S];
#pragma unroll
    for (int s = 0; s < S; ++s) cd[s].init((uint32_t)((wv * S + s) * (R + 2) * kRowPitch), lane);
    const uint32_t amax = (uint32_t)W - 1;
    uint32_t qmax = 0;
    // Table entry of the next token of every stream, read one step ahead.
    uint32_t e_next[S];
    // Byte address of (symbol q, this lane) in tab, q * 256 + lane * 4: a
    // trusted symbol is byte 0 of its load, and one byte permute places it
    // next to lane * 4 (which is below 256).
    const uint32_t lane4 = (uint32_t)lane * 4;
    const uint8_t *tabb = reinterpret_cast<const uint8_t *>(tab);
    // 16-bit starts: byte address q * 128 + column * 2; the entry is rebuilt
    // as start | (next start - start) << 16 (the difference mod 2^16 is the
    // frequency, 2^16 - start for the last symbol).
    const uint32_t tl2 = (uint32_t)lane_off * 2;
    auto e16 = [&](uint32_t ad) -> uint32_t {
        const uint32_t lo = *reinterpret_cast<const uint16_t *>(tabb + ad);
        const uint32_t hi = *reinterpret_cast<const uint16_t *>(tabb + ad + 128);
        return lo | ((hi - lo) << 16);
    };
    auto entry = [&](uint32_t q) -> uint32_t {
        if constexpr (T16) return e16(((TRUSTED ? q : min(q, amax)) << 7) | tl2);
        if (TRUSTED) return *reinterpret_cast<const uint32_t *>(tabb + __builtin_amdgcn_perm(q, lane4, 0x0c0c0400u));
        return tab[min(q, amax) * 64 + lane];
    };
    // Packed: table entry of token p of a group dword w. Byte layout: byte p
    // goes next to lane4 by one permute; nibble layout: token p sits at bit
    // 8 * (p % 4) + 4 * (p / 4) and is shifted to bits 8..11.
    auto pentry = [&](uint32_t w, int p) -> uint32_t {
        if constexpr (T16) {
            const int b = PK == 2 ? 8 * p : 8 * (p & 3) + 4 * (p >> 2);
            return e16((__builtin_amdgcn_ubfe(w, b, PK == 2 ? 8 : 4) << 7) | tl2);
        }
        uint32_t ad;
        if constexpr (PK == 2) {
            ad = __builtin_amdgcn_perm(w, lane4, 0x0c0c0000u | ((4u + (uint32_t)p) << 8));
        } else {
            const int b = 8 * (p & 3) + 4 * (p >> 2);
            ad = ((b >= 8 ? w >> (b - 8) : w << (8 - b)) & 0xF00u) | lane4;
        }
        return *reinterpret_cast<const uint32_t *>(tabb + ad);
    };
    if constexpr (PK != 0) {
#pragma unroll
        for (int s = 0; s < S; ++s) e_next[s] = pentry(rd[s][0], 0);
        for (int t0 = 0; t0 < nmax; t0 += KR) {
#pragma unroll
            for (int k = 0; k < KR; ++k) {
                const int t = t0 + k;
                uint32_t e[S];
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    e[s] = e_next[s];
                    if (k % TPD == TPD - 1) {
                        // Group k / TPD is used up: its slot takes the group RD ahead.
                        const int m = k / TPD;
                        rd[s][m] = __builtin_amdgcn_raw_buffer_load_b32(
                            srsrc, col * 4, (gb[s] + min(t0 / TPD + m + RD, gl[s])) * a.C * 4, 0);
                    }
                    e_next[s] = pentry(rd[s][((k + 1) / TPD) % RD], (k + 1) % TPD);
                }
#pragma unroll
                for (int s = 0; s < S; ++s)
                    if (t < n[s]) cd[s].step(e[s], stage, slot[s], lane);
            }
        }
    } else {
#pragma unroll
    for (int s = 0; s < S; ++s) {
        if (!TRUSTED) qmax = max(qmax, ring[s][0]);
        e_next[s] = entry(ring[s][0]);
    }
    for (int t0 = 0; t0 < nmax; t0 += kRing) {
#pragma unroll
        for (int k = 0; k < kRing; ++k) {
            const int t = t0 + k;
            uint32_t e[S];
#pragma unroll
            for (int s = 0; s < S; ++s) {
                e[s] = e_next[s];
                // Refill the slot just consumed with token t + kRing.
                const int last = max(n[s] - 1, 0);
                ring[s][k] = __builtin_amdgcn_raw_buffer_load_b8(srsrc, col, (row0[s] + min(t + kRing, last)) * a.C, 0);
                // Entry of token t + 1 (its symbol has been in the ring for a while).
                const uint32_t q = ring[s][(k + 1) % kRing];
                if (!TRUSTED) qmax = max(qmax, q);
                e_next[s] = entry(q);
            }
#pragma unroll
            for (int s = 0; s < S; ++s)
                if (t < n[s]) cd[s].step(e[s], stage, slot[s], lane);
        }
    }
    }

#pragma unroll
    for (int s = 0; s < S; ++s) {
        if (n[s] == 0) continue;
        const uint32_t len0 = cd[s].flush(stage, slot[s], lane);
        const uint32_t len = active ? len0 : 0u;
        const uint32_t incl = wave_incl_scan_u32(len, lane);
        const uint32_t total = (uint32_t)__shfl((int)incl, 63, 64);
        const uint32_t excl = incl - len;
        const uint8_t *lst = stage + (wv * S + s) * (R + 2) * kRowPitch;
        const bool ovf = __ballot(len > (uint32_t)kStageBytes) != 0;
        const bool gathered = total <= (uint32_t)(R * 64) && !ovf;
        if (gathered) {
            // Compact tile: gather the streams' bytes in stream order into
            // slot bytes [0, total) (64 consecutive bytes per store). Output
            // byte p belongs to the last stream k with excl_k <= p, found by a
            // binary search over the lanes' offsets; the spilled rows (>= R)
            // it may read lie beyond total. The fence orders the spill stores
            // of other lanes before these loads.
            // The loop is wave-uniform: the search reads other lanes' offsets.
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
            for (uint32_t p0 = 0; p0 < total; p0 += 64) {
                const uint32_t p = p0 + (uint32_t)lane;
                int k = 0;
                uint32_t sk = 0;
#pragma unroll
                for (int step = 32; step > 0; step >>= 1) {
                    const uint32_t sc = (uint32_t)__shfl((int)excl, k + step, 64);
                    if (sc <= p) {
                        k += step;
                        sk = sc;
                    }
                }
                if (p < total) {
                    const uint32_t i = p - sk;
                    uint32_t b;
                    if (i < (uint32_t)R) b = lst[(i + 1) * kRowPitch + k];
                    else b = __builtin_amdgcn_raw_buffer_load_b8(slot[s], (int)(i * 64 + k), 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b, slot[s], (int)p, 0, 0);
                }
            }
        } else {
            // Copy the used LDS rows 1.. to the slot's rows 0.. (64 lanes write
            // 256 contiguous bytes per store); k_compact gathers this tile.
            const uint32_t rows = min(wave_max_u32(len0), (uint32_t)R);
            const uint32_t *src = reinterpret_cast<const uint32_t *>(lst);
            for (uint32_t w = lane; w < rows * 16; w += 64)
                __builtin_amdgcn_raw_buffer_store_b32(src[((w >> 4) + 1) * (kRowPitch / 4) + (w & 15)], slot[s],
                                                      (int)(w * 4), 0, 0);
        }
        const int j = (g * NW + wv) * S + s;
        if (active) call_sec(a.lengths, a.cm, sl.b)[((int64_t)j * 2 * a.cm.Lc + sl.ls) * a.C + c] = (uint16_t)len;
        const int64_t tile = tile_index(j, slab, cb, a.L, a.CB);
        if (lane == 0) {
            a.tile_sum[tile] = total;
            a.tile_mode[tile] = gathered ? kTileGathered : ovf ? kTileOverflow : kTileRows;
        }
    }
    if (__ballot((active && (qmax > amax || bad))) && lane == 0) atomicOr(&a.hdr->status, kStCorrupt);
}

// ------------------------------------------------------------ chunk scan

struct ChunkScanArgs {
    const uint64_t *chunk_total;  // [NC * B], (chunk j, call b) at j * B + b
    uint64_t *chunk_off;          // call 0's
    uint64_t *size_dev;           // [B] or null
    uint8_t *header_size;         // call 0's, or null
    WsHeader *hdr;
    uint64_t payload_base;
    uint64_t cap;                 // each call's payload capacity
    int NC, B;
    CallMap cm;
};

// Pass 2: block b scans the chunk totals of call b into its chunk offsets
// and its size.
__global__ __launch_bounds__(1024) void k_chunk_scan(ChunkScanArgs a) {
    __shared__ uint64_t wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int b = blockIdx.x;
    uint64_t *chunk_off = call_sec(a.chunk_off, a.cm, b);
    uint64_t run = 0;
    for (int seg = 0; seg < a.NC; seg += 1024) {
        const int i = seg + tid;
        const uint64_t v = i < a.NC ? a.chunk_total[(int64_t)i * a.B + b] : 0ull;
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
        for (int k = 0; k < 16; ++k) {
            if (k < wv) before += wsum[k];
            total += wsum[k];
        }
        if (i < a.NC) chunk_off[i] = run + before + incl - v;
        run += total;
        __syncthreads();
    }
    if (tid == 0) {
        chunk_off[a.NC] = run;
        if (run > a.cap) atomicOr(&a.hdr->status, kStCapacity);
        const uint64_t size = a.payload_base + run;
        if (a.size_dev) a.size_dev[b] = size;
        if (a.header_size) {
            uint8_t *h = call_sec(a.header_size, a.cm, b);
            for (int i = 0; i < 8; ++i) h[i] = (uint8_t)(size >> (8 * i));
        }
    }
}

// ------------------------------------------------------------- compaction

struct CompactArgs {
    const uint8_t *staging;
    const uint16_t *lengths;
    const uint32_t *tile_sum;
    const uint8_t *tile_mode;
    const uint64_t *tile_off;   // relative to the chunk
    const uint64_t *chunk_off;
    uint8_t *payload;
    uint64_t cap;
    uint32_t *status;
    int64_t tiles;
    int L, C, CB;
    CallMap cm;
    // What the fix-up coder re-reads for an overflow tile.
    const uint8_t *sym;
    const int32_t *cdf;
    const uint16_t *cdf16;
    const uint32_t *wpre;
    int T, A;
    bool packed;   // symbols in the quantiser's packed layout
    bool nibbles;  // packed: slabs of at most 16 symbols as nibbles (PK 1), else bytes (PK 2)
    MaxTable mt;
};

// Fix-up of a tile with a stream longer than its staging slot: lane = stream
// re-encodes its symbols with the byte-at-a-time coder straight to the
// stream's final offset (base = the tile's).
__device__ void fixup_tile(const CompactArgs &a, int j, int slab, int cb, const SlabLoc &sl, uint64_t base,
                           int lane) {
    const int c = cb * 64 + lane;
    const bool active = c < a.C;
    const int n = min(kChunk, a.T - j * kChunk);
    const uint16_t *lengths = call_sec(a.lengths, a.cm, sl.b) + ((int64_t)j * 2 * a.cm.Lc + sl.ls) * a.C;
    const uint32_t len = active ? lengths[c] : 0u;
    const uint32_t incl = wave_incl_scan_u32(len, lane);
    if (!active) return;
    const int W = layer_w(a.mt, sl.kv, sl.l);
    const bool nib = a.nibbles && 2 * layer_m(a.mt, sl.kv, sl.l) + 1 <= 16;
    const uint16_t *cdf16 = call_sec(a.cdf16, a.cm, sl.b);
    const uint8_t *sp = a.sym + ((int64_t)slab * a.T + (int64_t)j * kChunk) * a.C + c;
    const uint8_t *slab_sym = a.sym + (int64_t)slab * a.T * a.C;
    RcEncHold enc;
    enc.init();
    GlobalSink sink{call_sec(a.payload, a.cm, sl.b), base + incl - len, a.cap, 0u, false};
    for (int t = 0; t < n; ++t) {
        uint32_t q;
        if (!a.packed) {
            q = sp[(int64_t)t * a.C];
        } else {
            const int tt = j * kChunk + t;
            if (nib) {
                const uint8_t b = slab_sym[((int64_t)(tt >> 3) * a.C + c) * 4 + (tt & 3)];
                q = (tt & 4) ? b >> 4 : b & 0xFu;
            } else {
                q = slab_sym[((int64_t)(tt >> 2) * a.C + c) * 4 + (tt & 3)];
            }
        }
        const uint32_t s = min(q, (uint32_t)W - 1);
        uint32_t lo, hi;
        cdf_bounds(a.cdf, cdf16, a.wpre, sl.ls, a.C, c, a.A, W, (int)s, lo, hi);
        const uint32_t f = hi > lo ? hi - lo : 1u;
        enc.encode(lo & 0xFFFFu, f, sink);
    }
    enc.flush(sink);
    if (sink.overflow) atomicOr(a.status, kStCapacity);
}

// One wave per tile. Every load a tile's copy depends on (its mode, byte
// count and offsets) is issued at once, so the copy waits for one round
// trip. Overflow tiles are re-encoded here by fixup_tile.
// LDS_ROWS: rows tiles are put in order in LDS (16 KiB per block) and leave
// as dwords; otherwise a byte at a time. The LDS costs residency, which a
// large grid needs (32K tokens: 2.31 vs 2.50 ms per call) and a small one
// does not (256 tokens: 120 vs 131 us).
template <bool LDS_ROWS>
__global__ __launch_bounds__(64) void k_compact(CompactArgs a) {
    const int lane = threadIdx.x;
    const int64_t tile = blockIdx.x;
    const int cb = (int)(tile % a.CB);
    const int64_t js = tile / a.CB;  // j * 2L + slab
    const int slab = (int)(js % (2 * a.L)), j = (int)(js / (2 * a.L));
    const SlabLoc sl = slab_loc(a.cm, slab);
    const uint32_t mode = a.tile_mode[tile];
    const uint32_t total = a.tile_sum[tile];
    const uint64_t base = call_sec(a.chunk_off, a.cm, sl.b)[j] + a.tile_off[tile];
    if (mode == kTileOverflow) {
        fixup_tile(a, j, slab, cb, sl, base, lane);
        return;
    }
    uint8_t *payload = call_sec(a.payload, a.cm, sl.b);
    const bool gathered = mode == kTileGathered;
    const uint8_t *src = a.staging + tile * (kStageBytes * 64);
    bool over = base + total > a.cap;
    if (gathered && !over && ((uintptr_t)payload & 3u) == 0) {
        // The encoder left the tile's bytes contiguous: copy them, whole
        // destination dwords by dword stores (each assembled from the two
        // aligned source dwords it straddles; the slot is 16 KiB aligned and
        // far longer than the tile, so the second read stays inside it), and
        // the at most three bytes at either end, which share their dwords
        // with the neighbouring tiles, by byte stores.
        const uint64_t end = base + total;
        const uint64_t wa = (base + 3) & ~3ull, we = end & ~3ull;
        const uint32_t *s32 = reinterpret_cast<const uint32_t *>(src);
        if (wa >= we) {
            if ((uint32_t)lane < total) payload[base + lane] = src[lane];
        } else {
            const uint32_t nhead = (uint32_t)(wa - base), ntail = (uint32_t)(end - we);
            if ((uint32_t)lane < nhead) payload[base + lane] = src[lane];
            if ((uint32_t)lane < ntail) payload[we + lane] = src[(uint32_t)(we - base) + lane];
            uint32_t *d32 = reinterpret_cast<uint32_t *>(payload + wa);
            const uint32_t nw = (uint32_t)((we - wa) >> 2);
            const uint32_t sh = nhead & 3u;  // source byte offset of every word
            constexpr int U = 12;            // words per lane in one round trip (a gathered tile has <= 2816 bytes)
            if (nw <= U * 64) {
                // Every load first, then every store: one round trip.
                uint32_t v0[U], v1[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t w = (uint32_t)lane + 64u * u;
                    const uint32_t si = (nhead >> 2) + w;  // aligned source word below the word's first byte
                    v0[u] = v1[u] = 0;
                    if (w < nw) {
                        v0[u] = s32[si];
                        v1[u] = s32[si + 1];
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t w = (uint32_t)lane + 64u * u;
                    if (w < nw) d32[w] = __builtin_amdgcn_alignbyte(v1[u], v0[u], sh);
                }
            } else {
                for (uint32_t w = lane; w < nw; w += 64) {
                    const uint32_t so = nhead + 4 * w;  // source byte of the word
                    d32[w] = __builtin_amdgcn_alignbyte(s32[(so >> 2) + 1], s32[so >> 2], sh);
                }
            }
        }
    } else if (gathered) {
        // The same copy a byte at a time (capacity overflow, unaligned payload).
        uint32_t p = lane;
        for (; p + 192 < total; p += 256) {
            uint32_t b[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) b[u] = src[p + 64 * u];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (base + p + 64 * u < a.cap) payload[base + p + 64 * u] = (uint8_t)b[u];
        }
        for (; p < total; p += 64)
            if (base + p < a.cap) payload[base + p] = src[p];
    } else if (LDS_ROWS && !over && ((uintptr_t)payload & 3u) == 0) {
        // [byte][lane] rows: byte i of stream k at slot byte i * 64 + k (no
        // stream is longer than the slot's 256 rows, or the tile would be an
        // overflow tile). Lane l reads the dwords of rows l / 16 + 4m, each
        // holding byte i of streams 4q .. 4q + 3 (q = l % 16), all of a group
        // of rows in one round trip, and puts every byte at its place in the
        // tile in LDS, offset by base % 4 so that the payload's aligned
        // dwords are aligned LDS words; the wave then stores those dwords
        // (and the bytes at either end) as the gathered copy does.
        __shared__ uint32_t gat_w[LDS_ROWS ? (kStageBytes * 64 + 8) / 4 : 1];
        uint8_t *gat = reinterpret_cast<uint8_t *>(gat_w);
        const int c = cb * 64 + lane;
        const uint16_t *lengths = call_sec(a.lengths, a.cm, sl.b) + ((int64_t)j * 2 * a.cm.Lc + sl.ls) * a.C;
        const uint32_t len = c < a.C ? lengths[c] : 0u;
        const uint32_t excl = wave_incl_scan_u32(len, lane) - len;
        const uint32_t rows = wave_max_u32(len);
        const uint32_t h = (uint32_t)(base & 3u);
        const int q = lane & 15, r0 = lane >> 4;
        uint32_t qlen[4], qoff[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            qlen[cc] = (uint32_t)__shfl((int)len, 4 * q + cc, 64);
            qoff[cc] = (uint32_t)__shfl((int)excl, 4 * q + cc, 64) + h;
        }
        // Rows are read through a buffer over the slot; past its 256 rows a
        // read returns 0 (and its bytes are not used).
        const __amdgpu_buffer_rsrc_t srsrc = make_rsrc(src, kStageBytes * 64);
        constexpr int U = 16;  // rows per lane per round trip (64 rows per wave)
        for (uint32_t i0 = 0; i0 < rows; i0 += 4 * U) {
            uint32_t v[U];
            const int voff = (int)(((i0 + (uint32_t)r0) * 16 + (uint32_t)q) * 4);
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b32(srsrc, voff + 256 * u, 0, 0);
            const uint32_t ir = i0 + (uint32_t)r0;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                uint8_t *g = gat + qoff[cc] + ir;  // row u's byte at g[4u]
                const uint32_t left = qlen[cc] > ir ? qlen[cc] - ir : 0u;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (4u * u < left) g[4 * u] = (uint8_t)(v[u] >> (8 * cc));
            }
        }
        __syncthreads();
        const uint64_t end = base + total;
        const uint64_t wa = (base + 3) & ~3ull, we = end & ~3ull;
        if (wa >= we) {
            if ((uint32_t)lane < total) payload[base + lane] = gat[h + lane];
        } else {
            const uint32_t nhead = (uint32_t)(wa - base), ntail = (uint32_t)(end - we);
            if ((uint32_t)lane < nhead) payload[base + lane] = gat[h + lane];
            if ((uint32_t)lane < ntail) payload[we + lane] = gat[h + (uint32_t)(we - base) + lane];
            uint32_t *d32 = reinterpret_cast<uint32_t *>(payload + wa);
            const uint32_t nw = (uint32_t)((we - wa) >> 2), w0 = (h + nhead) >> 2;
            for (uint32_t w = lane; w < nw; w += 64) d32[w] = gat_w[w0 + w];
        }
    } else {
        // [byte][lane] rows, a byte at a time (capacity overflow, unaligned
        // payload): output byte p belongs to the last stream k with excl_k <=
        // p (binary search over the lanes' offsets; the loop is wave-uniform
        // because the search reads other lanes).
        const int c = cb * 64 + lane;
        const uint16_t *lengths = call_sec(a.lengths, a.cm, sl.b) + ((int64_t)j * 2 * a.cm.Lc + sl.ls) * a.C;
        const uint32_t len = c < a.C ? lengths[c] : 0u;
        const uint32_t excl = wave_incl_scan_u32(len, lane) - len;
        for (uint32_t p0 = 0; p0 < total; p0 += 64) {
            const uint32_t p = p0 + (uint32_t)lane;
            int k = 0;
            uint32_t sk = 0;
#pragma unroll
            for (int step = 32; step > 0; step >>= 1) {
                const uint32_t sc = (uint32_t)__shfl((int)excl, k + step, 64);
                if (sc <= p) {
                    k += step;
                    sk = sc;
                }
            }
            if (p < total && base + p < a.cap) payload[base + p] = src[(p - sk) * 64 + k];
        }
    }
    if (__ballot(over) && lane == 0) atomicOr(a.status, kStCapacity);
}

// ---------------------------------------------------------------- launch

size_t encode_staging_bytes(const Dims &d) { return (size_t)d.tiles * kStageBytes * 64; }

// Grids of compaction blocks up to which rows tiles are ordered in LDS
// (k_compact's LDS_ROWS): sixteen per CU.
constexpr int64_t kCompactLdsTiles = 16 * 256;

constexpr int64_t kEncOneChunkWaves = 4 * 1024;
constexpr int64_t kEncOneChunkWaves4 = 256 * 256;

// Launch shape of k_encode: S chunks per lane, NW waves per block, and
// whether the call has slabs of at most 16 symbols (small) and others (large).
struct EncPlan {
    int S, NW, loga;
    unsigned blocks;
    bool small, large;
};

static EncPlan enc_plan(const Dims &d, const MaxTable &mt) {
    EncPlan p;
    p.S = d.NC >= 2 ? 2 : 1;
    // Four waves per block share a table when there are enough chunks.
    p.NW = d.NC >= 8 ? 4 : 1;
    // A grid of at most four one-chunk waves per SIMD (a call of a few
    // chunks) codes one chunk per lane: with the SIMD nearly to itself a
    // wave's time is its chain's latency, and two chains interleaved in one
    // wave take almost twice one (768 tokens of 32 x 1024 channels: 106 us
    // for the two-chunk launch against 57 for a one-chunk call's). Four-wave
    // blocks do the same up to 256 one-chunk waves per CU: a few rounds of
    // blocks, whose tail the smaller one-chunk blocks shorten (GLM-4-9B shape
    // at 16K tokens, 80 per CU: 0.53 -> 0.51 ms; the 32K-token call, 512
    // per CU, keeps two chunks per lane but in its wider launch).
    if (p.NW == 1 && (int64_t)d.NC * 2 * d.L * d.CB <= kEncOneChunkWaves) p.S = 1;
    if (p.NW == 4 && (int64_t)d.NC * 2 * d.L * d.CB <= kEncOneChunkWaves4) p.S = 1;
    const int ngroups = (d.NC + p.S * p.NW - 1) / (p.S * p.NW);
    p.blocks = (unsigned)((int64_t)ngroups * 2 * d.L * d.CB);
    p.loga = 4;
    while ((1 << p.loga) < d.A) ++p.loga;
    p.small = p.large = false;
    for (int kv = 0; kv < 2; ++kv)
        for (int l = 0; l < d.Lc; ++l) (2 * (mt.bins[kv][l] / 2 - 1) + 1 <= 16 ? p.small : p.large) = true;
    return p;
}

// Slabs of both kinds share a launch only for small grids; otherwise every
// trusted launch sees one kind, so one packed layout.
static bool enc_split(const EncPlan &p) { return p.loga > 4 && p.small && (!p.large || p.blocks >= 16384); }

// A launch that sees both kinds of slabs (a small grid) reads bytes for all
// of them; nibbles need a launch of 16-entry tables.
bool encode_packs(const Dims &d, const MaxTable &) { return d.T % 8 == 0; }

bool encode_nibbles(const Dims &d, const MaxTable &mt) {
    const EncPlan p = enc_plan(d, mt);
    return enc_split(p) || p.loga <= 4;
}

hipError_t launch_encode(const Dims &d, const MaxTable &mt, const uint8_t *sym, const int32_t *cdf,
                         const uint16_t *cdf16, const uint32_t *wpre, const EncodeOut &o, const EncodeWs &w,
                         bool trusted, bool packed, hipStream_t s) {
    const EncPlan plan = enc_plan(d, mt);
    if (packed && (!trusted || !encode_packs(d, mt))) return hipErrorInvalidValue;
    const int S = plan.S;
    EncArgs a;
    a.sym = sym;
    a.cdf = cdf;
    a.cdf16 = cdf16;
    a.wpre = wpre;
    a.mt = mt;
    a.staging = w.staging;
    a.tile_sum = w.tile_sum;
    a.tile_mode = w.tile_mode;
    a.lengths = o.lengths;
    a.hdr = w.hdr;
    a.L = d.L;
    a.T = d.T;
    a.C = d.C;
    a.A = d.A;
    a.NC = d.NC;
    a.CB = d.CB;
    a.cm = call_map(d);
    const int NW = plan.NW;
    const unsigned blocks = plan.blocks;
    dim3 grid(blocks);
    const dim3 block(64 * NW);
    const int loga = plan.loga;
    // Packed symbols: nibbles in a launch of 16-entry tables (slabs of at
    // most 16 symbols), bytes in a wider one (whose slabs may be of both
    // kinds).
#define CG_ENC(SS, LG, W)                                                                           \
    do {                                                                                            \
        if (!trusted) hipLaunchKernelGGL((k_encode<SS, LG, W, false, 0>), grid, block, 0, s, a);    \
        else if (!packed) hipLaunchKernelGGL((k_encode<SS, LG, W, true, 0>), grid, block, 0, s, a); \
        else hipLaunchKernelGGL((k_encode<SS, LG, W, true, (LG <= 4 ? 1 : 2)>), grid, block, 0, s, a); \
    } while (0)
#define CG_ENC_A(SS, W, LOGA_)                    \
    do {                                          \
        if (LOGA_ <= 4) CG_ENC(SS, 4, W);         \
        else if (LOGA_ == 5) CG_ENC(SS, 5, W);    \
        else if (LOGA_ == 6) CG_ENC(SS, 6, W);    \
        else CG_ENC(SS, 7, W);                    \
    } while (0)
    // wide1: the wider launch of a split with four-wave blocks codes one
    // chunk per lane, in twice the blocks: its 32-entry tables and 44-row
    // stages fit five two-chunk blocks per CU but eight one-chunk blocks,
    // and its few slabs (12 of 64 on the benchmark call) leave the chip
    // half idle in the tail of a two-chunk launch (2.38 -> 2.31 ms per
    // call; one chunk per lane in the 16-entry launch too, or a 60-row
    // stage, measured slower).
    auto launch = [&](int lg, bool wide1) {
        if (NW == 4 && wide1) {
            grid.x = (unsigned)((int64_t)((d.NC + 3) / 4) * 2 * d.L * d.CB);
            CG_ENC_A(1, 4, lg);
            grid.x = blocks;
        } else if (NW == 4) {
            if (S == 2) CG_ENC_A(2, 4, lg);
            else CG_ENC_A(1, 4, lg);
        } else if (S == 2) {
            CG_ENC_A(2, 1, lg);
        } else {
            CG_ENC_A(1, 1, lg);
        }
        return hipGetLastError();
    };
    // The quantiser's symbols of a slab stay below 2M + 1, so with trusted
    // symbols the slabs of at most 16 symbols (16-bin layers) take a launch
    // with 16-entry tables, whose blocks need half the LDS and fit the CU
    // more densely; the other slabs take the full width.
    const bool large = plan.large;
    hipError_t e;
    // Only worth a second launch when the grid is large (big calls, batches).
    if (trusted && enc_split(plan)) {
        a.nsym_lo = 0;
        a.nsym_hi = 16;
        if ((e = launch(4, false)) != hipSuccess) return e;
        if (large) {
            a.nsym_lo = 17;
            a.nsym_hi = 1 << 30;
            if ((e = launch(loga, true)) != hipSuccess) return e;
        }
    } else {
        a.nsym_lo = 0;
        a.nsym_hi = 1 << 30;
        if ((e = launch(loga, false)) != hipSuccess) return e;
    }
#undef CG_ENC_A
#undef CG_ENC

    TileScan ts{w.tile_sum, nullptr, w.tile_off, w.scan_tmp, w.chunk_total, nullptr, 0, nullptr, 0,
                &w.hdr->status, d.L, d.C, d.CB, d.NC, call_map(d)};
    if (call_scan_fits(ts)) {
        ChunkOut co;
        co.chunk_off = o.chunk_off;
        co.size_dev = o.size_dev;
        co.header_size = o.header_size;
        co.payload_base = o.payload_base;
        co.cap = o.cap;
        if ((e = launch_call_scan(ts, &co, s)) != hipSuccess) return e;
    } else {
        if ((e = launch_tile_scan(ts, s)) != hipSuccess) return e;
        ChunkScanArgs sa;
        sa.chunk_total = w.chunk_total;
        sa.chunk_off = o.chunk_off;
        sa.size_dev = o.size_dev;
        sa.header_size = o.header_size;
        sa.hdr = w.hdr;
        sa.payload_base = o.payload_base;
        sa.cap = o.cap;
        sa.NC = d.NC;
        sa.B = ncalls(d);
        sa.cm = call_map(d);
        hipLaunchKernelGGL(k_chunk_scan, dim3((unsigned)sa.B), dim3(1024), 0, s, sa);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    CompactArgs ca;
    ca.staging = w.staging;
    ca.lengths = o.lengths;
    ca.tile_sum = w.tile_sum;
    ca.tile_mode = w.tile_mode;
    ca.tile_off = w.tile_off;
    ca.chunk_off = o.chunk_off;
    ca.payload = o.payload;
    ca.cap = o.cap;
    ca.status = &w.hdr->status;
    ca.tiles = d.tiles;
    ca.L = d.L;
    ca.C = d.C;
    ca.CB = d.CB;
    ca.cm = call_map(d);
    ca.sym = sym;
    ca.cdf = cdf;
    ca.cdf16 = cdf16;
    ca.wpre = wpre;
    ca.T = d.T;
    ca.A = d.A;
    ca.packed = packed;
    ca.nibbles = packed && encode_nibbles(d, mt);
    ca.mt = mt;
    if (d.tiles <= kCompactLdsTiles) hipLaunchKernelGGL(k_compact<true>, dim3((unsigned)d.tiles), dim3(64), 0, s, ca);
    else hipLaunchKernelGGL(k_compact<false>, dim3((unsigned)d.tiles), dim3(64), 0, s, ca);
    return hipGetLastError();
}

}  // namespace cg
