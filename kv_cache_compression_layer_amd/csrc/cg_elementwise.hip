// Element-wise kernels of the CacheGen codec on gfx950: quantise, dequantise,
// workspace fills and the blob header.
//
// Quantisation follows the LMCache CacheGen page (0539edu.com/news/4720135),
// section 2: a symmetric per-layer quantiser whose scale is the absolute
// maximum over the channels of a (K|V, layer, token) row. Dequantisation
// follows section 5: t = (t - M) / M * scale, cast back to bf16.
//
// One wave owns one row of C channels: its loads are 16-byte vectors that
// cover the row contiguously (64 lanes x 16 B = 1 KiB per instruction), the
// absmax is a max over bf16 bit patterns (|x| orders like its bit pattern
// with the sign cleared) reduced across the wave, and the row stays in
// registers between the reduction and the quantisation.
#include "cg_internal.hpp"

namespace cg {

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t *__restrict__ p, uint32_t v, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

hipError_t launch_fill_u32(uint32_t *p, uint32_t v, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, s, p, v, n);
    return hipGetLastError();
}

// --------------------------------------------------------------- quantise

// Symbol of one element: q = round_half_even(x*f + M) with every fp32
// operation rounded on its own (the library is built without contraction).
// Adding 1.5 * 2^23 to a value in [-0.5, 2^22) rounds it to an integer (half
// to even) and leaves that integer in the low mantissa bits, so the symbol is
// the low byte of the sum. The clamp to [0, 2M] of the definition is a no-op
// here: |x| <= m gives |x*f| <= M(1 + 2^-23), so x*f + M lies within
// [-M*2^-23, 2M + M*2^-23] and rounds into [0, 2M].
__device__ __forceinline__ uint32_t quant_bits(float x, float f, float Mf) {
    const float y = __fmul_rn(x, f);
    const float z = __fadd_rn(y, Mf);
    return __float_as_uint(__fadd_rn(z, 12582912.0f));  // low byte = symbol
}

// Four bf16 values packed in two words -> four symbol bytes in one word.
__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, float f, float Mf) {
    const uint32_t a = quant_bits(__uint_as_float(w0 << 16), f, Mf);
    const uint32_t b = quant_bits(__uint_as_float(w0 & 0xFFFF0000u), f, Mf);
    const uint32_t c = quant_bits(__uint_as_float(w1 << 16), f, Mf);
    const uint32_t d = quant_bits(__uint_as_float(w1 & 0xFFFF0000u), f, Mf);
    // Byte 0 of each: perm selects bytes of {src0, src1} (src1 = bytes 0..3).
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // [a0, b0, 0, 0]
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x04000c0cu);  // [0, 0, c0, d0]
    return ab | cd;
}

__device__ __forceinline__ uint32_t quant1(uint32_t bits16, float f, float Mf) {
    return quant_bits(bf16_to_f32(bits16 & 0xFFFFu), f, Mf) & 0xFFu;
}

// Factor M/m of a row whose absmax has bits am (sign cleared), uniform across
// the wave. 0 for an all-zero row, so every symbol is M. A row whose factor
// overflows fp32 (an absmax below about M * 2^-128, so below 2^-122 for any
// bins) has no finite factor; it is quantised as an all-zero row too, and am
// becomes 0, the scale stored for it. Non-finite input (am >= 0x7F80) gives
// 0; the caller reports it.
__device__ __forceinline__ float row_factor(uint32_t &am, float Mf) {
    if (am == 0 || am >= 0x7F80u) return 0.0f;
    const float f = __fdiv_rn(Mf, bf16_to_f32(am));
    if (__float_as_uint(f) == 0x7F800000u) {
        am = 0;
        return 0.0f;
    }
    return f;
}

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

// Maximum over the wave, returned in a scalar register: DPP shifts within
// each row of 16 lanes (max is idempotent, so overlapping windows are fine),
// then the four row maxima by readlane.
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
    return max(max(r0, r1), max(r2, r3));
}

// Per-half max of |bf16| bit patterns (sign cleared) with packed 16-bit max.
__device__ __forceinline__ uint32_t absmax2(uint32_t acc, uint32_t w) {
    ushort2_t a = __builtin_bit_cast(ushort2_t, acc);
    ushort2_t b = __builtin_bit_cast(ushort2_t, w & 0x7FFF7FFFu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// NV 16-byte vectors per lane hold the row (C <= NV * 512, C % 8 == 0;
// FULL: C == NV * 512, so no lane is idle).
template <int NV, bool FULL>
__global__ __launch_bounds__(256) void k_quantize_vec(const uint16_t *__restrict__ kv,
                                                      uint8_t *__restrict__ sym,
                                                      uint16_t *__restrict__ scale,
                                                      uint32_t *__restrict__ status, int T,
                                                      int C, MaxTable mt, CallMap cm) {
    const int lane = threadIdx.x & 63;
    // The row is uniform across the wave; readfirstlane lets the compiler
    // keep the row arithmetic in scalar registers.
    const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (t >= T) return;
    const int slab = blockIdx.y;  // grid: (tokens/4, 2L)
    const SlabLoc sl = slab_loc(cm, slab);
    const int64_t row = (int64_t)slab * T + t;
    const uint16_t *src = kv + (((int64_t)sl.lv * 2 + sl.kv) * T + t) * C;
    uint8_t *dst = sym + row * C;

    uint4 v[NV];
    uint32_t am2 = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c0 = (i * 64 + lane) * 8;
        if (FULL || c0 < C) {
            v[i] = *reinterpret_cast<const uint4 *>(src + c0);
        } else {
            v[i] = make_uint4(0, 0, 0, 0);
        }
        am2 = absmax2(absmax2(absmax2(absmax2(am2, v[i].x), v[i].y), v[i].z), v[i].w);
    }
    uint32_t am = max(am2 & 0xFFFFu, am2 >> 16);
    am = wave_max_dpp(am);
    if (am >= 0x7F80u && lane == 0) atomicOr(status, kStNonfinite);
    const int M = layer_m(mt, sl.kv, sl.l);
    const float Mf = (float)M;
    // m == 0 gives f == 0, so every symbol is exactly M.
    const float f = row_factor(am, Mf);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c0 = (i * 64 + lane) * 8;
        if (FULL || c0 < C) {
            const uint32_t lo = quant4(v[i].x, v[i].y, f, Mf);
            const uint32_t hi = quant4(v[i].z, v[i].w, f, Mf);
            *reinterpret_cast<uint2 *>(dst + c0) = make_uint2(lo, hi);
        }
    }
    if (lane == 0) call_sec(scale, cm, sl.b)[(int64_t)sl.ls * T + t] = (uint16_t)am;
}

// Any C and alignment: two passes over the row (the second hits the cache).
__global__ __launch_bounds__(256) void k_quantize_any(const uint16_t *__restrict__ kv,
                                                      uint8_t *__restrict__ sym,
                                                      uint16_t *__restrict__ scale,
                                                      uint32_t *__restrict__ status, int T,
                                                      int C, MaxTable mt, CallMap cm) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int slab = blockIdx.y;  // grid: (tokens/4, 2L)
    const SlabLoc sl = slab_loc(cm, slab);
    const int64_t row = (int64_t)slab * T + t;
    const uint16_t *src = kv + (((int64_t)sl.lv * 2 + sl.kv) * T + t) * C;
    uint8_t *dst = sym + row * C;
    uint32_t am = 0;
    for (int c = lane; c < C; c += 64) am = max(am, (uint32_t)src[c] & 0x7FFFu);
    am = wave_max_u32(am);
    if (am >= 0x7F80u && lane == 0) atomicOr(status, kStNonfinite);
    const int M = layer_m(mt, sl.kv, sl.l);
    const float Mf = (float)M;
    const float f = row_factor(am, Mf);
    for (int c = lane; c < C; c += 64) dst[c] = (uint8_t)quant1(src[c], f, Mf);
    if (lane == 0) call_sec(scale, cm, sl.b)[(int64_t)sl.ls * T + t] = (uint16_t)am;
}

hipError_t launch_quantize(const Dims &d, const MaxTable &mt, const uint16_t *kv, uint8_t *sym,
                           uint16_t *scale, uint32_t *status, hipStream_t s) {
    const dim3 grid((unsigned)((d.T + 3) / 4), (unsigned)(2 * d.L)), block(256);
    const bool aligned = ((uintptr_t)kv % 16 == 0) && ((uintptr_t)sym % 8 == 0);
    if (aligned && d.C % 8 == 0 && d.C <= 2048) {
        const int nv = (d.C + 511) / 512;
        const bool full = d.C == nv * 512;
    const CallMap cm = call_map(d);
#define CG_QV(N)                                                                                      \
    if (full) hipLaunchKernelGGL((k_quantize_vec<N, true>), grid, block, 0, s, kv, sym, scale, status, d.T, d.C, mt, cm); \
    else hipLaunchKernelGGL((k_quantize_vec<N, false>), grid, block, 0, s, kv, sym, scale, status, d.T, d.C, mt, cm);
        switch (nv) {
        case 1: CG_QV(1) break;
        case 2: CG_QV(2) break;
        case 3: CG_QV(3) break;
        default: CG_QV(4) break;
        }
#undef CG_QV
    } else {
        hipLaunchKernelGGL(k_quantize_any, grid, block, 0, s, kv, sym, scale, status, d.T, d.C, mt, call_map(d));
    }
    return hipGetLastError();
}

// ------------------------------------------------- quantise + histogram

// The to_bytes path quantises and counts in one pass, so the symbols are
// not read back for the histogram. A block of NT / 64 waves (8, or 16 when
// the grid has fewer blocks than the chip has CUs) owns a tile of TT rows
// (tokens) of one (K|V, layer); each wave quantises four rows at a time
// exactly as k_quantize_vec does. Lane l always holds the same CW*NV channels
// ((i*64 + l)*CW + e), so the block keeps lane-column counters in LDS,
// uint32 [symbol][pair][lane] with the counts of channels e and e+1 of a
// pair in the low and high halves (TT <= 65535 keeps them in 16 bits); all
// lanes of an instruction hit distinct banks. Counts are added to the global
// uint32 [2,L,C,A] table at the end (non-zero entries only). Symbols are
// below A by construction.
//
// PACK: the symbols are written for the encoder in token groups instead of
// [T][C] rows (T % 8 == 0). With `nibbles`, a slab whose symbols fit four
// bits (2M + 1 <= 16) holds one dword per (8-token group g, channel c) at
// byte (g*C + c)*4, byte j of which carries token 8g + j in its low nibble
// and token 8g + 4 + j in its high nibble; the other slabs (all of them
// without `nibbles`) hold one dword per (4-token group, c), byte j = token
// 4g + j. Each wave then quantises 8 consecutive rows per group and
// assembles the dwords in registers.
//
// CW: channels per lane and load (8: 16-byte loads, C = 512 or 1024; 4:
// 8-byte loads, C = 256 or 768); a lane holds channels (i*64 + lane)*CW + e,
// i < NV, e < CW.
template <int NV, int CW, int LOGA, bool PACK, int NT>
__global__ __launch_bounds__(NT) void k_quantize_hist(const uint16_t *__restrict__ kv,
                                                       uint8_t *__restrict__ sym,
                                                       uint16_t *__restrict__ scale,
                                                       uint32_t *__restrict__ counts,
                                                       uint16_t *__restrict__ wire,
                                                       const uint32_t *__restrict__ wpre,
                                                       uint32_t *__restrict__ status, int T,
                                                       int C, int A, int TT, MaxTable mt, CallMap cm,
                                                       bool nibbles) {
    constexpr int NS = 1 << LOGA;
    constexpr int NWV = NT / 64;     // waves per block
    constexpr int NWD = CW / 2;      // 32-bit words (two bf16) per load
    constexpr int NP = NV * NWD;     // channel pairs per lane
    __shared__ __attribute__((aligned(16))) uint32_t hist[NS * NP * 64];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int slab = blockIdx.y;
    const SlabLoc sl = slab_loc(cm, slab);
    const int t0 = blockIdx.x * TT, t1 = min(T, t0 + TT);
    uint4 *h4 = reinterpret_cast<uint4 *>(hist);
    for (int i = threadIdx.x; i < NS * NP * 64 / 4; i += NT) h4[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();

    const int M = layer_m(mt, sl.kv, sl.l);
    const float Mf = (float)M;
    uint8_t *hb = reinterpret_cast<uint8_t *>(hist);
    const uint32_t lane4 = (uint32_t)lane * 4;
    const uint16_t *kv_slab = kv + ((int64_t)sl.lv * 2 + sl.kv) * T * (int64_t)C;
    uint8_t *sym_slab = sym + (int64_t)slab * T * (int64_t)C;
    uint16_t *scale_slab = call_sec(scale, cm, sl.b) + (int64_t)sl.ls * T;

    auto count = [&](uint32_t bits, int pair, bool odd) {
        const uint32_t q = __builtin_amdgcn_ubfe(bits, 0, LOGA);
        uint32_t *cnt = reinterpret_cast<uint32_t *>(hb + q * (NP * 256) + lane4 + pair * 256);
        __hip_atomic_fetch_add(cnt, odd ? 0x10000u : 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto load_row = [&](int t, uint32_t (&v)[NV][NWD]) {
        const uint16_t *src = kv_slab + (int64_t)t * C;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if constexpr (CW == 8) {
                const uint4 x = *reinterpret_cast<const uint4 *>(src + (i * 64 + lane) * 8);
                v[i][0] = x.x;
                v[i][1] = x.y;
                v[i][2] = x.z;
                v[i][3] = x.w;
            } else {
                const uint2 x = *reinterpret_cast<const uint2 *>(src + (i * 64 + lane) * 4);
                v[i][0] = x.x;
                v[i][1] = x.y;
            }
        }
    };
    // Packed: pw[h][i*CW + e] collects rows 4h..4h+3 of the current 8-row
    // group for channel (i*64 + lane)*CW + e, one byte per row.
    uint32_t pw[2][NV * CW];
    // gr: the row's place in its 8-row group (packed only; a constant after
    // unrolling, so the word and byte it fills are fixed at compile time).
    auto do_row = [&](int t, const uint32_t (&v)[NV][NWD], int gr) {
        uint32_t am2 = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int j = 0; j < NWD; ++j) am2 = absmax2(am2, v[i][j]);
        uint32_t am = wave_max_dpp(max(am2 & 0xFFFFu, am2 >> 16));
        if (am >= 0x7F80u && lane == 0) atomicOr(status, kStNonfinite);
        const float f = row_factor(am, Mf);
        uint8_t *dst = sym_slab + (int64_t)t * C;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            uint32_t qb[CW];
#pragma unroll
            for (int j = 0; j < NWD; ++j) {
                qb[2 * j] = quant_bits(__uint_as_float(v[i][j] << 16), f, Mf);
                qb[2 * j + 1] = quant_bits(__uint_as_float(v[i][j] & 0xFFFF0000u), f, Mf);
            }
            if constexpr (PACK) {
                // Byte gr % 4 of the channel's dword takes this row's symbol
                // (perm: selector 4 = byte 0 of qb, 0..3 = bytes of pw).
                const int h = gr >> 2, r = gr & 3;
                const uint32_t sel = (0x03020100u & ~(0xFFu << (8 * r))) | (4u << (8 * r));
#pragma unroll
                for (int e = 0; e < CW; ++e) {
                    pw[h][i * CW + e] = __builtin_amdgcn_perm(qb[e], pw[h][i * CW + e], sel);
                    // Pin the word: otherwise the four permutes of a word are
                    // recombined after the last row, holding every row's
                    // symbols in registers until then.
                    __asm__ volatile("" : "+v"(pw[h][i * CW + e]));
                }
            } else {
                const uint32_t lo = __builtin_amdgcn_perm(qb[1], qb[0], 0x0c0c0400u) |
                                    __builtin_amdgcn_perm(qb[3], qb[2], 0x04000c0cu);
                if constexpr (CW == 8) {
                    const uint32_t hi = __builtin_amdgcn_perm(qb[5], qb[4], 0x0c0c0400u) |
                                        __builtin_amdgcn_perm(qb[7], qb[6], 0x04000c0cu);
                    *reinterpret_cast<uint2 *>(dst + (i * 64 + lane) * 8) = make_uint2(lo, hi);
                } else {
                    *reinterpret_cast<uint32_t *>(dst + (i * 64 + lane) * 4) = lo;
                }
            }
#pragma unroll
            for (int e = 0; e < CW; ++e) count(qb[e], i * NWD + e / 2, (e & 1) != 0);
        }
        if (lane == 0) scale_slab[t] = (uint16_t)am;
    };

    if constexpr (PACK) {
        // Wave wv takes the 8-row groups t0 + 8*(wv + NWV k) (t0 and t1 are
        // multiples of 8).
        const bool nib = nibbles && 2 * M + 1 <= 16;
#pragma unroll
        for (int e = 0; e < NV * CW; ++e) pw[0][e] = pw[1][e] = 0;  // every byte is overwritten per group
        for (int g0 = t0 + 8 * wv; g0 < t1; g0 += 8 * NWV) {
            // Four rows in flight at a time.
#pragma unroll
            for (int r = 0; r < 8; r += 4) {
                uint32_t va[NV][NWD], vb[NV][NWD], vc[NV][NWD], vd[NV][NWD];
                load_row(g0 + r, va);
                load_row(g0 + r + 1, vb);
                load_row(g0 + r + 2, vc);
                load_row(g0 + r + 3, vd);
                do_row(g0 + r, va, r);
                do_row(g0 + r + 1, vb, r + 1);
                do_row(g0 + r + 2, vc, r + 2);
                do_row(g0 + r + 3, vd, r + 3);
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                // Channels (i*64 + lane)*CW .. +CW: 4*CW contiguous bytes per group row.
                const int64_t col = (int64_t)(i * 64 + lane) * CW;
                if (nib) {
                    uint32_t w[CW];
#pragma unroll
                    for (int e = 0; e < CW; ++e) w[e] = pw[0][i * CW + e] | (pw[1][i * CW + e] << 4);
                    uint4 *d4 = reinterpret_cast<uint4 *>(sym_slab + ((int64_t)(g0 >> 3) * C + col) * 4);
#pragma unroll
                    for (int u = 0; u < CW / 4; ++u) d4[u] = make_uint4(w[4 * u], w[4 * u + 1], w[4 * u + 2], w[4 * u + 3]);
                } else {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        uint4 *d4 = reinterpret_cast<uint4 *>(sym_slab + ((int64_t)((g0 >> 2) + h) * C + col) * 4);
#pragma unroll
                        for (int u = 0; u < CW / 4; ++u)
                            d4[u] = make_uint4(pw[h][i * CW + 4 * u], pw[h][i * CW + 4 * u + 1],
                                               pw[h][i * CW + 4 * u + 2], pw[h][i * CW + 4 * u + 3]);
                    }
                }
            }
        }
    } else {
        // Wave wv takes rows t0 + wv + NWV k, four in flight at a time.
        int t = t0 + wv;
        for (; t + 3 * NWV < t1; t += 4 * NWV) {
            uint32_t va[NV][NWD], vb[NV][NWD], vc[NV][NWD], vd[NV][NWD];
            load_row(t, va);
            load_row(t + NWV, vb);
            load_row(t + 2 * NWV, vc);
            load_row(t + 3 * NWV, vd);
            do_row(t, va, 0);
            do_row(t + NWV, vb, 0);
            do_row(t + 2 * NWV, vc, 0);
            do_row(t + 3 * NWV, vd, 0);
        }
        for (; t < t1; t += NWV) {
            uint32_t va[NV][NWD];
            load_row(t, va);
            do_row(t, va, 0);
        }
    }
    __syncthreads();

    if (wire) {
        // The block saw every token of the slab: build its CDF tables here.
        // Thread col < NP * 64 owns the counter column (pair, lane), i.e.
        // channels c and c + 1, whose tables (W entries each, W = the
        // slab's table width, adjacent in the wire section) it scans from
        // the counts and writes itself: 4W contiguous bytes, one 128-byte
        // line for W = 32. Entries from NS on (a table wider than the
        // counters: a launch for slabs of at most NS symbols) have all T
        // tokens below them.
        constexpr int NCOL = NP * 64;
        constexpr int WMAX = 32;  // the fused path takes alphabets up to 32
        static_assert(NS <= WMAX, "counters fit the widest table");
        const int col = threadIdx.x;
        const int W = layer_w(mt, sl.kv, sl.l);
        bool bad = false;
        if (col < NCOL) {
            const int pr = col / 64, ln = col % 64;
            const int c = ((pr / NWD) * 64 + ln) * CW + (pr % NWD) * 2;
            const uint64_t S = kProbOne - (uint32_t)W;
            const double invT = 1.0 / (double)T;
            uint32_t cum_lo = 0, cum_hi = 0;
            // Entry q of channels c and c + 1 (call in increasing q).
            auto entry = [&](int q, uint32_t &a0, uint32_t &a1) {
                const uint32_t v = q < NS ? hist[q * NCOL + col] : 0u;
                a0 = (uint32_t)(div_rne((uint64_t)cum_lo * S, (uint32_t)T, invT) + q) & 0xFFFFu;
                a1 = (uint32_t)(div_rne((uint64_t)cum_hi * S, (uint32_t)T, invT) + q) & 0xFFFFu;
                cum_lo += v & 0xFFFFu;
                cum_hi += v >> 16;
            };
            uint16_t *t = call_sec(wire, cm, sl.b) + (wpre ? (int64_t)wpre[sl.ls] : (int64_t)sl.ls * A) * C +
                          (int64_t)c * W;
            // Lanes with 16 channels (C = 1024) hold all of a table pair in
            // registers and store it at once: the whole 128-byte line leaves
            // in one burst (128 calls of 256 tokens: 2.71 vs 2.89 ms). With
            // fewer channels per lane the kernel's registers are fewer than
            // that would take, so eight entries of each table are stored at
            // a time.
            constexpr bool kWhole = NV * CW >= 16;
            if (kWhole && W % 8 == 0) {
                uint32_t x[WMAX / 2], y[WMAX / 2];
#pragma unroll
                for (int q = 0; q < WMAX; q += 2) {
                    x[q / 2] = y[q / 2] = 0;
                    if (q < W) {
                        uint32_t a0, a1, b0, b1;
                        entry(q, a0, a1);
                        entry(q + 1, b0, b1);
                        x[q / 2] = a0 | (b0 << 16);
                        y[q / 2] = a1 | (b1 << 16);
                    }
                }
                uint4 *t4 = reinterpret_cast<uint4 *>(t);
                uint4 *u4 = reinterpret_cast<uint4 *>(t + W);
#pragma unroll
                for (int i = 0; i < WMAX / 8; ++i)
                    if (i < W / 8) t4[i] = make_uint4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
#pragma unroll
                for (int i = 0; i < WMAX / 8; ++i)
                    if (i < W / 8) u4[i] = make_uint4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);
            } else if (W % 8 == 0) {
                // C is a multiple of 256 and c even, so both tables start on
                // 16-byte boundaries: eight entries of each per 16-byte store.
                uint4 *t4 = reinterpret_cast<uint4 *>(t);
                uint4 *u4 = reinterpret_cast<uint4 *>(t + W);
#pragma unroll
                for (int i = 0; i < WMAX / 8; ++i) {
                    if (i < W / 8) {
                        uint32_t x[4], y[4];
#pragma unroll
                        for (int k = 0; k < 8; k += 2) {
                            uint32_t a0, a1, b0, b1;
                            entry(8 * i + k, a0, a1);
                            entry(8 * i + k + 1, b0, b1);
                            x[k / 2] = a0 | (b0 << 16);
                            y[k / 2] = a1 | (b1 << 16);
                        }
                        t4[i] = make_uint4(x[0], x[1], x[2], x[3]);
                        u4[i] = make_uint4(y[0], y[1], y[2], y[3]);
                    }
                }
            } else {
#pragma unroll
                for (int q = 0; q < WMAX; ++q) {
                    if (q < W) {
                        uint32_t a0, a1;
                        entry(q, a0, a1);
                        t[q] = (uint16_t)a0;
                        t[W + q] = (uint16_t)a1;
                    }
                }
            }
            // Counts of symbols at or above the width: not the quantiser's.
#pragma unroll
            for (int q = 0; q < NS; ++q)
                if (q >= W) bad |= hist[q * NCOL + col] != 0;
        }
        if (__ballot(bad) && lane == 0) atomicOr(status, kStCorrupt);
        return;
    }

    // Flush: word (s, pair, lane) holds channels c and c + 1 of symbol s.
    for (int wi = threadIdx.x; wi < NS * NP * 64; wi += NT) {
        const uint32_t v = hist[wi];
        if (!v) continue;
        const int s = wi / (NP * 64), pr = (wi / 64) % NP, ln = wi % 64;
        const int c = ((pr / NWD) * 64 + ln) * CW + (pr % NWD) * 2;
        if (s >= A) {
            atomicOr(status, kStCorrupt);
            continue;
        }
        uint32_t *dst = counts + ((int64_t)slab * C + c) * A + s;
        if (v & 0xFFFFu) atomicAdd(dst, v & 0xFFFFu);
        if (v >> 16) atomicAdd(dst + A, v >> 16);
    }
}

// Tokens per block: at most 1024 blocks over the call, floor(1024 / 2L) per
// slab (a tile of T * 2L / 1024 rounded up could leave a few blocks past the
// chip's resident ones to run alone in a second round: the GLM-4-9B shape,
// 80 slabs of 16K tokens, 1040 -> 960 blocks, 0.49 -> 0.48 ms per
// cg_to_bytes), at least 256 and at most 32768 rows (16-bit counters).
static int64_t quantize_hist_rows(const Dims &d) {
    const int64_t per_slab = std::max<int64_t>(1, 1024 / (2 * (int64_t)d.L));
    int64_t TT = ((int64_t)d.T + per_slab - 1) / per_slab;
    TT = ((TT + 15) / 16) * 16;
    if (TT < 256) TT = 256;
    if (TT > 32768) TT = 32768;
    return TT;
}

// Calls too small to give the fused kernel 16 blocks (a few layers of a
// few tokens) run faster as one wave per row in k_quantize_vec plus the
// separate histogram. (With eight-wave blocks the bar was 64 blocks: the
// OPT-125m shape at 64 tokens, 24 slabs, took 83 us fused against 73
// unfused per to_bytes call; with the sixteen-wave blocks of small grids it
// takes 59 fused against 62.)
bool quantize_hist_fits(const Dims &d, const void *kv, const void *sym) {
    const int64_t TT = quantize_hist_rows(d);
    return (d.C == 256 || d.C == 512 || d.C == 768 || d.C == 1024) && d.A <= 32 && (uintptr_t)kv % 16 == 0 &&
           (uintptr_t)sym % 16 == 0 && 2 * (int64_t)d.L * ((d.T + TT - 1) / TT) >= 16;
}

bool quantize_hist_fuses_cdf(const Dims &d, const void *wire) {
    return quantize_hist_rows(d) >= d.T && (uintptr_t)wire % 16 == 0 && d.cstride % 16 == 0;
}

hipError_t launch_quantize_hist(const Dims &d, const MaxTable &mt, const uint16_t *kv, uint8_t *sym,
                                uint16_t *scale, uint32_t *counts, uint16_t *wire, const uint32_t *wpre,
                                uint32_t *status, bool packed, bool nibbles, hipStream_t s) {
    const int64_t TT = quantize_hist_rows(d);
    if (wire && !quantize_hist_fuses_cdf(d, wire)) return hipErrorInvalidValue;
    if (packed && d.T % 8 != 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((d.T + TT - 1) / TT), (unsigned)(2 * d.L));
    // A grid with fewer blocks than the chip has CUs (a short call) gives
    // each block 16 waves: twice the rows in flight per CU.
    const bool wide = (int64_t)grid.x * grid.y < 256;
    int loga = 2;
    while ((1 << loga) < d.A) ++loga;
    const int tt = (int)TT;
    const CallMap cm = call_map(d);
#define CG_QH_T(NV, CW, LG, PK, NT)                                                                              \
    hipLaunchKernelGGL((k_quantize_hist<NV, CW, LG, PK, NT>), grid, dim3(NT), 0, s, kv, sym, scale, counts, wire, \
                       wpre, status, d.T, d.C, d.A, tt, mt, cm, nibbles)
#define CG_QH(NV, CW, LG)                                  \
    do {                                                   \
        if (packed) {                                      \
            if (wide) CG_QH_T(NV, CW, LG, true, 1024);     \
            else CG_QH_T(NV, CW, LG, true, 512);           \
        } else {                                           \
            if (wide) CG_QH_T(NV, CW, LG, false, 1024);    \
            else CG_QH_T(NV, CW, LG, false, 512);          \
        }                                                  \
    } while (0)
#define CG_QH_A(NV, CW)                         \
    do {                                        \
        switch (loga) {                         \
        case 2: CG_QH(NV, CW, 2); break;        \
        case 3: CG_QH(NV, CW, 3); break;        \
        case 4: CG_QH(NV, CW, 4); break;        \
        default: CG_QH(NV, CW, 5); break;       \
        }                                       \
    } while (0)
    switch (d.C) {
    case 256: CG_QH_A(1, 4); break;
    case 512: CG_QH_A(1, 8); break;
    case 768: CG_QH_A(3, 4); break;
    default: CG_QH_A(2, 8); break;
    }
#undef CG_QH_A
#undef CG_QH
#undef CG_QH_T
    return hipGetLastError();
}

// ------------------------------------------------------------- dequantise

// dq[q] = fl32((q - M) / M) for q in [0, 128), one table per wave in LDS.
__device__ __forceinline__ void build_dq(float *dq, int M, int lane) {
    const float Mf = (float)M;
    dq[lane] = __fdiv_rn((float)(lane - M), Mf);
    dq[lane + 64] = __fdiv_rn((float)(lane + 64 - M), Mf);
}

__global__ __launch_bounds__(256) void k_dequantize(const uint8_t *__restrict__ sym,
                                                    const uint16_t *__restrict__ scale,
                                                    uint16_t *__restrict__ out, int L, int T, int C,
                                                    MaxTable mt, int vec8) {
    __shared__ float dq_all[4][128];
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    const int slab = blockIdx.y, k = slab >= L ? 1 : 0, l = slab - k * L;  // grid: (tokens/4, 2L)
    const int64_t row = (int64_t)slab * T + t;
    float *dq = dq_all[wv];
    build_dq(dq, layer_m(mt, k, l), lane);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const float m = bf16_to_f32(scale[row]);
    const uint8_t *src = sym + row * C;
    uint16_t *dst = out + (((int64_t)l * 2 + k) * T + t) * C;
    if (vec8) {
        for (int c0 = lane * 8; c0 < C; c0 += 512) {
            const uint2 q = *reinterpret_cast<const uint2 *>(src + c0);
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = e < 2 ? q.x : q.y;
                const int sh = (e & 1) * 16;
                const uint32_t a = f32_to_bf16_rne(__fmul_rn(dq[(w >> sh) & 0x7F], m));
                const uint32_t b = f32_to_bf16_rne(__fmul_rn(dq[(w >> (sh + 8)) & 0x7F], m));
                o[e] = a | (b << 16);
            }
            *reinterpret_cast<uint4 *>(dst + c0) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    } else {
        for (int c = lane; c < C; c += 64)
            dst[c] = (uint16_t)f32_to_bf16_rne(__fmul_rn(dq[src[c] & 0x7F], m));
    }
}

hipError_t launch_dequantize(const Dims &d, const MaxTable &mt, const uint8_t *sym,
                             const uint16_t *scale, uint16_t *kv_out, hipStream_t s) {
    const int vec8 = (d.C % 8 == 0) && ((uintptr_t)sym % 8 == 0) && ((uintptr_t)kv_out % 16 == 0);
    hipLaunchKernelGGL(k_dequantize, dim3((unsigned)((d.T + 3) / 4), (unsigned)(2 * d.L)), dim3(256), 0, s, sym, scale,
                       kv_out, d.L, d.T, d.C, mt, vec8);
    return hipGetLastError();
}

// ------------------------------------------------------------ blob header

// One block per blob (blob b at blob + b * stride). Block 0 also zeroes the
// workspace status word when given one: this kernel runs first, so the call
// needs no launch of its own for that.
__global__ __launch_bounds__(256) void k_blob_header(uint8_t *__restrict__ blob, uint64_t stride, HeaderBytes h,
                                                     BlobLayout lay, uint64_t end_scales,
                                                     uint64_t end_cdf, uint64_t end_off,
                                                     uint64_t end_len, uint32_t *__restrict__ status) {
    if (status && blockIdx.x == 0 && threadIdx.x == 0) *status = 0;
    blob += (uint64_t)blockIdx.x * stride;
    for (uint32_t i = threadIdx.x; i < h.n; i += blockDim.x) blob[i] = h.b[i];
    // Zero the gaps between the end of each section and the next one.
    const uint64_t from[4] = {end_scales, end_cdf, end_off, end_len};
    const uint64_t to[4] = {lay.off_cdf, lay.off_chunk_off, lay.off_lengths, lay.off_payload};
    for (int g = 0; g < 4; ++g)
        for (uint64_t i = from[g] + threadIdx.x; i < to[g]; i += blockDim.x) blob[i] = 0;
}

hipError_t launch_blob_header(uint8_t *blob, const HeaderBytes &h, const BlobLayout &lay,
                              const Dims &d, hipStream_t s, int nblobs, uint64_t stride, uint32_t *status) {
    const uint64_t end_scales = lay.off_scales + 4ull * d.L * d.T;
    const uint64_t end_cdf = lay.off_cdf + 2ull * d.C * (uint64_t)d.tab_entries;
    const uint64_t end_off = lay.off_chunk_off + 8ull * (d.NC + 1);
    const uint64_t end_len = lay.off_lengths + 4ull * d.NC * d.L * d.C;
    hipLaunchKernelGGL(k_blob_header, dim3((unsigned)nblobs), dim3(256), 0, s, blob, stride, h, lay, end_scales,
                       end_cdf, end_off, end_len, status);
    return hipGetLastError();
}

}  // namespace cg
