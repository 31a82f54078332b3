// Histogram and integer CDF of the CacheGen codec on gfx950.
//
// LMCache CacheGen page (0539edu.com/news/4720135), section 3: the symbols of
// every (K|V, layer, channel) are counted over the tokens, the counts are
// accumulated into a CDF, and the CDF is scaled to 16-bit precision by the
// factor 2^16 - (Lp - 1) plus a ramp 0..Lp-1 so that it is strictly
// increasing. Section 4 says the page's implementation builds the CDF on the
// GPU directly from the symbols; so does this one.
//
// Histogram: a block of 256 threads owns 256 channels of one (K|V, layer)
// over a tile of tokens. Each thread owns one channel, so its counters need
// no atomics across threads: they sit in LDS as uint32 [A][256] (row s,
// column = thread), which keeps every LDS access of a wave on distinct banks
// whatever the symbols are; an increment is one ds_add. Loads are one byte
// per thread, 256 contiguous bytes per token row, eight rows in flight. At
// the end of the tile the non-zero counters are added to the global uint32
// counts with atomics.
#include "cg_internal.hpp"

namespace cg {

__global__ __launch_bounds__(256) void k_histogram(const uint8_t *__restrict__ sym,
                                                   uint32_t *__restrict__ counts,
                                                   uint32_t *__restrict__ status, int L, int T,
                                                   int C, int A, int TT) {
    extern __shared__ uint32_t hist[];  // [A][256]
    const int tid = threadIdx.x;
    const int slab = blockIdx.z;                 // kv * L + l
    const int c = blockIdx.y * 256 + tid;
    const int t0 = blockIdx.x * TT;
    const int t1 = min(T, t0 + TT);
    for (int s = 0; s < A; ++s) hist[s * 256 + tid] = 0;
    if (c >= C) return;
    const uint8_t *p = sym + ((int64_t)slab * T + t0) * C + c;
    const uint32_t amax = (uint32_t)A - 1;
    uint32_t qmax = 0;
    auto bump = [&](uint32_t q) {
        qmax = max(qmax, q);
        __hip_atomic_fetch_add(&hist[min(q, amax) * 256 + tid], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    int t = t0;
    for (; t + 8 <= t1; t += 8) {
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = p[(int64_t)i * C];
        p += 8 * (int64_t)C;
#pragma unroll
        for (int i = 0; i < 8; ++i) bump(q[i]);
    }
    for (; t < t1; ++t, p += C) bump(p[0]);
    if (qmax > amax) atomicOr(status, kStCorrupt);
    uint32_t *dst = counts + ((int64_t)slab * C + c) * A;
    for (int s = 0; s < A; ++s) {
        const uint32_t v = hist[s * 256 + tid];
        if (v) atomicAdd(dst + s, v);
    }
}

// Histogram for C % 4 == 0: one wave owns 256 channels (4 per lane, read as
// one 32-bit word per token row) of one (K|V, layer) over a tile of at most
// 65535 tokens, so two 16-bit counts fit one 32-bit word. Counters are
// lane-private in LDS as uint32 [symbol][pair][lane] (pair 0 holds channels
// 4*lane and 4*lane+1 in its low and high halves, pair 1 the next two), which
// keeps every ds_add of a wave on distinct banks; 32 rows are in flight per
// lane. The table covers 2^LOGA symbols; symbols are read as LOGA-bit fields
// (so the LDS index stays in range) and the OR of all words flags symbols
// >= 2^LOGA; a count for a symbol in [A, 2^LOGA) flags the rest.
template <int LOGA>
__global__ __launch_bounds__(64) void k_histogram4(const uint8_t *__restrict__ sym,
                                                   uint32_t *__restrict__ counts,
                                                   uint32_t *__restrict__ status, int T, int C, int A,
                                                   int TT) {
    constexpr int NS = 1 << LOGA;
    constexpr int U = 32;
    __shared__ __attribute__((aligned(16))) uint32_t hist[NS * 2 * 64];
    const int lane = threadIdx.x;
    const int slab = blockIdx.z;
    const int c0 = blockIdx.y * 256 + lane * 4;
    const int t0 = blockIdx.x * TT;
    const int t1 = min(T, t0 + TT);
    uint4 *h4 = reinterpret_cast<uint4 *>(hist);
#pragma unroll
    for (int i = 0; i < NS * 2 * 64 / 4 / 64; ++i) h4[i * 64 + lane] = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();
    if (c0 >= C) return;
    const uint8_t *p = sym + ((int64_t)slab * T + t0) * C + c0;
    const uint32_t lane4 = (uint32_t)lane * 4;
    uint8_t *hb = reinterpret_cast<uint8_t *>(hist);
    uint32_t acc = 0;
    auto bump = [&](uint32_t w) {
        acc |= w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t q = __builtin_amdgcn_ubfe(w, 8 * e, LOGA);
            uint32_t *cnt = reinterpret_cast<uint32_t *>(hb + (q << 9) + lane4 + (e >> 1) * 256);
            __hip_atomic_fetch_add(cnt, (e & 1) ? 0x10000u : 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        }
    };
    int t = t0;
    for (; t + U <= t1; t += U) {
        uint32_t w[U];
#pragma unroll
        for (int i = 0; i < U; ++i) w[i] = *reinterpret_cast<const uint32_t *>(p + (int64_t)i * C);
        p += (int64_t)U * C;
#pragma unroll
        for (int i = 0; i < U; ++i) bump(w[i]);
    }
    for (; t < t1; ++t, p += C) bump(*reinterpret_cast<const uint32_t *>(p));
    bool bad = (acc & ~(0x01010101u * (uint32_t)(NS - 1))) != 0;
    __builtin_amdgcn_wave_barrier();
    uint32_t *dst = counts + ((int64_t)slab * C + c0) * A;
    for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const uint32_t v = hist[(s * 2 + pr) * 64 + lane];
            if (!v) continue;
            if (s >= A) {
                bad = true;
                continue;
            }
            const uint32_t lo = v & 0xFFFFu, hi = v >> 16;
            if (lo) atomicAdd(dst + (2 * pr) * A + s, lo);
            if (hi) atomicAdd(dst + (2 * pr + 1) * A + s, hi);
        }
    }
    if (bad) atomicOr(status, kStCorrupt);
}

hipError_t launch_histogram(const Dims &d, const uint8_t *sym, uint32_t *counts,
                            uint32_t *status, hipStream_t s) {
    const int64_t slabs = 2LL * d.L;
    if (d.C % 4 == 0 && (uintptr_t)sym % 4 == 0) {
        // Token tiles of at most 65535 (16-bit counts) and enough waves to fill the chip.
        const int cgroups = (d.C + 255) / 256;
        int TT = min(d.T, 32768);
        while (slabs * cgroups * ((d.T + TT - 1) / TT) < 8192 && TT > 256) TT = (TT + 1) / 2;
        const dim3 grid((unsigned)((d.T + TT - 1) / TT), (unsigned)cgroups, (unsigned)slabs);
        int loga = 2;
        while ((1 << loga) < d.A) ++loga;
        switch (loga) {
        case 2: hipLaunchKernelGGL(k_histogram4<2>, grid, dim3(64), 0, s, sym, counts, status, d.T, d.C, d.A, TT); break;
        case 3: hipLaunchKernelGGL(k_histogram4<3>, grid, dim3(64), 0, s, sym, counts, status, d.T, d.C, d.A, TT); break;
        case 4: hipLaunchKernelGGL(k_histogram4<4>, grid, dim3(64), 0, s, sym, counts, status, d.T, d.C, d.A, TT); break;
        case 5: hipLaunchKernelGGL(k_histogram4<5>, grid, dim3(64), 0, s, sym, counts, status, d.T, d.C, d.A, TT); break;
        case 6: hipLaunchKernelGGL(k_histogram4<6>, grid, dim3(64), 0, s, sym, counts, status, d.T, d.C, d.A, TT); break;
        default: hipLaunchKernelGGL(k_histogram4<7>, grid, dim3(64), 0, s, sym, counts, status, d.T, d.C, d.A, TT); break;
        }
        return hipGetLastError();
    }
    // Any C: one byte per thread and channel.
    const int cgroups = (d.C + 255) / 256;
    int TT = d.T;
    while (slabs * cgroups * ((d.T + TT - 1) / TT) < 2048 && TT > 512) TT = (TT + 1) / 2;
    const dim3 grid((unsigned)((d.T + TT - 1) / TT), (unsigned)cgroups, (unsigned)slabs);
    const size_t lds = (size_t)d.A * 256 * sizeof(uint32_t);
    hipLaunchKernelGGL(k_histogram, grid, dim3(256), lds, s, sym, counts, status, d.L, d.T, d.C,
                       d.A, TT);
    return hipGetLastError();
}

// cdf[k] = round_half_even(cum[k] * (2^16 - W) / T) + k, cum[k] the count of
// symbols below k, k = 0..W, W the table's width (the call's alphabet A, or
// the layer's bins for per-layer tables). G lanes per table (G = the power
// of two >= A, at most 64; 64 / G tables per wave): lane k reads count k
// (coalesced), the segmented scan of G lanes gives cum, and lane k writes
// entry k of the table (the first lane of a table also writes entry W). An
// alphabet above 64 takes two rounds of 64, the second starting from the
// first one's total. int32 tables are [2,L,C,A+1] with 2^16 past entry W; u16
// wire tables hold entries 0..W-1 at wpre[ls] * C + c * W of their call's
// section (wpre null: one width A, ls * A).
template <int G>
__global__ __launch_bounds__(256) void k_cdf(const uint32_t *__restrict__ counts,
                                             int32_t *__restrict__ cdf,
                                             uint16_t *__restrict__ wire,
                                             const uint32_t *__restrict__ wpre,
                                             uint32_t *__restrict__ status, int64_t ntab, int A,
                                             int T, int C, MaxTable mt, CallMap cm) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t tab = wave * (64 / G) + lane / G;
    const int k0 = lane & (G - 1);
    const bool live = tab < ntab;
    const int slab = live ? (int)(tab / C) : 0;
    const int c = (int)(tab - (int64_t)slab * C);
    const SlabLoc sl = slab_loc(cm, slab);
    const int W = layer_w(mt, sl.kv, sl.l);
    const uint64_t S = kProbOne - (uint32_t)W;
    const double invT = 1.0 / (double)T;
    uint16_t *wt = wire && live ? call_sec(wire, cm, sl.b) +
                                      (wpre ? (int64_t)wpre[sl.ls] : (int64_t)sl.ls * A) * C + (int64_t)c * W
                                : nullptr;
    uint64_t base = 0;
    bool bad = false;
    for (int kb = 0; kb < A; kb += G) {
        const int k = kb + k0;
        const uint32_t h = live && k < A ? counts[tab * A + k] : 0u;
        bad |= k >= W && h != 0;
        uint32_t incl = h;
#pragma unroll
        for (int o = 1; o < G; o <<= 1) {
            const uint32_t t = (uint32_t)__shfl_up((int)incl, o, G);
            if (k0 >= o) incl += t;
        }
        if (live && k < A) {
            const uint32_t v = k < W ? (uint32_t)(div_rne((base + incl - h) * S, (uint32_t)T, invT) + (uint64_t)k)
                                     : kProbOne;
            if (cdf) cdf[tab * (A + 1) + k] = (int32_t)v;
            if (wt && k < W) wt[k] = (uint16_t)v;
        }
        base += (uint32_t)__shfl((int)incl, G - 1, G);
    }
    if (live && k0 == 0) {
        // Entry W is 2^16 exactly when the counts add up to T.
        if (cdf) cdf[tab * (A + 1) + A] = W == A ? (int32_t)(div_rne(base * S, (uint32_t)T, invT) + (uint64_t)A)
                                                 : (int32_t)kProbOne;
        bad |= base != (uint64_t)T;
    }
    if (__ballot(live && bad) && lane == 0) atomicOr(status, kStCorrupt);
}

hipError_t launch_cdf(const Dims &d, const MaxTable &mt, const uint32_t *counts, int32_t *cdf,
                      uint16_t *cdf_wire, const uint32_t *wpre, uint32_t *status, hipStream_t s) {
    const int64_t ntab = 2LL * d.L * d.C;
#define CG_CDF(GG)                                                                                      \
    hipLaunchKernelGGL(k_cdf<GG>, dim3((unsigned)((ntab + 4 * (64 / GG) - 1) / (4 * (64 / GG)))), dim3(256), \
                       0, s, counts, cdf, cdf_wire, wpre, status, ntab, d.A, d.T, d.C, mt, call_map(d))
    if (d.A <= 8) CG_CDF(8);
    else if (d.A <= 16) CG_CDF(16);
    else if (d.A <= 32) CG_CDF(32);
    else CG_CDF(64);
#undef CG_CDF
    return hipGetLastError();
}

// wpre[s] = the sum of the table widths of the (K|V, layer) slabs of a call
// before s, s = 0..2Lc (so wpre[2Lc] is the whole section's entries per
// channel); every call of a batch places its tables alike.
__global__ __launch_bounds__(1024) void k_table_prefix(MaxTable mt, int L, uint32_t *__restrict__ wpre) {
    __shared__ uint32_t wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = 2 * L;
    uint32_t run = 0;
    for (int seg = 0; seg < n; seg += 1024) {
        const int i = seg + tid;
        uint32_t v = 0;
        if (i < n) {
            const int kv = i >= L ? 1 : 0;
            v = (uint32_t)layer_w(mt, kv, i - kv * L);
        }
        const uint32_t incl = wave_incl_scan_u32(v, lane);
        if (lane == 63) wsum[wv] = incl;
        __syncthreads();
        uint32_t before = 0, total = 0;
        for (int k = 0; k < 16; ++k) {
            if (k < wv) before += wsum[k];
            total += wsum[k];
        }
        if (i < n) wpre[i] = run + before + incl - v;
        run += total;
        __syncthreads();
    }
    if (tid == 0) wpre[n] = run;
}

hipError_t launch_table_prefix(const Dims &d, const MaxTable &mt, uint32_t *wpre, hipStream_t s) {
    hipLaunchKernelGGL(k_table_prefix, dim3(1), dim3(1024), 0, s, mt, d.Lc, wpre);
    return hipGetLastError();
}

}  // namespace cg
