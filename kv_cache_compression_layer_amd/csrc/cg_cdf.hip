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

hipError_t launch_histogram(const Dims &d, const uint8_t *sym, uint32_t *counts,
                            uint32_t *status, hipStream_t s) {
    // Token tiles: enough blocks to fill the chip.
    const int cgroups = (d.C + 255) / 256;
    const int64_t slabs = 2LL * d.L;
    int TT = d.T;
    while (slabs * cgroups * ((d.T + TT - 1) / TT) < 2048 && TT > 512) TT = (TT + 1) / 2;
    const dim3 grid((unsigned)((d.T + TT - 1) / TT), (unsigned)cgroups, (unsigned)slabs);
    const size_t lds = (size_t)d.A * 256 * sizeof(uint32_t);
    hipLaunchKernelGGL(k_histogram, grid, dim3(256), lds, s, sym, counts, status, d.L, d.T, d.C,
                       d.A, TT);
    return hipGetLastError();
}

// round_half_even(num / T) for num < 2^48: a double-precision quotient is
// within one of the true quotient; the integer remainder fixes it exactly.
__device__ __forceinline__ uint64_t div_rne(uint64_t num, uint32_t T, double invT) {
    int64_t q = (int64_t)((double)num * invT);
    int64_t r = (int64_t)num - q * (int64_t)T;
    while (r < 0) { --q; r += T; }
    while (r >= (int64_t)T) { ++q; r -= T; }
    if (2 * r > (int64_t)T || (2 * r == (int64_t)T && (q & 1))) ++q;
    return (uint64_t)q;
}

// One thread per table: cdf[k] = round_half_even(cum[k] * (2^16 - A) / T) + k.
__global__ __launch_bounds__(256) void k_cdf(const uint32_t *__restrict__ counts,
                                             int32_t *__restrict__ cdf,
                                             uint16_t *__restrict__ wire,
                                             uint32_t *__restrict__ status, int64_t ntab, int A,
                                             int T) {
    const int64_t tab = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (tab >= ntab) return;
    const uint64_t S = kProbOne - (uint32_t)A;
    const double invT = 1.0 / (double)T;
    const uint32_t *h = counts + tab * A;
    int32_t *out = cdf + tab * (A + 1);
    uint16_t *w = wire ? wire + tab * A : nullptr;
    uint64_t cum = 0;
    for (int k = 0; k <= A; ++k) {
        const uint32_t v = (uint32_t)(div_rne(cum * S, (uint32_t)T, invT) + (uint64_t)k);
        out[k] = (int32_t)v;
        if (k < A) {
            if (w) w[k] = (uint16_t)v;
            cum += h[k];
        }
    }
    if (cum != (uint64_t)T) atomicOr(status, kStCorrupt);
}

hipError_t launch_cdf(const Dims &d, const uint32_t *counts, int32_t *cdf, uint16_t *cdf_wire,
                      uint32_t *status, hipStream_t s) {
    const int64_t ntab = 2LL * d.L * d.C;
    hipLaunchKernelGGL(k_cdf, dim3((unsigned)((ntab + 255) / 256)), dim3(256), 0, s, counts, cdf,
                       cdf_wire, status, ntab, d.A, d.T);
    return hipGetLastError();
}

}  // namespace cg
