/*
 * CacheGen KV-cache codec -- CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY: a plain, slow, scalar implementation that defines
 * the expected output of every stage of the codec. Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark use it. It shares no code,
 * header, table or constant with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no FMA contraction, so
 * every float operation below is one correctly rounded IEEE operation).
 *
 * Sources (see cachegen_oracle.h for the full titles):
 *   [P2 s1] LMCache CacheGen page, section 1: per-layer bins.
 *   [P2 s2] section 2: symmetric per-layer quantisation with absmax scales.
 *   [P2 s3] section 3: per-(layer, channel) histogram, cumulative sum, scaling
 *           to 16-bit precision and the ramp that makes the CDF strictly
 *           increasing.
 *   [P2 s4] section 4: arithmetic coding in batches of at most 256 tokens,
 *           each batch a byte stream plus one length per stream.
 *   [P2 s5] section 5: decoding with the CDF and the prefix sums of the
 *           lengths, then the inverse scaling t = (t - C) / C * max.
 *
 * Readings where the page leaves a step open (each is stated where it is
 * used): fp32 arithmetic in the quantiser with each operation rounded
 * separately; round-half-even; an all-zero row maps to the centre symbol;
 * one alphabet size A = max bins for every table; the CDF counts all tokens
 * of the call; the coder is a byte-oriented 32-bit range coder (see
 * ocg_encode_stream); lengths are 16-bit.
 */
#include "cachegen_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define CHUNK_TOKENS 256
#define PROB_BITS 16
#define PROB_ONE (1u << PROB_BITS)
#define TOP (1ull << 24)
#define WORD (1ull << 32)

/* ---------------------------------------------------------------- helpers */

static float bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* float32 -> bf16 for a value that is already a bf16 value (low 16 bits 0). */
static uint16_t bf16_exact_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Round a double to the nearest bf16 value, ties to even. The quantum of the
 * binade of |x| (bf16 keeps 8 significant bits; below 2^-126 the quantum is
 * 2^-133) is a power of two, so x / quantum is exact and nearbyint() under
 * the default rounding mode performs the one rounding. */
static uint16_t bf16_round_double(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double ax = fabs(x);
    if (ax == 0.0)
        return sign;
    int e;
    frexp(ax, &e);           /* ax = f * 2^e with f in [0.5, 1) */
    int ex = e - 1;          /* floor(log2(ax)) */
    if (ex < -126)
        ex = -126;
    double quantum = ldexp(1.0, ex - 7);
    double r = nearbyint(ax / quantum) * quantum;
    float f = (float)r; /* exact: r has at most 8 significant bits */
    if (isinf(f))
        return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | bf16_exact_bits(f));
}

/* round_half_even(a / b) for a >= 0, b > 0, exactly. */
static uint64_t div_round_half_even(uint64_t a, uint64_t b)
{
    uint64_t q = a / b, r = a % b;
    if (2 * r > b || (2 * r == b && (q & 1)))
        ++q;
    return q;
}

static int bins_ok(int L, const uint8_t *bk, const uint8_t *bv)
{
    for (int l = 0; l < L; ++l)
        if (bk[l] < 4 || bk[l] > 128 || bv[l] < 4 || bv[l] > 128)
            return 0;
    return 1;
}

/* --------------------------------------------------------- [P2 s1] bins */

int ocg_default_bins(int nlayers, uint8_t *bins_k, uint8_t *bins_v)
{
    if (nlayers < 1 || !bins_k || !bins_v)
        return OCG_ERR_ARG;
    for (int l = 0; l < nlayers; ++l) {
        if (nlayers < 10) {
            bins_k[l] = 32;
            bins_v[l] = 32;
        } else {
            bins_k[l] = (uint8_t)(l < 10 ? 32 : 16);
            bins_v[l] = (uint8_t)(l < 2 ? 32 : 16);
        }
    }
    return 0;
}

/* ------------------------------------------------------ [P2 s2] quantise */

/* For each (kv, layer, token) row of C channels:
 *   M   = bins // 2 - 1 for the row's layer (K or V list);
 *   m   = max_c |x_c|  (the scale; a bf16 value, stored exactly);
 *   q_c = round_half_even(x_c * (M / m) + M), clamped to [0, 2M].
 * The page's expression is two tensor operations (a product by the factor,
 * then the addition of M); they are evaluated in fp32 as the three separately
 * rounded operations f = M / m, y = x * f, z = y + M. A row with m == 0 has
 * no scale to divide by; every symbol of it is M (so it decodes to zero).
 * Nor has a row whose factor M / m overflows fp32 (m below about
 * M * 2^-128, so below 2^-122 for any bins): the page's expression gives no
 * finite value there, and such a row is quantised as an all-zero row, with
 * scale 0. */
int ocg_quantize(int L, int T, int C, const uint8_t *bins_k, const uint8_t *bins_v,
                 const uint16_t *kv, uint8_t *sym, uint16_t *scale)
{
    if (L < 1 || T < 1 || C < 1 || !kv || !sym || !scale || !bins_ok(L, bins_k, bins_v))
        return OCG_ERR_ARG;
    for (int k = 0; k < 2; ++k) {
        for (int l = 0; l < L; ++l) {
            int M = (k == 0 ? bins_k[l] : bins_v[l]) / 2 - 1;
            float Mf = (float)M;
            for (int t = 0; t < T; ++t) {
                const uint16_t *row = kv + (((size_t)l * 2 + k) * T + t) * C;
                uint8_t *out = sym + (((size_t)k * L + l) * T + t) * C;
                float m = 0.0f;
                for (int c = 0; c < C; ++c) {
                    float a = fabsf(bf16_value(row[c]));
                    if (!isfinite(a))
                        return OCG_ERR_NONFINITE;
                    if (a > m)
                        m = a;
                }
                float f = m == 0.0f ? 0.0f : Mf / m;
                if (m == 0.0f || isinf(f)) {
                    /* No finite factor: an all-zero row, or an absmax so
                     * small (below about M * 2^-128) that M / m overflows
                     * fp32. Either row is quantised as all-zero: every
                     * symbol M, scale 0 (it decodes to zeros). */
                    scale[((size_t)k * L + l) * T + t] = 0;
                    for (int c = 0; c < C; ++c)
                        out[c] = (uint8_t)M;
                    continue;
                }
                scale[((size_t)k * L + l) * T + t] = bf16_exact_bits(m);
                for (int c = 0; c < C; ++c) {
                    float y = bf16_value(row[c]) * f;
                    float z = y + Mf;
                    long q = lrintf(z);
                    if (q < 0)
                        q = 0;
                    if (q > 2 * M)
                        q = 2 * M;
                    out[c] = (uint8_t)q;
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------- [P2 s3] histogram + CDF */

/* cnt[kv,l,c,s] = number of tokens t of the call with sym[kv,l,t,c] == s. */
int ocg_histogram(int L, int T, int C, int A, const uint8_t *sym, uint32_t *cnt)
{
    if (L < 1 || T < 1 || C < 1 || A < 2 || !sym || !cnt)
        return OCG_ERR_ARG;
    memset(cnt, 0, sizeof(uint32_t) * 2 * (size_t)L * C * A);
    for (int k = 0; k < 2; ++k)
        for (int l = 0; l < L; ++l)
            for (int t = 0; t < T; ++t) {
                const uint8_t *row = sym + (((size_t)k * L + l) * T + t) * C;
                for (int c = 0; c < C; ++c) {
                    if (row[c] >= A)
                        return OCG_ERR_ARG;
                    cnt[(((size_t)k * L + l) * C + c) * A + row[c]]++;
                }
            }
    return 0;
}

/* The cumulative distribution of a (kv, layer, channel) table is cum[k]/T
 * with cum[k] = sum_{s<k} cnt[s], k = 0..W (Lp = W + 1 entries, W the table's
 * alphabet). It is scaled to 16-bit precision by multiplying with
 * 2^16 - (Lp - 1) = 2^16 - W and adding the ramp k, so that every symbol
 * keeps a frequency of at least 1 and the table is strictly increasing, from
 * 0 to 2^16. The scaled value cum*S/T is rounded half-to-even from the exact
 * rational.
 *
 * The page normalises with one Lp but leaves open what it is. Two readings
 * are built: every table of the call has the call's alphabet, W = A = the
 * largest bins of any layer (widths == NULL, the default), or every table of
 * (kv, layer) has its layer's own alphabet, W = bins of that layer (widths =
 * [2, L] table widths). Tables are stored [2, L, C, A + 1] either way; the
 * entries of a narrower table past its end W hold 2^16 (they belong to no
 * symbol). A count at or past W is an error. */
static int cdf_tables(int L, int T, int C, int A, const uint8_t *widths, const uint32_t *cnt,
                      int32_t *cdf)
{
    if (L < 1 || T < 1 || C < 1 || A < 2 || A > 255 || !cnt || !cdf)
        return OCG_ERR_ARG;
    for (size_t tab = 0; tab < 2 * (size_t)L * C; ++tab) {
        const int W = widths ? widths[tab / (size_t)C] : A;
        if (W < 2 || W > A)
            return OCG_ERR_ARG;
        const uint64_t S = PROB_ONE - (uint64_t)W;
        const uint32_t *h = cnt + tab * A;
        int32_t *out = cdf + tab * (A + 1);
        uint64_t cum = 0;
        for (int k = 0; k <= W; ++k) {
            out[k] = (int32_t)(div_round_half_even(cum * S, (uint64_t)T) + (uint64_t)k);
            if (k < W)
                cum += h[k];
        }
        for (int k = W + 1; k <= A; ++k)
            out[k] = (int32_t)PROB_ONE;
        for (int k = W; k < A; ++k)
            if (h[k])
                return OCG_ERR_ARG;
        if (cum != (uint64_t)T)
            return OCG_ERR_ARG;
    }
    return 0;
}

int ocg_cdf(int L, int T, int C, int A, const uint32_t *cnt, int32_t *cdf)
{
    return cdf_tables(L, T, C, A, NULL, cnt, cdf);
}

int ocg_cdf_w(int L, int T, int C, int A, const uint8_t *widths, const uint32_t *cnt, int32_t *cdf)
{
    if (!widths)
        return OCG_ERR_ARG;
    return cdf_tables(L, T, C, A, widths, cnt, cdf);
}

/* ------------------------------------------------- [P2 s4] range coder */

/* A carry into the bytes already written: trailing 0xFF bytes wrap to 0x00
 * and the byte before them is incremented. The coded value always stays
 * below 1, so a carry never runs past the first byte. */
static int add_carry(uint8_t *out, int64_t n)
{
    int64_t i = n - 1;
    while (i >= 0 && out[i] == 0xFF) {
        out[i] = 0;
        --i;
    }
    if (i < 0)
        return OCG_ERR_CORRUPT;
    out[i]++;
    return 0;
}

/* The page describes CDF-driven arithmetic coding with 16-bit tables but not
 * the coder itself. The reading used here is the classic range coder (an
 * arithmetic coder that emits bytes): a 32-bit window [low, low + range) of
 * the code interval, total frequency 2^16.
 *
 *   start:   low = 0, range = 2^32 - 1.
 *   symbol:  r = range >> 16; low += r * cdf[s] (a carry past 2^32 goes into
 *            the bytes already written); range = r * (cdf[s+1] - cdf[s]);
 *            while range < 2^24: write the top byte of low, shift low and
 *            range left by 8.
 *   finish:  v = the smallest multiple of 2^24 that is >= low. v lies inside
 *            the interval because range >= 2^24. If v == 2^32 it is a carry
 *            and nothing more is written; otherwise the top byte of v is
 *            written if it is not zero.
 */
int64_t ocg_encode_stream(const uint8_t *sym, int n, const int32_t *cdf, int A,
                          uint8_t *out, int64_t cap)
{
    uint64_t low = 0, range = WORD - 1;
    int64_t len = 0;
    for (int i = 0; i < n; ++i) {
        int s = sym[i];
        if (s < 0 || s >= A)
            return OCG_ERR_ARG;
        uint64_t r = range >> PROB_BITS;
        low += r * (uint64_t)cdf[s];
        if (low >= WORD) {
            low -= WORD;
            if (add_carry(out, len))
                return OCG_ERR_CORRUPT;
        }
        range = r * (uint64_t)(cdf[s + 1] - cdf[s]);
        while (range < TOP) {
            if (len >= cap)
                return OCG_ERR_CAPACITY;
            out[len++] = (uint8_t)(low >> 24);
            low = (low << 8) & (WORD - 1);
            range <<= 8;
        }
    }
    uint64_t v = ((low + TOP - 1) / TOP) * TOP;
    if (v == WORD) {
        if (add_carry(out, len))
            return OCG_ERR_CORRUPT;
    } else if (v != 0) {
        if (len >= cap)
            return OCG_ERR_CAPACITY;
        out[len++] = (uint8_t)(v >> 24);
    }
    return len;
}

/* Decoder: bytes past the stored length read as zero. code holds the offset
 * of the coded value from low inside the 32-bit window. The symbol is the s
 * with cdf[s] <= code / r < cdf[s+1] (found by a linear scan here); then the
 * window is narrowed exactly as in the encoder. code < range holds after
 * every step for a well-formed stream. */
int ocg_decode_stream(const uint8_t *in, int64_t len, int n, const int32_t *cdf, int A,
                      uint8_t *sym)
{
    int64_t pos = 0;
    uint64_t code = 0, range = WORD - 1;
    for (int i = 0; i < 4; ++i, ++pos)
        code = (code << 8) | (pos < len ? in[pos] : 0u);
    for (int i = 0; i < n; ++i) {
        uint64_t r = range >> PROB_BITS;
        uint64_t v = code / r;
        if (v > PROB_ONE - 1)
            v = PROB_ONE - 1;
        int s = 0;
        while (s + 1 < A && (uint64_t)cdf[s + 1] <= v)
            ++s;
        sym[i] = (uint8_t)s;
        code -= r * (uint64_t)cdf[s];
        range = r * (uint64_t)(cdf[s + 1] - cdf[s]);
        while (range < TOP) {
            code = ((code << 8) | (pos < len ? in[pos] : 0u)) & (WORD - 1);
            ++pos;
            range <<= 8;
        }
        if (code >= range)
            return OCG_ERR_CORRUPT;
    }
    return 0;
}

static int nchunks_of(int T) { return (T + CHUNK_TOKENS - 1) / CHUNK_TOKENS; }

/* Tables of width W (widths[kv*L + l], or A for all) stored with stride A + 1. */
static int64_t encode_all(int L, int T, int C, int A, const uint8_t *widths, const uint8_t *sym,
                          const int32_t *cdf, uint8_t *payload, int64_t cap, uint16_t *lengths,
                          uint64_t *chunk_off)
{
    if (L < 1 || T < 1 || C < 1 || A < 2 || !sym || !cdf || !lengths || !chunk_off)
        return OCG_ERR_ARG;
    int NC = nchunks_of(T);
    uint8_t stream[CHUNK_TOKENS];
    uint8_t tmp[4 * CHUNK_TOKENS];
    int64_t off = 0;
    for (int j = 0; j < NC; ++j) {
        chunk_off[j] = (uint64_t)off;
        int t0 = j * CHUNK_TOKENS;
        int n = T - t0 < CHUNK_TOKENS ? T - t0 : CHUNK_TOKENS;
        for (int k = 0; k < 2; ++k)
            for (int l = 0; l < L; ++l)
                for (int c = 0; c < C; ++c) {
                    for (int i = 0; i < n; ++i)
                        stream[i] = sym[(((size_t)k * L + l) * T + t0 + i) * C + c];
                    const int32_t *tab = cdf + (((size_t)k * L + l) * C + c) * (A + 1);
                    const int W = widths ? widths[k * L + l] : A;
                    int64_t len = ocg_encode_stream(stream, n, tab, W, tmp, sizeof tmp);
                    if (len < 0)
                        return len;
                    if (len > 0xFFFF)
                        return OCG_ERR_CAPACITY;
                    if (off + len > cap)
                        return OCG_ERR_CAPACITY;
                    if (len)
                        memcpy(payload + off, tmp, (size_t)len);
                    lengths[((size_t)j * 2 * L + (size_t)k * L + l) * C + c] = (uint16_t)len;
                    off += len;
                }
    }
    chunk_off[NC] = (uint64_t)off;
    return off;
}

int64_t ocg_encode(int L, int T, int C, int A, const uint8_t *sym, const int32_t *cdf,
                   uint8_t *payload, int64_t cap, uint16_t *lengths, uint64_t *chunk_off)
{
    return encode_all(L, T, C, A, NULL, sym, cdf, payload, cap, lengths, chunk_off);
}

int64_t ocg_encode_w(int L, int T, int C, int A, const uint8_t *widths, const uint8_t *sym,
                     const int32_t *cdf, uint8_t *payload, int64_t cap, uint16_t *lengths,
                     uint64_t *chunk_off)
{
    if (!widths)
        return OCG_ERR_ARG;
    return encode_all(L, T, C, A, widths, sym, cdf, payload, cap, lengths, chunk_off);
}

static int decode_all(int L, int T, int C, int A, const uint8_t *widths, const uint8_t *payload,
                      int64_t payload_bytes, const uint16_t *lengths, const uint64_t *chunk_off,
                      const int32_t *cdf, uint8_t *sym)
{
    if (L < 1 || T < 1 || C < 1 || A < 2 || !lengths || !chunk_off || !cdf || !sym)
        return OCG_ERR_ARG;
    int NC = nchunks_of(T);
    uint8_t stream[CHUNK_TOKENS];
    if (chunk_off[0] != 0)
        return OCG_ERR_CORRUPT;
    for (int j = 0; j < NC; ++j) {
        uint64_t off = chunk_off[j];
        int t0 = j * CHUNK_TOKENS;
        int n = T - t0 < CHUNK_TOKENS ? T - t0 : CHUNK_TOKENS;
        for (int k = 0; k < 2; ++k)
            for (int l = 0; l < L; ++l)
                for (int c = 0; c < C; ++c) {
                    uint16_t len = lengths[((size_t)j * 2 * L + (size_t)k * L + l) * C + c];
                    if (off + len > (uint64_t)payload_bytes)
                        return OCG_ERR_CORRUPT;
                    const int32_t *tab = cdf + (((size_t)k * L + l) * C + c) * (A + 1);
                    const int W = widths ? widths[k * L + l] : A;
                    int rc = ocg_decode_stream(payload + off, len, n, tab, W, stream);
                    if (rc)
                        return rc;
                    for (int i = 0; i < n; ++i)
                        sym[(((size_t)k * L + l) * T + t0 + i) * C + c] = stream[i];
                    off += len;
                }
        if (off != chunk_off[j + 1])
            return OCG_ERR_CORRUPT;
    }
    return 0;
}

int ocg_decode(int L, int T, int C, int A, const uint8_t *payload, int64_t payload_bytes,
               const uint16_t *lengths, const uint64_t *chunk_off, const int32_t *cdf,
               uint8_t *sym)
{
    return decode_all(L, T, C, A, NULL, payload, payload_bytes, lengths, chunk_off, cdf, sym);
}

int ocg_decode_w(int L, int T, int C, int A, const uint8_t *widths, const uint8_t *payload,
                 int64_t payload_bytes, const uint16_t *lengths, const uint64_t *chunk_off,
                 const int32_t *cdf, uint8_t *sym)
{
    if (!widths)
        return OCG_ERR_ARG;
    return decode_all(L, T, C, A, widths, payload, payload_bytes, lengths, chunk_off, cdf, sym);
}

/* ------------------------------------------------------ [P2 s5] dequantise */

/* x = (q - M) / M * m for each symbol, then cast back to the input dtype.
 * The page's expression is two tensor operations on the decoded symbols;
 * read in fp32, the precision the quantiser is read in ([P2 s2]), they are
 * the separately rounded operations r = fl((q - M) / M) and x = fl(r * m),
 * followed by one round-to-nearest-even to bf16. (Where the exact quotient
 * times m is a bf16 midpoint, these roundings decide the tie, so the
 * result is not always the bf16 nearest to the exact rational.) */
int ocg_dequantize(int L, int T, int C, const uint8_t *bins_k, const uint8_t *bins_v,
                   const uint8_t *sym, const uint16_t *scale, uint16_t *out)
{
    if (L < 1 || T < 1 || C < 1 || !sym || !scale || !out || !bins_ok(L, bins_k, bins_v))
        return OCG_ERR_ARG;
    for (int k = 0; k < 2; ++k)
        for (int l = 0; l < L; ++l) {
            int M = (k == 0 ? bins_k[l] : bins_v[l]) / 2 - 1;
            float Mf = (float)M;
            for (int t = 0; t < T; ++t) {
                float m = bf16_value(scale[((size_t)k * L + l) * T + t]);
                const uint8_t *q = sym + (((size_t)k * L + l) * T + t) * C;
                uint16_t *o = out + (((size_t)l * 2 + k) * T + t) * C;
                for (int c = 0; c < C; ++c) {
                    float r = (float)((int)q[c] - M) / Mf;
                    float x = r * m;
                    /* (double)x is exact, so this is the one rounding of x to bf16. */
                    o[c] = bf16_round_double((double)x);
                }
            }
        }
    return 0;
}

/* ------------------------------------------------------------------ blob */

#define HDR_FIXED 48
#define ALIGN 64

static int64_t align_up(int64_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

static int max_bins(int L, const uint8_t *bk, const uint8_t *bv)
{
    int A = 0;
    for (int l = 0; l < L; ++l) {
        if (bk[l] > A)
            A = bk[l];
        if (bv[l] > A)
            A = bv[l];
    }
    return A;
}

struct layout {
    int64_t header, scales, cdf, offsets, lengths, payload;
};

/* Table widths of the blob format: fmt 0 gives every table the call's
 * alphabet A, fmt 1 gives the tables of (kv, l) the bins of that layer. */
static void table_widths(int L, const uint8_t *bk, const uint8_t *bv, int fmt, uint8_t *w)
{
    const int A = max_bins(L, bk, bv);
    for (int l = 0; l < L; ++l) {
        w[l] = (uint8_t)(fmt ? bk[l] : A);
        w[L + l] = (uint8_t)(fmt ? bv[l] : A);
    }
}

/* entries = the sum of the table widths over the 2L (kv, layer) slabs; the
 * u16 table section holds C tables of each slab, slab after slab. */
static struct layout layout_of(int L, int T, int C, int64_t entries)
{
    struct layout s;
    int64_t NC = nchunks_of(T);
    s.header = 0;
    s.scales = align_up(HDR_FIXED + 2 * (int64_t)L);
    s.cdf = s.scales + align_up(2 * 2 * (int64_t)L * T);
    s.offsets = s.cdf + align_up(2 * (int64_t)C * entries);
    s.lengths = s.offsets + align_up(8 * (NC + 1));
    s.payload = s.lengths + align_up(2 * NC * 2 * (int64_t)L * C);
    return s;
}

static void put16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put32(uint8_t *p, uint32_t v) { for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
static void put64(uint8_t *p, uint64_t v) { for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
static uint16_t get16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get32(const uint8_t *p) { uint32_t v = 0; for (int i = 3; i >= 0; --i) v = (v << 8) | p[i]; return v; }
static uint64_t get64(const uint8_t *p) { uint64_t v = 0; for (int i = 7; i >= 0; --i) v = (v << 8) | p[i]; return v; }

int64_t ocg_blob_bound(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v)
{
    if (L < 1 || T < 1 || H < 1 || D < 1 || !bins_ok(L, bins_k, bins_v))
        return OCG_ERR_ARG;
    int C = H * D;
    struct layout s = layout_of(L, T, C, 2 * (int64_t)L * max_bins(L, bins_k, bins_v));
    int64_t NS = (int64_t)nchunks_of(T) * 2 * L * C;
    return s.payload + NS * (4 * CHUNK_TOKENS);
}

/* Writes everything of the blob but the payload: the zeroed front, the
 * header and the scale, table, chunk-offset and length sections. The pay
 * payload bytes must already sit at the payload offset (or be written there
 * afterwards). Returns the blob size or a negative code. */
int64_t ocg_blob_write(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v, int fmt,
                       const uint16_t *scale, const int32_t *cdf, const uint16_t *lengths,
                       const uint64_t *chunk_off, int64_t pay, uint8_t *blob, int64_t cap)
{
    if (L < 1 || L > 1024 || T < 1 || H < 1 || D < 1 || !blob || !scale || !cdf || !lengths || !chunk_off ||
        pay < 0 || !bins_ok(L, bins_k, bins_v) || (fmt != 0 && fmt != 1))
        return OCG_ERR_ARG;
    int C = H * D, A = max_bins(L, bins_k, bins_v), NC = nchunks_of(T);
    uint8_t W[2048];
    table_widths(L, bins_k, bins_v, fmt, W);
    int64_t entries = 0;
    for (int i = 0; i < 2 * L; ++i)
        entries += W[i];
    struct layout s = layout_of(L, T, C, entries);
    if (cap < s.payload + pay)
        return OCG_ERR_CAPACITY;
    memset(blob, 0, (size_t)s.payload);
    /* header */
    memcpy(blob, "CGMX", 4);
    put16(blob + 4, 1);
    put16(blob + 6, 1);
    put32(blob + 8, (uint32_t)L);
    put32(blob + 12, (uint32_t)T);
    put32(blob + 16, (uint32_t)H);
    put32(blob + 20, (uint32_t)D);
    put32(blob + 24, CHUNK_TOKENS);
    put32(blob + 28, (uint32_t)NC);
    put32(blob + 32, (uint32_t)A);
    put32(blob + 36, (uint32_t)fmt);
    put64(blob + 40, (uint64_t)(s.payload + pay));
    memcpy(blob + HDR_FIXED, bins_k, (size_t)L);
    memcpy(blob + HDR_FIXED + L, bins_v, (size_t)L);
    for (size_t i = 0; i < 2 * (size_t)L * T; ++i)
        put16(blob + s.scales + 2 * i, scale[i]);
    {
        /* Entries 0..W-1 of every table, slab after slab (entry W is 2^16). */
        int64_t e = 0;
        for (size_t tab = 0; tab < 2 * (size_t)L * C; ++tab) {
            const int w = W[tab / (size_t)C];
            for (int k = 0; k < w; ++k)
                put16(blob + s.cdf + 2 * (e++), (uint16_t)cdf[tab * (A + 1) + k]);
        }
    }
    for (int j = 0; j <= NC; ++j)
        put64(blob + s.offsets + 8 * j, chunk_off[j]);
    for (size_t i = 0; i < (size_t)NC * 2 * L * C; ++i)
        put16(blob + s.lengths + 2 * i, lengths[i]);
    return s.payload + pay;
}

int64_t ocg_blob_payload_offset(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v, int fmt)
{
    if (L < 1 || L > 1024 || T < 1 || H < 1 || D < 1 || !bins_ok(L, bins_k, bins_v) || (fmt != 0 && fmt != 1))
        return OCG_ERR_ARG;
    uint8_t W[2048];
    table_widths(L, bins_k, bins_v, fmt, W);
    int64_t entries = 0;
    for (int i = 0; i < 2 * L; ++i)
        entries += W[i];
    return layout_of(L, T, H * D, entries).payload;
}

int64_t ocg_to_bytes_fmt(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v,
                         int fmt, const uint16_t *kv, uint8_t *blob, int64_t cap)
{
    if (L < 1 || L > 1024 || T < 1 || H < 1 || D < 1 || !kv || !blob || !bins_ok(L, bins_k, bins_v) ||
        (fmt != 0 && fmt != 1))
        return OCG_ERR_ARG;
    int C = H * D, A = max_bins(L, bins_k, bins_v), NC = nchunks_of(T);
    uint8_t W[2048];
    table_widths(L, bins_k, bins_v, fmt, W);
    int64_t entries = 0;
    for (int i = 0; i < 2 * L; ++i)
        entries += W[i];
    struct layout s = layout_of(L, T, C, entries);
    if (cap < s.payload)
        return OCG_ERR_CAPACITY;
    size_t n = 2 * (size_t)L * T * C;
    uint8_t *sym = malloc(n);
    uint16_t *scale = malloc(sizeof(uint16_t) * 2 * (size_t)L * T);
    uint32_t *cnt = malloc(sizeof(uint32_t) * 2 * (size_t)L * C * A);
    int32_t *cdf = malloc(sizeof(int32_t) * 2 * (size_t)L * C * (A + 1));
    uint16_t *lengths = malloc(sizeof(uint16_t) * (size_t)NC * 2 * L * C);
    uint64_t *chunk_off = malloc(sizeof(uint64_t) * ((size_t)NC + 1));
    int64_t rc = OCG_ERR_ARG;
    if (!sym || !scale || !cnt || !cdf || !lengths || !chunk_off)
        goto done;
    if ((rc = ocg_quantize(L, T, C, bins_k, bins_v, kv, sym, scale)))
        goto done;
    if ((rc = ocg_histogram(L, T, C, A, sym, cnt)))
        goto done;
    if ((rc = cdf_tables(L, T, C, A, W, cnt, cdf)))
        goto done;
    int64_t pay = encode_all(L, T, C, A, W, sym, cdf, blob + s.payload, cap - s.payload, lengths, chunk_off);
    if (pay < 0) {
        rc = pay;
        goto done;
    }
    if ((rc = ocg_blob_write(L, T, H, D, bins_k, bins_v, fmt, scale, cdf, lengths, chunk_off, pay, blob, cap)) < 0)
        goto done;
    rc = s.payload + pay;
done:
    free(sym);
    free(scale);
    free(cnt);
    free(cdf);
    free(lengths);
    free(chunk_off);
    return rc;
}

int64_t ocg_to_bytes(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v,
                     const uint16_t *kv, uint8_t *blob, int64_t cap)
{
    return ocg_to_bytes_fmt(L, T, H, D, bins_k, bins_v, 0, kv, blob, cap);
}

/* dims: nlayers, ntokens, nheads, head_size, chunk_tokens, nchunks, alphabet,
 * table format. */
int ocg_blob_header(const uint8_t *blob, int64_t size, int32_t dims[8], uint8_t *bins_k,
                    uint8_t *bins_v, int max_layers)
{
    if (!blob || size < HDR_FIXED || memcmp(blob, "CGMX", 4) || get16(blob + 4) != 1 ||
        get16(blob + 6) != 1)
        return OCG_ERR_CORRUPT;
    for (int i = 0; i < 8; ++i)
        dims[i] = (int32_t)get32(blob + 8 + 4 * i);
    if (dims[7] != 0 && dims[7] != 1)
        return OCG_ERR_CORRUPT;
    int L = dims[0];
    if (L < 1 || L > max_layers || size < HDR_FIXED + 2 * (int64_t)L)
        return OCG_ERR_CORRUPT;
    memcpy(bins_k, blob + HDR_FIXED, (size_t)L);
    memcpy(bins_v, blob + HDR_FIXED + L, (size_t)L);
    if (dims[1] < 1 || dims[2] < 1 || dims[3] < 1 || dims[4] != CHUNK_TOKENS ||
        dims[5] != nchunks_of(dims[1]) || !bins_ok(L, bins_k, bins_v) ||
        dims[6] != max_bins(L, bins_k, bins_v) || (int64_t)get64(blob + 40) != size)
        return OCG_ERR_CORRUPT;
    return 0;
}

/* Reads the scale, table, chunk-offset and length sections of a blob whose
 * header ocg_blob_header accepted, into arrays sized by that header (scale
 * [2,L,T], cdf int32 [2,L,C,A+1] with 2^16 past each table's width, lengths
 * [NC,2L,C], chunk_off [NC+1]); *payload_off receives the payload's offset.
 * Rejects tables that are not strictly increasing from 0 and a last chunk
 * offset that is not the payload size. */
int ocg_blob_sections(const uint8_t *blob, int64_t size, uint16_t *scale, int32_t *cdf, uint16_t *lengths,
                      uint64_t *chunk_off, int64_t *payload_off)
{
    int32_t dims[8];
    uint8_t bk[1024], bv[1024];
    int rc = ocg_blob_header(blob, size, dims, bk, bv, 1024);
    if (rc)
        return rc;
    if (!scale || !cdf || !lengths || !chunk_off || !payload_off)
        return OCG_ERR_ARG;
    int L = dims[0], T = dims[1], C = dims[2] * dims[3], NC = dims[5], A = dims[6];
    uint8_t W[2048];
    table_widths(L, bk, bv, dims[7], W);
    int64_t entries = 0;
    for (int i = 0; i < 2 * L; ++i)
        entries += W[i];
    struct layout s = layout_of(L, T, C, entries);
    if (size < s.payload)
        return OCG_ERR_CORRUPT;
    for (size_t i = 0; i < 2 * (size_t)L * T; ++i)
        scale[i] = get16(blob + s.scales + 2 * i);
    {
        int64_t e = 0;
        for (size_t tab = 0; tab < 2 * (size_t)L * C; ++tab) {
            const int w = W[tab / (size_t)C];
            int32_t *t = cdf + tab * (A + 1);
            for (int k = 0; k < w; ++k)
                t[k] = get16(blob + s.cdf + 2 * (e++));
            for (int k = w; k <= A; ++k)
                t[k] = PROB_ONE;
            if (t[0] != 0)
                return OCG_ERR_CORRUPT;
            for (int k = 0; k < w; ++k)
                if (t[k + 1] <= t[k])
                    return OCG_ERR_CORRUPT;
        }
    }
    for (int j = 0; j <= NC; ++j)
        chunk_off[j] = get64(blob + s.offsets + 8 * j);
    for (size_t i = 0; i < (size_t)NC * 2 * L * C; ++i)
        lengths[i] = get16(blob + s.lengths + 2 * i);
    if ((int64_t)chunk_off[NC] != size - s.payload)
        return OCG_ERR_CORRUPT;
    *payload_off = s.payload;
    return 0;
}

int ocg_from_bytes(const uint8_t *blob, int64_t size, uint16_t *kv_out)
{
    int32_t dims[8];
    uint8_t bk[1024], bv[1024];
    int rc = ocg_blob_header(blob, size, dims, bk, bv, 1024);
    if (rc)
        return rc;
    int L = dims[0], T = dims[1], C = dims[2] * dims[3], NC = dims[5], A = dims[6];
    uint8_t W[2048];
    table_widths(L, bk, bv, dims[7], W);
    uint16_t *scale = malloc(sizeof(uint16_t) * 2 * (size_t)L * T);
    int32_t *cdf = malloc(sizeof(int32_t) * 2 * (size_t)L * C * (A + 1));
    uint16_t *lengths = malloc(sizeof(uint16_t) * (size_t)NC * 2 * L * C);
    uint64_t *chunk_off = malloc(sizeof(uint64_t) * ((size_t)NC + 1));
    uint8_t *sym = malloc(2 * (size_t)L * T * C);
    int64_t pay_off = 0;
    rc = OCG_ERR_ARG;
    if (!scale || !cdf || !lengths || !chunk_off || !sym)
        goto done;
    if ((rc = ocg_blob_sections(blob, size, scale, cdf, lengths, chunk_off, &pay_off)))
        goto done;
    if ((rc = decode_all(L, T, C, A, W, blob + pay_off, size - pay_off, lengths, chunk_off, cdf, sym)))
        goto done;
    rc = ocg_dequantize(L, T, C, bk, bv, sym, scale, kv_out);
done:
    free(scale);
    free(cdf);
    free(lengths);
    free(chunk_off);
    free(sym);
    return rc;
}
