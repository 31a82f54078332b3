/*
 * Test-only driver: runs the oracle's whole-call paths on small seeded inputs
 * so that a build with AddressSanitizer and UndefinedBehaviorSanitizer can
 * check them for out-of-bounds accesses, leaks and undefined behaviour. It
 * exercises the one-thread and multi-threaded encode and decode, both table
 * formats, ragged token counts, and the rejection of corrupt blobs (a
 * truncated blob, a chunk offset and a length that disagree with the
 * payload). Exit status 0 when every result is as expected.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cachegen_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void)
{
    /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

/* A bf16 value of moderate magnitude with a random sign (exponent 118..133). */
static uint16_t random_bf16(void)
{
    uint32_t r = next_u32();
    uint16_t exp = (uint16_t)(118 + (r % 16));
    return (uint16_t)(((r >> 8) & 0x8000u) | (exp << 7) | ((r >> 16) & 0x7Fu));
}

static int run_case(int L, int T, int H, int D, int fmt, int threads)
{
    const size_t n = (size_t)L * 2 * T * H * D;
    uint16_t *kv = malloc(n * sizeof *kv);
    uint16_t *out1 = malloc(n * sizeof *out1);
    uint16_t *out2 = malloc(n * sizeof *out2);
    uint8_t bk[64], bv[64];
    for (int l = 0; l < L; ++l) {
        bk[l] = (uint8_t)(4 + next_u32() % 125);
        bv[l] = (uint8_t)(4 + next_u32() % 125);
    }
    for (size_t i = 0; i < n; ++i)
        kv[i] = (i % 97 == 0) ? 0 : random_bf16();
    const int64_t cap = ocg_blob_bound(L, T, H, D, bk, bv);
    uint8_t *b1 = malloc((size_t)cap), *b2 = malloc((size_t)cap);
    int bad = 0;
    const int64_t s1 = ocg_to_bytes_fmt(L, T, H, D, bk, bv, fmt, kv, b1, cap);
    const int64_t s2 = ocg_to_bytes_mt(L, T, H, D, bk, bv, fmt, kv, b2, cap, threads);
    if (s1 <= 0 || s1 != s2 || memcmp(b1, b2, (size_t)s1)) {
        fprintf(stderr, "encode mismatch L=%d T=%d fmt=%d: %lld vs %lld\n", L, T, fmt, (long long)s1,
                (long long)s2);
        bad = 1;
    }
    if (!bad) {
        const int r1 = ocg_from_bytes(b1, s1, out1);
        const int r2 = ocg_from_bytes_mt(b1, s1, out2, threads);
        if (r1 || r2 || memcmp(out1, out2, n * sizeof *out1)) {
            fprintf(stderr, "decode mismatch L=%d T=%d fmt=%d: %d %d\n", L, T, fmt, r1, r2);
            bad = 1;
        }
        /* Corrupt blobs are rejected, not read out of bounds. */
        if (ocg_from_bytes(b1, s1 - 1, out1) == 0 || ocg_from_bytes_mt(b1, s1 - 1, out2, threads) == 0) {
            fprintf(stderr, "truncated blob accepted\n");
            bad = 1;
        }
        int32_t dims[8];
        uint8_t hk[1024], hv[1024];
        ocg_blob_header(b1, s1, dims, hk, hv, 1024);
        const int64_t pay = ocg_blob_payload_offset(L, T, H, D, bk, bv, fmt);
        const int NC = (T + 255) / 256;
        const int64_t off_len = pay - ((2 * (int64_t)NC * 2 * L * H * D + 63) / 64 * 64);
        memcpy(b2, b1, (size_t)s1);
        b2[off_len] = 0xFF;  /* first length: 0x..FF */
        b2[off_len + 1] = 0x01;
        if (ocg_from_bytes(b2, s1, out1) == 0 || ocg_from_bytes_mt(b2, s1, out2, threads) == 0) {
            fprintf(stderr, "bad length accepted\n");
            bad = 1;
        }
    }
    free(kv);
    free(out1);
    free(out2);
    free(b1);
    free(b2);
    return bad;
}

int main(void)
{
    int bad = 0;
    bad |= run_case(1, 1, 1, 8, 0, 2);
    bad |= run_case(3, 257, 2, 24, 1, 3);
    bad |= run_case(2, 700, 1, 40, 0, 4);
    bad |= run_case(5, 130, 3, 8, 1, 8);
    if (!bad)
        printf("oracle sanitizer driver: ok\n");
    return bad;
}
