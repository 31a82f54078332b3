/*
 * Test-only driver for the host side of the C ABI, built with
 * AddressSanitizer and UBSan together with a host-sanitized build of the
 * library's API translation unit. It needs no GPU: it calls the host-only
 * entry points (messages, bins, descriptor checks, sizes, layouts, header
 * parsing of real, truncated and corrupted headers) and the device entry
 * points with arguments that fail validation, which return before anything
 * is launched. Exit status 0 when every call returns what it should.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cachegen.h"

static int failures = 0;
#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static void put32(uint8_t *p, uint32_t v) { for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i)); }

/* A header as cg_to_bytes writes it (the sizes only; no sections). */
static size_t make_header(uint8_t *h, int L, int T, int H, int D, const uint8_t *bk, const uint8_t *bv) {
    cg_desc d = {L, T, H, D, bk, bv, CG_TABLES_SHARED, 0};
    cg_blob_info info;
    memset(h, 0, 48 + 2 * (size_t)L);
    memcpy(h, "CGMX", 4);
    h[4] = 1;
    h[6] = 1;
    put32(h + 8, (uint32_t)L);
    put32(h + 12, (uint32_t)T);
    put32(h + 16, (uint32_t)H);
    put32(h + 20, (uint32_t)D);
    put32(h + 24, CG_CHUNK_TOKENS);
    put32(h + 28, (uint32_t)((T + 255) / 256));
    int A = 0;
    for (int l = 0; l < L; ++l) {
        if (bk[l] > A) A = bk[l];
        if (bv[l] > A) A = bv[l];
    }
    put32(h + 32, (uint32_t)A);
    EXPECT(cg_blob_layout(&d, &info) == CG_OK);
    const uint64_t size = info.off_payload + 100;
    for (int i = 0; i < 8; ++i) h[40 + i] = (uint8_t)(size >> (8 * i));
    memcpy(h + 48, bk, (size_t)L);
    memcpy(h + 48 + L, bv, (size_t)L);
    return 48 + 2 * (size_t)L;
}

int main(void) {
    for (int c = -12; c <= 2; ++c) EXPECT(cg_strerror(c) != NULL && strlen(cg_strerror(c)) > 0);
    EXPECT(cg_version() >= 2);

    uint8_t bk[1100], bv[1100];
    EXPECT(cg_default_bins(0, bk, bv) != CG_OK);
    EXPECT(cg_default_bins(1025, bk, bv) != CG_OK);
    EXPECT(cg_default_bins(1, NULL, bv) != CG_OK);
    EXPECT(cg_default_bins(40, bk, bv) == CG_OK && bk[9] == 32 && bk[10] == 16 && bv[1] == 32 && bv[2] == 16);
    EXPECT(cg_default_bins(1024, bk, bv) == CG_OK);

    /* Descriptor checks. */
    cg_desc d = {32, 32768, 8, 128, bk, bv, CG_TABLES_SHARED, 0};
    EXPECT(cg_desc_check(&d) == CG_OK);
    EXPECT(cg_desc_check(NULL) != CG_OK);
    cg_desc e = d;
    e.bins_k = NULL;
    EXPECT(cg_desc_check(&e) == CG_E_INVAL);
    e = d;
    e.nlayers = 0;
    EXPECT(cg_desc_check(&e) != CG_OK);
    e = d;
    e.nlayers = 1025;
    EXPECT(cg_desc_check(&e) != CG_OK);
    e = d;
    e.ntokens = -5;
    EXPECT(cg_desc_check(&e) != CG_OK);
    e = d;
    e.nheads = 1 << 20;
    e.head_size = 1 << 20;
    EXPECT(cg_desc_check(&e) != CG_OK);
    e = d;
    e.table_format = 7;
    EXPECT(cg_desc_check(&e) != CG_OK);
    uint8_t badb[32];
    memset(badb, 3, sizeof badb);
    e = d;
    e.bins_v = badb;
    EXPECT(cg_desc_check(&e) == CG_E_INVAL);

    /* Sizes and layouts for every operation, and a bad operation. */
    for (int op = 0; op <= 6; ++op) EXPECT(cg_workspace_bytes(&d, op) >= 256);
    EXPECT(cg_workspace_bytes(&d, 99) < 0);
    EXPECT(cg_workspace_bytes(&e, CG_OP_TO_BYTES) < 0);
    EXPECT(cg_encode_bound(&d) == (int64_t)128 * 64 * 1024 * CG_MAX_STREAM_BYTES);
    EXPECT(cg_blob_bound(&d) > cg_encode_bound(&d));
    cg_blob_info info;
    EXPECT(cg_blob_layout(&d, &info) == CG_OK && info.off_payload % 64 == 0 && info.nchunks == 128);
    EXPECT(cg_blob_layout(NULL, &info) != CG_OK);
    EXPECT(cg_workspace_bytes_batch(&d, 2, (size_t)cg_blob_bound(&d), CG_OP_TO_BYTES) > 0);
    EXPECT(cg_workspace_bytes_batch(&d, 0, 64, CG_OP_TO_BYTES) < 0);

    /* Header parsing: a real header, every truncation of it, and corruptions. */
    uint8_t h[48 + 2 * 40];
    uint8_t ok_k[40], ok_v[40], out_k[40], out_v[40];
    cg_default_bins(40, ok_k, ok_v);
    const size_t hn = make_header(h, 40, 16384, 2, 128, ok_k, ok_v);
    EXPECT(cg_blob_peek(h, hn, &info, out_k, out_v, 40) == CG_OK && info.nlayers == 40 &&
           memcmp(out_k, ok_k, 40) == 0 && memcmp(out_v, ok_v, 40) == 0);
    for (size_t n = 0; n < hn; ++n) {
        uint8_t *copy = malloc(n ? n : 1); /* exactly n bytes: any read past them is reported */
        memcpy(copy, h, n);
        EXPECT(cg_blob_peek(copy, n, &info, out_k, out_v, 40) != CG_OK);
        free(copy);
    }
    EXPECT(cg_blob_peek(h, hn, &info, out_k, out_v, 39) == CG_E_CAPACITY);
    for (size_t i = 0; i < 48; ++i) {
        uint8_t c[sizeof h];
        memcpy(c, h, sizeof h);
        c[i] ^= 0x5A;
        (void)cg_blob_peek(c, hn, &info, out_k, out_v, 40); /* must not read out of bounds */
    }
    uint8_t c2[sizeof h];
    memcpy(c2, h, sizeof h);
    c2[48] = 3; /* bins below 4 */
    EXPECT(cg_blob_peek(c2, hn, &info, out_k, out_v, 40) == CG_E_CORRUPT);
    put32(c2, 0);
    EXPECT(cg_blob_peek(c2, hn, &info, out_k, out_v, 40) == CG_E_CORRUPT);

    /* Device entry points with arguments that fail validation: nothing is
     * launched (no GPU is needed). */
    uint64_t dummy[64];
    void *p = dummy;
    EXPECT(cg_to_bytes(&d, NULL, p, 1 << 20, p, p, (size_t)-1, NULL) == CG_E_INVAL);
    EXPECT(cg_to_bytes(&d, p, p, 1 << 20, p, NULL, (size_t)-1, NULL) == CG_E_INVAL);
    EXPECT(cg_to_bytes(&d, p, p, 1 << 20, p, p, 16, NULL) == CG_E_WORKSPACE);
    EXPECT(cg_from_bytes(&e, p, 64, p, p, 1 << 20, NULL) == CG_E_INVAL);
    EXPECT(cg_from_bytes(&d, p, 64, p, p, 16, NULL) == CG_E_WORKSPACE);
    EXPECT(cg_from_bytes_noalloc(&d, NULL, 64, p, (uint32_t *)p, NULL) == CG_E_INVAL);
    EXPECT(cg_from_bytes_noalloc(&d, p, 64, p, NULL, NULL) == CG_E_INVAL);
    cg_desc big = {64, 16384, 32, 128, bk, bv, CG_TABLES_SHARED, 0};
    cg_default_bins(64, bk, bv);
    EXPECT(cg_from_bytes_noalloc(&big, p, 64, p, (uint32_t *)p, NULL) == CG_E_WORKSPACE);
    cg_default_bins(40, bk, bv);
    int64_t wsb = cg_workspace_bytes(&d, CG_OP_FROM_BYTES);
    EXPECT(cg_from_bytes_chunks(&d, p, 64, 3, 3, p, p, (size_t)wsb, NULL) == CG_E_INVAL);
    EXPECT(cg_from_bytes_chunks(&d, p, 64, -1, 3, p, p, (size_t)wsb, NULL) == CG_E_INVAL);
    EXPECT(cg_from_bytes_chunks(&d, p, 64, 0, 129, p, p, (size_t)wsb, NULL) == CG_E_INVAL);
    EXPECT(cg_from_bytes_paged(&d, p, 64, p, 0, 0, 3, (const int32_t *)p, 10, p, (size_t)wsb, NULL) != CG_OK);
    EXPECT(cg_quantize(&d, NULL, p, p, p, 1 << 20, NULL) == CG_E_INVAL);
    EXPECT(cg_build_cdf(&d, NULL, p, p, 1 << 20, NULL) != CG_OK);
    EXPECT(cg_encode(&d, p, p, p, 16, p, p, p, 16, NULL) != CG_OK);
    EXPECT(cg_decode(&d, NULL, 0, p, p, p, p, p, 16, NULL) != CG_OK);
    EXPECT(cg_dequantize(&d, NULL, p, p, NULL, 0, NULL) == CG_E_INVAL);
    EXPECT(cg_to_bytes_batch(&d, 0, p, p, 64, p, p, 1 << 20, NULL) != CG_OK);
    EXPECT(cg_from_bytes_batch(&d, -1, p, 64, p, p, p, 1 << 20, NULL) != CG_OK);
    EXPECT(cg_read_status(NULL, NULL) == CG_E_INVAL);

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("abi sanitizer driver: ok\n");
    return 0;
}
