/*
 * CacheGen KV-cache codec -- CPU oracle, multi-threaded driver.
 *
 * TEST INFRASTRUCTURE ONLY, like cachegen_oracle.c: the tests use it to check
 * the benchmark-sized workloads whole, and the CPU-baseline leg of the
 * benchmark times it on all host cores. The product never links or calls it.
 *
 * It performs no step of the codec. In the LMCache CacheGen page
 * ("LMCache 中的 KV Cache 压缩：CacheGen 编解码原理、配置方式与源码解析",
 * 0539edu.com/news/4720135) the scale of a row (section 2), the CDF of a
 * (layer, channel) (section 3) and the streams (section 4) of a (K|V, layer)
 * slab depend on that slab's values only, so each layer is a complete
 * one-layer call of the oracle. This driver hands layers to POSIX threads,
 * runs the one-layer calls of cachegen_oracle.c on each, and moves their
 * results into the whole call's layout: scales, tables and lengths by index,
 * the payload by copying each layer's streams of one chunk and one of K|V to
 * their place in stream order (chunk, K|V, layer, channel). The output is
 * therefore byte for byte that of the one-thread calls, which the CPU tests
 * check.
 */
#include "cachegen_oracle.h"

#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define CHUNK 256
#define STREAM_CAP (4 * CHUNK) /* the oracle's own per-stream output bound */

/* ------------------------------------------------------------ thread pool */

typedef int (*item_fn)(void *ctx, int i);

struct pool {
    item_fn fn;
    void *ctx;
    int n;
    int next; /* next item, taken with an atomic add */
    int rc;   /* first negative code seen */
};

static void *worker(void *arg)
{
    struct pool *p = arg;
    for (;;) {
        int i = __atomic_fetch_add(&p->next, 1, __ATOMIC_RELAXED);
        if (i >= p->n)
            break;
        int rc = p->fn(p->ctx, i);
        if (rc < 0) {
            int zero = 0;
            __atomic_compare_exchange_n(&p->rc, &zero, rc, 0, __ATOMIC_RELAXED, __ATOMIC_RELAXED);
        }
    }
    return NULL;
}

/* Runs fn(ctx, i) for i in [0, n) on up to nthreads threads (the calling
 * thread is one of them). Returns 0 or the first negative code. */
static int parallel_for(int n, int nthreads, item_fn fn, void *ctx)
{
    struct pool p = {fn, ctx, n, 0, 0};
    if (nthreads > n)
        nthreads = n;
    if (nthreads < 1)
        nthreads = 1;
    pthread_t *tid = malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid)
        return OCG_ERR_ARG;
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, worker, &p) != 0)
            break;
        ++started;
    }
    worker(&p);
    for (int t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    return p.rc;
}

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

/* ------------------------------------------------------------- quantise */

struct qctx {
    int L, T, C;
    const uint8_t *bk, *bv;
    const uint16_t *kv;
    uint8_t *sym;
    uint16_t *scale;
};

static int quantize_layer(void *vc, int l)
{
    struct qctx *q = vc;
    const size_t TC = (size_t)q->T * q->C;
    uint8_t *sym = malloc(2 * TC);
    uint16_t *scale = malloc(sizeof(uint16_t) * 2 * (size_t)q->T);
    int rc = OCG_ERR_ARG;
    if (sym && scale)
        rc = ocg_quantize(1, q->T, q->C, q->bk + l, q->bv + l, q->kv + (size_t)l * 2 * TC, sym, scale);
    if (rc == 0)
        for (int k = 0; k < 2; ++k) {
            memcpy(q->sym + ((size_t)k * q->L + l) * TC, sym + k * TC, TC);
            memcpy(q->scale + ((size_t)k * q->L + l) * q->T, scale + (size_t)k * q->T,
                   sizeof(uint16_t) * (size_t)q->T);
        }
    free(sym);
    free(scale);
    return rc;
}

int ocg_quantize_mt(int L, int T, int C, const uint8_t *bins_k, const uint8_t *bins_v,
                    const uint16_t *kv, uint8_t *sym, uint16_t *scale, int nthreads)
{
    if (L < 1 || T < 1 || C < 1 || !bins_k || !bins_v || !kv || !sym || !scale)
        return OCG_ERR_ARG;
    struct qctx q = {L, T, C, bins_k, bins_v, kv, sym, scale};
    return parallel_for(L, nthreads, quantize_layer, &q);
}

/* --------------------------------------------------------------- encode */

/* One layer's one-layer call: scales [2,1,T], tables [2,1,C,A+1], lengths
 * [NC,2,C], chunk offsets [NC+1] and payload. */
struct layer_out {
    uint16_t *scale;
    int32_t *cdf;
    uint16_t *lengths;
    uint64_t *chunk_off;
    uint8_t *payload;
    int64_t bytes;
};

struct ectx {
    int L, T, C, A, NC;
    const uint8_t *bk, *bv;
    const uint8_t *widths; /* [2, L] */
    const uint16_t *kv;
    struct layer_out *out;
};

static int encode_layer(void *vc, int l)
{
    struct ectx *e = vc;
    struct layer_out *o = &e->out[l];
    const int T = e->T, C = e->C, A = e->A, NC = e->NC;
    const size_t TC = (size_t)T * C;
    const int64_t cap = (int64_t)NC * 2 * C * STREAM_CAP;
    uint8_t w2[2] = {e->widths[l], e->widths[e->L + l]};
    uint8_t *sym = malloc(2 * TC);
    uint32_t *cnt = malloc(sizeof(uint32_t) * 2 * (size_t)C * A);
    o->scale = malloc(sizeof(uint16_t) * 2 * (size_t)T);
    o->cdf = malloc(sizeof(int32_t) * 2 * (size_t)C * (A + 1));
    o->lengths = malloc(sizeof(uint16_t) * (size_t)NC * 2 * C);
    o->chunk_off = malloc(sizeof(uint64_t) * ((size_t)NC + 1));
    o->payload = malloc((size_t)cap);
    int64_t rc = OCG_ERR_ARG;
    if (!sym || !cnt || !o->scale || !o->cdf || !o->lengths || !o->chunk_off || !o->payload)
        goto done;
    if ((rc = ocg_quantize(1, T, C, e->bk + l, e->bv + l, e->kv + (size_t)l * 2 * TC, sym, o->scale)))
        goto done;
    if ((rc = ocg_histogram(1, T, C, A, sym, cnt)))
        goto done;
    if ((rc = ocg_cdf_w(1, T, C, A, w2, cnt, o->cdf)))
        goto done;
    rc = ocg_encode_w(1, T, C, A, w2, sym, o->cdf, o->payload, cap, o->lengths, o->chunk_off);
    if (rc >= 0) {
        o->bytes = rc;
        rc = 0;
    }
done:
    free(sym);
    free(cnt);
    return (int)rc;
}

static void free_layers(struct layer_out *out, int L)
{
    if (!out)
        return;
    for (int l = 0; l < L; ++l) {
        free(out[l].scale);
        free(out[l].cdf);
        free(out[l].lengths);
        free(out[l].chunk_off);
        free(out[l].payload);
    }
    free(out);
}

static int64_t sum16(const uint16_t *p, int n)
{
    int64_t s = 0;
    for (int i = 0; i < n; ++i)
        s += p[i];
    return s;
}

int64_t ocg_to_bytes_mt(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v,
                        int fmt, const uint16_t *kv, uint8_t *blob, int64_t cap, int nthreads)
{
    if (!kv || !blob || !bins_k || !bins_v)
        return OCG_ERR_ARG;
    const int64_t off_payload = ocg_blob_payload_offset(L, T, H, D, bins_k, bins_v, fmt);
    if (off_payload < 0)
        return off_payload;
    if (cap < off_payload)
        return OCG_ERR_CAPACITY;
    const int C = H * D, A = max_bins(L, bins_k, bins_v), NC = (T + CHUNK - 1) / CHUNK;
    uint8_t widths[2048];
    for (int l = 0; l < L; ++l) {
        widths[l] = (uint8_t)(fmt ? bins_k[l] : A);
        widths[L + l] = (uint8_t)(fmt ? bins_v[l] : A);
    }
    struct layer_out *out = calloc((size_t)L, sizeof *out);
    uint16_t *scale = malloc(sizeof(uint16_t) * 2 * (size_t)L * T);
    int32_t *cdf = malloc(sizeof(int32_t) * 2 * (size_t)L * C * (A + 1));
    uint16_t *lengths = malloc(sizeof(uint16_t) * (size_t)NC * 2 * L * C);
    uint64_t *chunk_off = malloc(sizeof(uint64_t) * ((size_t)NC + 1));
    int64_t rc = OCG_ERR_ARG;
    if (!out || !scale || !cdf || !lengths || !chunk_off)
        goto done;
    struct ectx e = {L, T, C, A, NC, bins_k, bins_v, widths, kv, out};
    if ((rc = parallel_for(L, nthreads, encode_layer, &e)) < 0)
        goto done;
    /* Scales, tables and lengths of layer l go to their (K|V, l) places. */
    for (int l = 0; l < L; ++l)
        for (int k = 0; k < 2; ++k) {
            memcpy(scale + ((size_t)k * L + l) * T, out[l].scale + (size_t)k * T, sizeof(uint16_t) * (size_t)T);
            memcpy(cdf + ((size_t)k * L + l) * C * (A + 1), out[l].cdf + (size_t)k * C * (A + 1),
                   sizeof(int32_t) * (size_t)C * (A + 1));
            for (int j = 0; j < NC; ++j)
                memcpy(lengths + ((size_t)j * 2 * L + (size_t)k * L + l) * C, out[l].lengths + ((size_t)j * 2 + k) * C,
                       sizeof(uint16_t) * (size_t)C);
        }
    /* Payload in stream order: chunk, then K|V, then layer. */
    int64_t off = 0;
    for (int j = 0; j < NC; ++j) {
        chunk_off[j] = (uint64_t)off;
        for (int k = 0; k < 2; ++k)
            for (int l = 0; l < L; ++l) {
                const uint16_t *ln = out[l].lengths + (size_t)j * 2 * C;
                const int64_t start = (int64_t)out[l].chunk_off[j] + (k ? sum16(ln, C) : 0);
                const int64_t n = sum16(ln + (size_t)k * C, C);
                if (off_payload + off + n > cap) {
                    rc = OCG_ERR_CAPACITY;
                    goto done;
                }
                if (n)
                    memcpy(blob + off_payload + off, out[l].payload + start, (size_t)n);
                off += n;
            }
    }
    chunk_off[NC] = (uint64_t)off;
    rc = ocg_blob_write(L, T, H, D, bins_k, bins_v, fmt, scale, cdf, lengths, chunk_off, off, blob, cap);
done:
    free_layers(out, L);
    free(scale);
    free(cdf);
    free(lengths);
    free(chunk_off);
    return rc;
}

/* --------------------------------------------------------------- decode */

struct dctx {
    int L, T, C, A, NC;
    const uint8_t *bk, *bv, *widths;
    const uint8_t *payload;
    const uint16_t *scale;
    const int32_t *cdf;
    const uint16_t *lengths;
    const uint64_t *seg_off; /* [NC, 2L] payload offset of the streams of (chunk, K|V, layer) */
    uint16_t *kv_out;
};

static int decode_layer(void *vc, int l)
{
    struct dctx *d = vc;
    const int L = d->L, T = d->T, C = d->C, A = d->A, NC = d->NC;
    const size_t TC = (size_t)T * C;
    uint8_t w2[2] = {d->widths[l], d->widths[L + l]};
    uint16_t *len = malloc(sizeof(uint16_t) * (size_t)NC * 2 * C);
    uint64_t *off = malloc(sizeof(uint64_t) * ((size_t)NC + 1));
    int32_t *cdf = malloc(sizeof(int32_t) * 2 * (size_t)C * (A + 1));
    uint16_t *scale = malloc(sizeof(uint16_t) * 2 * (size_t)T);
    uint8_t *sym = malloc(2 * TC);
    uint8_t *pay = NULL;
    int rc = OCG_ERR_ARG;
    if (!len || !off || !cdf || !scale || !sym)
        goto done;
    int64_t total = 0;
    for (int j = 0; j < NC; ++j)
        for (int k = 0; k < 2; ++k) {
            memcpy(len + ((size_t)j * 2 + k) * C, d->lengths + ((size_t)j * 2 * L + (size_t)k * L + l) * C,
                   sizeof(uint16_t) * (size_t)C);
            total += sum16(len + ((size_t)j * 2 + k) * C, C);
        }
    pay = malloc((size_t)total + 1);
    if (!pay)
        goto done;
    int64_t p = 0;
    for (int j = 0; j < NC; ++j) {
        off[j] = (uint64_t)p;
        for (int k = 0; k < 2; ++k) {
            const int64_t n = sum16(len + ((size_t)j * 2 + k) * C, C);
            if (n)
                memcpy(pay + p, d->payload + d->seg_off[(size_t)j * 2 * L + (size_t)k * L + l], (size_t)n);
            p += n;
        }
    }
    off[NC] = (uint64_t)p;
    for (int k = 0; k < 2; ++k) {
        memcpy(cdf + (size_t)k * C * (A + 1), d->cdf + ((size_t)k * L + l) * C * (A + 1),
               sizeof(int32_t) * (size_t)C * (A + 1));
        memcpy(scale + (size_t)k * T, d->scale + ((size_t)k * L + l) * T, sizeof(uint16_t) * (size_t)T);
    }
    if ((rc = ocg_decode_w(1, T, C, A, w2, pay, total, len, off, cdf, sym)))
        goto done;
    rc = ocg_dequantize(1, T, C, d->bk + l, d->bv + l, sym, scale, d->kv_out + (size_t)l * 2 * TC);
done:
    free(len);
    free(off);
    free(cdf);
    free(scale);
    free(sym);
    free(pay);
    return rc;
}

int ocg_from_bytes_mt(const uint8_t *blob, int64_t size, uint16_t *kv_out, int nthreads)
{
    int32_t dims[8];
    uint8_t bk[1024], bv[1024];
    int rc = ocg_blob_header(blob, size, dims, bk, bv, 1024);
    if (rc)
        return rc;
    if (!kv_out)
        return OCG_ERR_ARG;
    const int L = dims[0], T = dims[1], C = dims[2] * dims[3], NC = dims[5], A = dims[6], fmt = dims[7];
    uint8_t widths[2048];
    for (int l = 0; l < L; ++l) {
        widths[l] = (uint8_t)(fmt ? bk[l] : A);
        widths[L + l] = (uint8_t)(fmt ? bv[l] : A);
    }
    uint16_t *scale = malloc(sizeof(uint16_t) * 2 * (size_t)L * T);
    int32_t *cdf = malloc(sizeof(int32_t) * 2 * (size_t)L * C * (A + 1));
    uint16_t *lengths = malloc(sizeof(uint16_t) * (size_t)NC * 2 * L * C);
    uint64_t *chunk_off = malloc(sizeof(uint64_t) * ((size_t)NC + 1));
    uint64_t *seg_off = malloc(sizeof(uint64_t) * (size_t)NC * 2 * L);
    int64_t pay_off = 0;
    rc = OCG_ERR_ARG;
    if (!scale || !cdf || !lengths || !chunk_off || !seg_off)
        goto done;
    if ((rc = ocg_blob_sections(blob, size, scale, cdf, lengths, chunk_off, &pay_off)))
        goto done;
    /* Where the streams of each (chunk, K|V, layer) start; the chunk offsets
     * must agree with the lengths, and no stream may end past the payload. */
    rc = OCG_ERR_CORRUPT;
    if (chunk_off[0] != 0)
        goto done;
    const uint64_t pay_bytes = (uint64_t)(size - pay_off);
    for (int j = 0; j < NC; ++j) {
        uint64_t o = chunk_off[j];
        for (int s = 0; s < 2 * L; ++s) {
            seg_off[(size_t)j * 2 * L + s] = o;
            o += (uint64_t)sum16(lengths + ((size_t)j * 2 * L + s) * C, C);
            if (o > pay_bytes)
                goto done;
        }
        if (o != chunk_off[j + 1])
            goto done;
    }
    struct dctx d = {L, T, C, A, NC, bk, bv, widths, blob + pay_off, scale, cdf, lengths, seg_off, kv_out};
    rc = parallel_for(L, nthreads, decode_layer, &d);
done:
    free(scale);
    free(cdf);
    free(lengths);
    free(chunk_off);
    free(seg_off);
    return rc;
}
