/*
 * CacheGen KV-cache codec -- CPU oracle, public declarations.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path includes, links or
 * calls this. It is used by tests/, by the smoke check and by the CPU baseline
 * leg of the benchmark, to produce the expected result of every stage.
 *
 * Sources:
 *   [P2]  "LMCache 中的 KV Cache 压缩：CacheGen 编解码原理、配置方式与源码解析"
 *         (0539edu.com/news/4720135), sections 1 (QuantizationSpec),
 *         2 (quantisation), 3 (CDF estimation and normalisation),
 *         4 (arithmetic coding and GPU kernels), 5 (decoding and dequantisation).
 *
 * All tensors are plain host arrays in C order. bf16 values are passed as
 * their uint16 bit patterns. Every function returns 0 (or a size) on success
 * and a negative code on failure; the codes are listed below.
 */
#ifndef CACHEGEN_ORACLE_H
#define CACHEGEN_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OCG_ERR_ARG       (-1) /* bad argument or shape                        */
#define OCG_ERR_CAPACITY  (-3) /* output buffer too small                      */
#define OCG_ERR_CORRUPT   (-4) /* malformed stream, header or lengths          */
#define OCG_ERR_NONFINITE (-5) /* NaN or Inf in the input                      */

/* Default per-layer bins ([P2] section 1): fewer than 10 layers -> 32 for
 * every K and V layer; otherwise K gets 32 for layers 0..9 and 16 after,
 * V gets 32 for layers 0..1 and 16 after. */
int ocg_default_bins(int nlayers, uint8_t *bins_k, uint8_t *bins_v);

/* Quantise ([P2] section 2). kv: bf16 [L,2,T,C]; sym: uint8 [2,L,T,C];
 * scale: bf16 [2,L,T] (per (K|V, layer, token) absmax over channels). */
int ocg_quantize(int L, int T, int C, const uint8_t *bins_k, const uint8_t *bins_v,
                 const uint16_t *kv, uint8_t *sym, uint16_t *scale);

/* Symbol counts over all T tokens ([P2] section 3). cnt: uint32 [2,L,C,A]. */
int ocg_histogram(int L, int T, int C, int A, const uint8_t *sym, uint32_t *cnt);

/* Integer CDF ([P2] section 3): cdf: int32 [2,L,C,A+1],
 * cdf[k] = round_half_even(cum[k] * (2^16 - A) / T) + k. */
int ocg_cdf(int L, int T, int C, int A, const uint32_t *cnt, int32_t *cdf);

/* The same with a width per (kv, layer) table (widths [2, L], each in
 * [2, A]): table (kv, l, c) has widths[kv*L + l] symbols and is normalised
 * with 2^16 - that width; entries past its end hold 2^16. */
int ocg_cdf_w(int L, int T, int C, int A, const uint8_t *widths, const uint32_t *cnt, int32_t *cdf);

/* Range-code one stream of n symbols with the table cdf[0..A]. Returns the
 * number of bytes written to out, or a negative code. */
int64_t ocg_encode_stream(const uint8_t *sym, int n, const int32_t *cdf, int A,
                          uint8_t *out, int64_t cap);

/* Decode n symbols from a stream of len bytes. Returns 0 or OCG_ERR_CORRUPT. */
int ocg_decode_stream(const uint8_t *in, int64_t len, int n, const int32_t *cdf, int A,
                      uint8_t *sym);

/* Encode every stream ([P2] section 4). Streams are (chunk j, kv, layer,
 * channel) in that nesting order, chunk j covering tokens
 * [256j, min(256j+256, T)). lengths: uint16 [NC,2L,C]; chunk_off: uint64
 * [NC+1] payload offsets of each chunk; payload: concatenated streams.
 * Returns the payload size or a negative code. */
int64_t ocg_encode(int L, int T, int C, int A, const uint8_t *sym, const int32_t *cdf,
                   uint8_t *payload, int64_t cap, uint16_t *lengths, uint64_t *chunk_off);
int64_t ocg_encode_w(int L, int T, int C, int A, const uint8_t *widths, const uint8_t *sym,
                     const int32_t *cdf, uint8_t *payload, int64_t cap, uint16_t *lengths,
                     uint64_t *chunk_off);

/* Inverse of ocg_encode ([P2] section 5): offsets of each stream are the
 * chunk offset plus the prefix sum of the lengths. */
int ocg_decode(int L, int T, int C, int A, const uint8_t *payload, int64_t payload_bytes,
               const uint16_t *lengths, const uint64_t *chunk_off, const int32_t *cdf,
               uint8_t *sym);
int ocg_decode_w(int L, int T, int C, int A, const uint8_t *widths, const uint8_t *payload,
                 int64_t payload_bytes, const uint16_t *lengths, const uint64_t *chunk_off,
                 const int32_t *cdf, uint8_t *sym);

/* Dequantise ([P2] section 5): x = (q - M) / M * scale with M = bins//2 - 1
 * of the element's layer, as two separately rounded fp32 operations (the
 * quotient, then the product), then rounded to bf16 (nearest, ties to even).
 * out: bf16 [L,2,T,C]. */
int ocg_dequantize(int L, int T, int C, const uint8_t *bins_k, const uint8_t *bins_v,
                   const uint8_t *sym, const uint16_t *scale, uint16_t *out);

/* Whole blob. Layout (little-endian; every section starts on a 64-byte
 * boundary, gaps are zero):
 *   header  : "CGMX", u16 version 1, u16 dtype 1 (bf16), u32 L, T, H, D,
 *             chunk (256), NC, A, reserved 0, u64 blob size, u8 bins_k[L],
 *             u8 bins_v[L];
 *   scales  : bf16 [2,L,T];
 *   cdf     : u16 [2,L,C,A] (entries 0..A-1; entry A is 2^16);
 *   offsets : u64 [NC+1] chunk offsets into the payload;
 *   lengths : u16 [NC,2L,C];
 *   payload : the streams.
 * Returns the blob size or a negative code. */
int64_t ocg_blob_bound(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v);
int64_t ocg_to_bytes(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v,
                     const uint16_t *kv, uint8_t *blob, int64_t cap);
/* The same for table format fmt: 0 = one alphabet A for every table, 1 = the
 * tables of (kv, layer) have the bins of that layer; the u16 table section is
 * then ragged (C tables of width W per slab, slab after slab) and header
 * bytes 36..39 hold fmt. */
int64_t ocg_to_bytes_fmt(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v,
                         int fmt, const uint16_t *kv, uint8_t *blob, int64_t cap);
/* Parses the header; dims = {L, T, H, D, chunk, NC, A}. */
int ocg_blob_header(const uint8_t *blob, int64_t size, int32_t dims[8], uint8_t *bins_k,
                    uint8_t *bins_v, int max_layers);
int ocg_from_bytes(const uint8_t *blob, int64_t size, uint16_t *kv_out);

/* The blob's two halves, for drivers that compute the stages themselves.
 * ocg_blob_write: header and every section but the payload (the pay payload
 * bytes sit at the offset ocg_blob_payload_offset returns); returns the blob
 * size. ocg_blob_sections: the sections of a blob whose header is valid, into
 * arrays sized by that header (cdf int32 [2,L,C,A+1], 2^16 past each table's
 * width); checks the tables and the last chunk offset. */
int64_t ocg_blob_write(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v, int fmt,
                       const uint16_t *scale, const int32_t *cdf, const uint16_t *lengths,
                       const uint64_t *chunk_off, int64_t pay, uint8_t *blob, int64_t cap);
int64_t ocg_blob_payload_offset(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v,
                                int fmt);
int ocg_blob_sections(const uint8_t *blob, int64_t size, uint16_t *scale, int32_t *cdf, uint16_t *lengths,
                      uint64_t *chunk_off, int64_t *payload_off);

/* Multi-threaded drivers (cachegen_oracle_mt.c). They run the single-layer
 * calls above on each layer's K and V slabs on nthreads POSIX threads and
 * move the results into place; the arithmetic is that of the calls above,
 * unchanged, so the output is byte for byte that of the one-thread calls. */
int ocg_quantize_mt(int L, int T, int C, const uint8_t *bins_k, const uint8_t *bins_v,
                    const uint16_t *kv, uint8_t *sym, uint16_t *scale, int nthreads);
int64_t ocg_to_bytes_mt(int L, int T, int H, int D, const uint8_t *bins_k, const uint8_t *bins_v,
                        int fmt, const uint16_t *kv, uint8_t *blob, int64_t cap, int nthreads);
int ocg_from_bytes_mt(const uint8_t *blob, int64_t size, uint16_t *kv_out, int nthreads);

#ifdef __cplusplus
}
#endif

#endif
