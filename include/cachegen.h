/*
 * cachegen.h -- C ABI of libcachegen_mi355x.so, the CacheGen KV-cache codec
 * for AMD Instinct MI355X (gfx950), in hand-written HIP.
 *
 * The codec follows the LMCache CacheGen page
 *   "LMCache 中的 KV Cache 压缩：CacheGen 编解码原理、配置方式与源码解析"
 *   (0539edu.com/news/4720135), cited below as [P2 sN] for its section N:
 *   s1 QuantizationSpec (per-layer bins), s2 quantisation, s3 CDF estimation
 *   and normalisation, s4 arithmetic coding and the GPU kernels, s5 decoding
 *   and dequantisation.
 *
 * Conventions
 * -----------
 * - Every entry point returns CG_OK (0) or a negative CG_E_* code. Argument,
 *   shape and capacity checks happen on the host before anything is
 *   launched; on such an error nothing is launched.
 * - Pointers marked "device" are HIP device pointers. The caller allocates
 *   and owns every buffer, including the workspace `ws`; the library never
 *   allocates, frees or keeps state between calls, so concurrent calls on
 *   different streams with different workspaces are safe. (The one
 *   exception is cg_from_bytes_noalloc, whose workspace is a fixed device
 *   array inside the library; see there.)
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *   device work is enqueued asynchronously on it, in order.
 * - Conditions only the device can see (NaN/Inf input, a corrupt stream,
 *   a payload beyond capacity) are recorded in a status word at the start of
 *   `ws`; cg_read_status() waits for the stream and returns them as a code.
 *   Each device entry point clears that word first.
 * - Layouts are C order. bf16 tensors hold raw bf16 bit patterns.
 *   KV:      bf16  [nlayers, 2, ntokens, nheads, head_size]  ([P2 s2], [P2 s5])
 *   symbols: uint8 [2, nlayers, ntokens, C]       (K before V; C = nheads*head_size)
 *   scales:  bf16  [2, nlayers, ntokens]          (absmax over channels)
 *   cdf:     int32 [2, nlayers, C, A+1]           (A = max of all bins)
 *   lengths: uint16 [NC, 2*nlayers, C]            (NC = ceil(ntokens/256))
 *   chunk_off: uint64 [NC+1]                      (payload offset of each chunk)
 *   Streams are ordered (chunk, K|V, layer, channel); stream (j, kv, l, c)
 *   holds the symbols of tokens [256j, min(256j+256, ntokens)) of channel c.
 */
#ifndef CACHEGEN_H
#define CACHEGEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ----------------------------------------------------------------- codes */
#define CG_OK            0
#define CG_E_INVAL      (-1) /* null pointer, bad bins, bad op, bad sizes     */
#define CG_E_SHAPE      (-2) /* dimensions out of range                       */
#define CG_E_CAPACITY   (-3) /* output buffer too small                       */
#define CG_E_CORRUPT    (-4) /* malformed blob, stream, CDF or lengths        */
#define CG_E_NONFINITE  (-5) /* NaN or Inf in the KV input                    */
#define CG_E_HIP        (-6) /* a HIP runtime call failed                     */
#define CG_E_WORKSPACE  (-7) /* workspace smaller than cg_workspace_bytes()   */

#define CG_CHUNK_TOKENS     256  /* tokens per coder stream ([P2 s4])        */
#define CG_MAX_LAYERS       1024
#define CG_MIN_BINS         4
#define CG_MAX_BINS         128
#define CG_MAX_STREAM_BYTES 513  /* worst-case coded size of a 256-symbol stream */

/* Table formats ([P2 s3] normalises each table with 2^16 - (Lp - 1) and
 * the ramp arange(Lp) but leaves Lp open).
 * CG_TABLES_SHARED: every table has the call's alphabet A = the largest bins
 *   of any K or V layer (Lp = A + 1); the u16 table section is [2,L,C,A].
 * CG_TABLES_PER_LAYER: the tables of (K|V, layer) have that layer's own
 *   alphabet W = its bins (Lp = W + 1, S = 2^16 - W); the u16 table section
 *   holds, for each (K|V, layer) in turn, C tables of W entries. Same
 *   symbols, coder and output; fewer table bytes when the bins differ, which
 *   matters for short calls (at 256 tokens the tables are most of a blob). */
#define CG_TABLES_SHARED    0
#define CG_TABLES_PER_LAYER 1

/* Problem descriptor. bins_k / bins_v are HOST arrays of length nlayers
 * holding the number of quantisation bins of each layer ([P2 s1]); each must
 * be in [4, 128]. Valid shapes: 1 <= nlayers <= 1024, ntokens >= 1,
 * nheads >= 1, head_size >= 1, 2*nlayers*ntokens*nheads*head_size < 2^40 and
 * ntokens*nheads*head_size < 2^31 (one (K|V, layer) slab). table_format:
 * CG_TABLES_SHARED or CG_TABLES_PER_LAYER (else CG_E_INVAL); reserved: 0. */
typedef struct cg_desc {
    int32_t nlayers;
    int32_t ntokens;
    int32_t nheads;
    int32_t head_size;
    const uint8_t *bins_k;
    const uint8_t *bins_v;
    int32_t table_format;
    int32_t reserved;
} cg_desc;

/* Blob layout, as written by cg_to_bytes and read by cg_blob_peek. Offsets
 * are byte offsets from the start of the blob; every section is 64-byte
 * aligned and the gaps are zero. Header (little-endian): "CGMX", u16
 * version 1, u16 dtype 1 (bf16), u32 nlayers, ntokens, nheads, head_size,
 * chunk_tokens (256), nchunks, alphabet, table_format, u64 blob_size, then
 * u8 bins_k[nlayers], u8 bins_v[nlayers]. Sections: scales bf16 [2,L,T];
 * cdf u16: entries 0..W-1 of each table (entry W is 2^16), [2,L,C,A] for
 * CG_TABLES_SHARED, per (K|V, layer) C tables of its bins entries for
 * CG_TABLES_PER_LAYER; chunk_off u64 [NC+1]; lengths u16 [NC,2L,C];
 * payload. */
typedef struct cg_blob_info {
    int32_t nlayers, ntokens, nheads, head_size;
    int32_t chunk_tokens, nchunks, alphabet, table_format;
    uint64_t blob_size;      /* 0 when unknown (cg_blob_layout)           */
    uint64_t header_bytes;
    uint64_t off_scales, off_cdf, off_chunk_off, off_lengths, off_payload;
} cg_blob_info;

/* Operation selector for cg_workspace_bytes. */
enum cg_op {
    CG_OP_QUANTIZE = 0,
    CG_OP_BUILD_CDF = 1,
    CG_OP_ENCODE = 2,
    CG_OP_DECODE = 3,
    CG_OP_DEQUANTIZE = 4,
    CG_OP_TO_BYTES = 5,
    CG_OP_FROM_BYTES = 6
};

/* ------------------------------------------------------- host-only calls */

/* Message for a status code (static storage). */
const char *cg_strerror(int code);

/* Library ABI version (2: cg_desc carries the table format). */
int cg_version(void);

/* Default bins ([P2 s1]): with fewer than 10 layers every K and V layer gets
 * 32 bins; otherwise K layers 0..9 get 32 and the rest 16, V layers 0..1
 * get 32 and the rest 16. bins_k / bins_v: host arrays of nlayers bytes. */
int cg_default_bins(int32_t nlayers, uint8_t *bins_k, uint8_t *bins_v);

/* Validates a descriptor: CG_OK, CG_E_INVAL or CG_E_SHAPE. */
int cg_desc_check(const cg_desc *desc);

/* Bytes of workspace `op` needs (>= 256), or a negative code. */
int64_t cg_workspace_bytes(const cg_desc *desc, int op);

/* Upper bound of the payload cg_encode can produce: NS * 513 bytes with
 * NS = NC * 2 * nlayers * C streams. Negative code on a bad descriptor. */
int64_t cg_encode_bound(const cg_desc *desc);

/* Upper bound of the blob cg_to_bytes can produce. */
int64_t cg_blob_bound(const cg_desc *desc);

/* Section offsets of the blob for `desc` (blob_size set to 0). */
int cg_blob_layout(const cg_desc *desc, cg_blob_info *out);

/* [P2 s4, s5] The encoder output carries, beside the streams, what the
 * decoder needs to restore them (the page pickles it with the bytes and
 * lengths); this parses the header of the flat blob that replaces the pickle.
 * Parses a blob header held in HOST memory (the first n bytes of a blob; n
 * must cover the header, i.e. 48 + 2*nlayers bytes). Fills `out` and copies
 * the bins into bins_k / bins_v (host arrays of bins_cap bytes). Returns
 * CG_E_CORRUPT for a bad magic, version, dtype, shape or bins, and
 * CG_E_CAPACITY if bins_cap < nlayers. */
int cg_blob_peek(const void *header, size_t n, cg_blob_info *out, uint8_t *bins_k,
                 uint8_t *bins_v, int32_t bins_cap);

/* Waits for `stream`, then returns the device status recorded in `ws` by the
 * last entry point that used it: CG_OK, CG_E_NONFINITE, CG_E_CORRUPT or
 * CG_E_CAPACITY (CG_E_HIP if the wait or the copy fails). */
int cg_read_status(const void *ws, void *stream);

/* ------------------------------------------------------------ stage calls */

/* [P2 s2] Quantise. For each (kv, layer, token) row: m = max |x| over the C
 * channels, M = bins//2 - 1 of that layer, q = round_half_even(x*(M/m) + M)
 * in fp32 with each operation rounded separately, clamped to [0, 2M]; a row
 * with m = 0 gives q = M. kv: device bf16 [L,2,T,H,D]; sym: device uint8
 * [2,L,T,C]; scale: device bf16 [2,L,T] (m, exact). NaN/Inf input records
 * CG_E_NONFINITE. */
int cg_quantize(const cg_desc *desc, const void *kv, uint8_t *sym, uint16_t *scale, void *ws,
                size_t ws_bytes, void *stream);

/* [P2 s3] Histogram of each (kv, layer, channel) over all ntokens tokens and
 * its integer CDF: cdf[k] = round_half_even(cum[k] * (2^16 - W) / T) + k for
 * k = 0..W, so cdf[0] = 0, cdf[W] = 2^16 and every symbol keeps frequency
 * >= 1, with W the table's width (A, or the layer's bins for
 * CG_TABLES_PER_LAYER; entries W+1..A then hold 2^16). sym: device uint8
 * [2,L,T,C] (every symbol < W); cdf: device int32 [2,L,C,A+1]. */
int cg_build_cdf(const cg_desc *desc, const uint8_t *sym, int32_t *cdf, void *ws,
                 size_t ws_bytes, void *stream);

/* [P2 s4] Range-code every stream (byte-wise 32-bit range coder, 16-bit
 * tables) and concatenate them in stream order. payload: device buffer of
 * `cap` bytes (cap >= cg_encode_bound() can never overflow; a smaller cap
 * records CG_E_CAPACITY if exceeded); lengths: device uint16 [NC,2L,C]
 * bytes per stream; chunk_off: device uint64 [NC+1], chunk_off[NC] is the
 * payload size. cdf: int32 [2,L,C,A+1] tables of the desc's format (as
 * cg_build_cdf writes them); a symbol at or past its table's width records
 * CG_E_CORRUPT. */
int cg_encode(const cg_desc *desc, const uint8_t *sym, const int32_t *cdf, uint8_t *payload,
              size_t cap, uint16_t *lengths, uint64_t *chunk_off, void *ws, size_t ws_bytes,
              void *stream);

/* [P2 s5] Decode every stream: its offset is the chunk offset plus the prefix
 * sum of the lengths before it in the chunk; symbols are found by search in
 * the CDF. Bytes past a stream's length read as zero. payload_bytes bounds
 * every read. A malformed stream, or chunk offsets that disagree with the
 * lengths, record CG_E_CORRUPT. sym: device uint8 [2,L,T,C]. */
int cg_decode(const cg_desc *desc, const uint8_t *payload, size_t payload_bytes,
              const uint16_t *lengths, const uint64_t *chunk_off, const int32_t *cdf,
              uint8_t *sym, void *ws, size_t ws_bytes, void *stream);

/* [P2 s5] Dequantise: x = bf16_round((q - M) / M * m) with fp32 division and
 * product. sym: device uint8 [2,L,T,C]; scale: device bf16 [2,L,T];
 * kv_out: device bf16 [L,2,T,H,D]. */
int cg_dequantize(const cg_desc *desc, const uint8_t *sym, const uint16_t *scale, void *kv_out,
                  void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------ whole-blob calls */

/* [P2 s2-s4] to_bytes (the page's CacheGenSerializer.to_bytes on
 * [L,2,T,H,D]): split into K and V, quantise, histogram and CDF, range-code
 * the 256-token streams and serialise. The whole encode path on bf16 KV, writing the blob
 * described at cg_blob_info into `blob` (device, `cap` bytes; cap >=
 * cg_blob_bound() can never overflow). The blob size is written to
 * *blob_size_dev (device uint64) and into the header. */
int cg_to_bytes(const cg_desc *desc, const void *kv, uint8_t *blob, size_t cap,
                uint64_t *blob_size_dev, void *ws, size_t ws_bytes, void *stream);

/* [P2 s5] from_bytes (the page's CacheGenDeserializer.from_bytes): stream
 * offsets from the prefix sums of the lengths, CDF-driven decode, (t - M) / M
 * * max and the stack back to [L,2,T,H,D] in bf16. The whole decode path. `desc` must be the one cg_blob_peek
 * returned for this blob (bins included); blob: device; blob_size: its size
 * in bytes; kv_out: device bf16 [L,2,T,H,D]. */
int cg_from_bytes(const cg_desc *desc, const uint8_t *blob, size_t blob_size, void *kv_out,
                  void *ws, size_t ws_bytes, void *stream);

/* from_bytes for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same decode and output as cg_from_bytes, with no workspace argument and no
 * allocation. Its workspace is a fixed 4 MiB device array inside the library,
 * one per GPU (the current device's), kept until the process ends; calls
 * whose cg_workspace_bytes(desc, CG_OP_FROM_BYTES) exceeds 4 MiB return
 * CG_E_WORKSPACE before launching anything (the 32-layer, 1024-channel,
 * 32768-token call needs about 1.05 MiB). status_dev: caller-owned device
 * uint32 (4-byte aligned) that the call clears and then sets to the status
 * bits; cg_read_status(status_dev, stream) turns it into a code. Every call
 * on a GPU shares that GPU's array: calls that overlap in time on one GPU
 * (different streams or threads) race and must not be made. The stream's
 * device must be the current device. */
int cg_from_bytes_noalloc(const cg_desc *desc, const uint8_t *blob, size_t blob_size, void *kv_out,
                          uint32_t *status_dev, void *stream);

/* from_bytes of a range of chunks: decodes chunks [chunk_begin, chunk_end)
 * (tokens [256*chunk_begin, min(256*chunk_end, T))) of a blob whose bytes
 * have arrived only up to blob_size: the header and sections before the
 * payload, and the payload up to the end of chunk chunk_end - 1
 * (off_payload + chunk_off[chunk_end] bytes). Those tokens of kv_out
 * [L,2,T,H,D] are written as cg_from_bytes writes them; the other tokens are
 * left untouched. With this a receiver decodes chunk j while chunk j + 1 is
 * still in transfer: the stream decomposition of [P2 s4] makes every chunk
 * decodable on its own once its lengths and tables are known ([P2 s5]).
 * 0 <= chunk_begin < chunk_end <= nchunks, else CG_E_INVAL. A chunk of the
 * range whose chunk offsets disagree with its lengths or reach beyond
 * blob_size records CG_E_CORRUPT. Bytes of the blob beyond blob_size are
 * never read, so they may be in transfer meanwhile.
 * Workspace: cg_workspace_bytes(CG_OP_FROM_BYTES); calls that overlap in time
 * need workspaces of their own. */
int cg_from_bytes_chunks(const cg_desc *desc, const uint8_t *blob, size_t blob_size, int32_t chunk_begin,
                         int32_t chunk_end, void *kv_out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- batches
 * Many small calls of one shape, as LMCache makes them (one to_bytes per KV
 * chunk of 64..768 tokens, each with its own tables, [P2 benchmark]), in one
 * launch sequence. Call b's KV is kv + b * (its element count), i.e. kv is
 * [batch, L, 2, T, H, D]; call b's blob is written at blobs + b * blob_stride
 * and is byte for byte the blob cg_to_bytes writes for that call alone; its
 * size goes to blob_sizes_dev[b] (device uint64) and into its header.
 * blob_stride: a multiple of 8, >= the header and sections (cg_blob_layout's
 * off_payload); >= cg_blob_bound() can never overflow. With a smaller
 * stride a call that does not fit records CG_E_CAPACITY: blob_sizes_dev then
 * holds the size every call needs, and the blobs are not usable. Blobs
 * 16-byte aligned with a stride that is a multiple of 16 are the fast case
 * (the quantiser then writes the tables in place itself). Workspace:
 * cg_workspace_bytes_batch(desc, batch, blob_stride, CG_OP_TO_BYTES /
 * CG_OP_FROM_BYTES). batch * nlayers <= 32767.
 *
 * cg_from_bytes_batch decodes such a batch of blobs (all with this desc) to
 * kv_out [batch, L, 2, T, H, D]; blob_sizes_dev holds each blob's size. A
 * blob whose header, size or chunk offsets disagree with desc or with its
 * lengths records CG_E_CORRUPT; its tokens are then undefined, those of the
 * other blobs are not affected, and no read leaves the blob's stride.
 * Both calls read and write every blob's sections in place: the batch moves
 * no blob bytes beyond those of the calls themselves. */
int64_t cg_workspace_bytes_batch(const cg_desc *desc, int32_t batch, size_t blob_stride, int op);
int cg_to_bytes_batch(const cg_desc *desc, int32_t batch, const void *kv, uint8_t *blobs, size_t blob_stride,
                      uint64_t *blob_sizes_dev, void *ws, size_t ws_bytes, void *stream);
int cg_from_bytes_batch(const cg_desc *desc, int32_t batch, const uint8_t *blobs, size_t blob_stride,
                        const uint64_t *blob_sizes_dev, void *kv_out, void *ws, size_t ws_bytes, void *stream);

/* from_bytes into a paged KV cache (the layout a serving engine keeps: fixed
 * blocks of block_size tokens, located through a block table), as the decode
 * step of a remote read that feeds such an engine. Same decode and
 * dequantisation as cg_from_bytes ([P2 s5]); only the destination of each
 * token row differs: element (l, kv, t, h, d) of the [L,2,T,H,D] result goes
 * to the bf16 element
 *   kv_cache[l*layer_stride + kv*kv_stride
 *            + (block_table[t / block_size] * block_size + t % block_size) * C
 *            + h*D + d]
 * (strides in elements). kv_cache: device bf16, caller-owned, large enough
 * for every address above; block_table: device int32 [ceil(T/block_size)],
 * each entry in [0, num_blocks); block_size: a power of two >= 4; one
 * (layer, K|V) region of num_blocks+1 blocks must span < 4 GiB (CG_E_SHAPE
 * otherwise). Rows of blocks that are not in the table are left untouched.
 * A table entry outside [0, num_blocks) records CG_E_CORRUPT and the rows of
 * that block are not written. Workspace: cg_workspace_bytes(CG_OP_FROM_BYTES). */
int cg_from_bytes_paged(const cg_desc *desc, const uint8_t *blob, size_t blob_size, void *kv_cache,
                        int64_t layer_stride, int64_t kv_stride, int32_t block_size,
                        const int32_t *block_table, int32_t num_blocks, void *ws, size_t ws_bytes,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CACHEGEN_H */
