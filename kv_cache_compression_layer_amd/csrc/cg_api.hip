// C ABI of libcachegen_mi355x.so: argument checks, sizes, the blob header and
// the composition of the kernels of each entry point. See include/cachegen.h
// for the contract of every call.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "cg_internal.hpp"

using namespace cg;

// Workspace of cg_from_bytes_noalloc: file-scope device memory, one copy per
// GPU the library runs on, held until the process ends. Host code never
// passes this name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the device address that hipGetSymbolAddress returns for
// the current device.
constexpr size_t kNoAllocScratchBytes = 4u << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr uint64_t kAlign = 64;       // blob section alignment
constexpr uint64_t kWsAlign = 256;    // workspace region alignment
constexpr uint32_t kHdrFixed = 48;    // fixed part of the blob header

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

int bins_valid(const uint8_t *b, int L) {
    for (int l = 0; l < L; ++l)
        if (b[l] < CG_MIN_BINS || b[l] > CG_MAX_BINS) return 0;
    return 1;
}

// Validates the descriptor and derives the sizes of the call.
int make_dims(const cg_desc *desc, Dims &d) {
    if (!desc || !desc->bins_k || !desc->bins_v) return CG_E_INVAL;
    if (desc->nlayers < 1 || desc->nlayers > CG_MAX_LAYERS || desc->ntokens < 1 ||
        desc->nheads < 1 || desc->head_size < 1)
        return CG_E_SHAPE;
    const int64_t C = (int64_t)desc->nheads * desc->head_size;
    if (C > (1 << 20)) return CG_E_SHAPE;  // keeps every grid dimension in range
    if (!bins_valid(desc->bins_k, desc->nlayers) || !bins_valid(desc->bins_v, desc->nlayers))
        return CG_E_INVAL;
    d.L = desc->nlayers;
    d.Lc = d.L;
    d.cstride = 0;
    d.T = desc->ntokens;
    d.H = desc->nheads;
    d.D = desc->head_size;
    d.C = (int)C;
    int A = 0;
    for (int l = 0; l < d.L; ++l) A = A > desc->bins_k[l] ? A : desc->bins_k[l];
    for (int l = 0; l < d.L; ++l) A = A > desc->bins_v[l] ? A : desc->bins_v[l];
    d.A = A;
    if (desc->table_format != CG_TABLES_SHARED && desc->table_format != CG_TABLES_PER_LAYER) return CG_E_INVAL;
    d.fmt = desc->table_format;
    d.tab_entries = 0;
    d.wmin = A;
    for (int l = 0; l < d.L; ++l) {
        d.tab_entries += d.fmt ? (int64_t)desc->bins_k[l] + desc->bins_v[l] : 2LL * A;
        if (d.fmt) d.wmin = std::min<int>(d.wmin, std::min(desc->bins_k[l], desc->bins_v[l]));
    }
    d.NC = (d.T + kChunk - 1) / kChunk;
    d.CB = (d.C + 63) / 64;
    d.N = 2LL * d.L * d.T * d.C;
    d.NS = (int64_t)d.NC * 2 * d.L * d.C;
    d.tiles = (int64_t)d.NC * 2 * d.L * d.CB;
    if (d.N >= (1LL << 40) || d.tiles >= (1LL << 31)) return CG_E_SHAPE;
    // Kernels address one (K|V, layer) slab with 32-bit byte offsets.
    if ((int64_t)d.T * d.C >= (1LL << 31)) return CG_E_SHAPE;
    return CG_OK;
}

void make_max_table(const cg_desc *desc, const Dims &d, MaxTable &mt) {
    memset(&mt, 0, sizeof mt);
    for (int l = 0; l < desc->nlayers; ++l) {
        mt.bins[0][l] = desc->bins_k[l];
        mt.bins[1][l] = desc->bins_v[l];
    }
    mt.per_layer = d.fmt == CG_TABLES_PER_LAYER;
    mt.A = d.A;
}

// Sizes of a batch: one call (d) and the call of batch * L layers that runs
// it (vd), whose blob sections lie stride bytes apart per call.
constexpr int kMaxBatchLayers = 32767;  // grid y-dimension of the per-slab kernels is 2 * layers

int make_dims_batch(const cg_desc *desc, int batch, uint64_t stride, Dims &d, Dims &vd) {
    int rc = make_dims(desc, d);
    if (rc) return rc;
    if (batch < 1 || (int64_t)batch * d.L > kMaxBatchLayers) return CG_E_SHAPE;
    vd = d;
    vd.L = batch * d.L;
    vd.Lc = d.L;
    vd.cstride = stride;
    vd.tab_entries = (int64_t)batch * d.tab_entries;
    vd.N = 2LL * vd.L * vd.T * vd.C;
    vd.NS = (int64_t)vd.NC * 2 * vd.L * vd.C;
    vd.tiles = (int64_t)vd.NC * 2 * vd.L * vd.CB;
    if (vd.N >= (1LL << 40) || vd.tiles >= (1LL << 31)) return CG_E_SHAPE;
    return CG_OK;
}

BlobLayout blob_layout(const Dims &d) {
    BlobLayout b;
    b.header_bytes = align_up(kHdrFixed + 2ull * d.L, kAlign);
    b.off_scales = b.header_bytes;
    b.off_cdf = b.off_scales + align_up(4ull * d.L * d.T, kAlign);
    b.off_chunk_off = b.off_cdf + align_up(2ull * d.C * (uint64_t)d.tab_entries, kAlign);
    b.off_lengths = b.off_chunk_off + align_up(8ull * (d.NC + 1), kAlign);
    b.off_payload = b.off_lengths + align_up(4ull * d.NC * d.L * d.C, kAlign);
    return b;
}

// Workspace regions (byte offsets; 0 = unused). Region 0 is the WsHeader.
struct WsLayout {
    uint64_t counts = 0, tile_sum = 0, tile_mode = 0, tile_off = 0, chunk_total = 0, staging = 0,
             sym = 0, scan = 0, wpre = 0;
    uint64_t clear_end = kWsAlign;  // bytes from 0 that must start zeroed
    uint64_t total = kWsAlign;
};

WsLayout ws_layout(const Dims &d, int op) {
    WsLayout w;
    uint64_t off = kWsAlign;
    auto take = [&](uint64_t bytes) {
        const uint64_t o = off;
        off += align_up(bytes, kWsAlign);
        return o;
    };
    switch (op) {
    case CG_OP_BUILD_CDF:
        w.counts = take(4ull * 2 * d.L * d.C * d.A);
        w.clear_end = off;
        break;
    case CG_OP_ENCODE:
        w.tile_sum = take(4ull * d.tiles);
        w.tile_mode = take((uint64_t)d.tiles);
        w.tile_off = take(8ull * d.tiles);
        w.chunk_total = take(8ull * d.NC * ncalls(d));
        w.staging = take(encode_staging_bytes(d));
        w.scan = take(tile_scan_tmp_bytes(d));
        break;
    case CG_OP_DECODE:
        w.tile_off = take(8ull * d.tiles);
        w.scan = take(tile_scan_tmp_bytes(d));
        break;
    case CG_OP_FROM_BYTES:
        w.tile_off = take(8ull * d.tiles);
        w.scan = take(tile_scan_tmp_bytes(d));
        w.wpre = take(4ull * (2 * d.L + 1));
        break;
    case CG_OP_TO_BYTES:
        w.counts = take(4ull * 2 * d.L * d.C * d.A);
        w.clear_end = off;
        w.tile_sum = take(4ull * d.tiles);
        w.tile_mode = take((uint64_t)d.tiles);
        w.tile_off = take(8ull * d.tiles);
        w.chunk_total = take(8ull * d.NC * ncalls(d));
        w.staging = take(encode_staging_bytes(d));
        w.sym = take((uint64_t)d.N);
        w.scan = take(tile_scan_tmp_bytes(d));
        w.wpre = take(4ull * (2 * d.L + 1));
        break;
    default:
        break;
    }
    w.total = off;
    return w;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? CG_OK : CG_E_HIP; }

// Common prologue of the device entry points.
int prologue(const cg_desc *desc, int op, void *ws, size_t ws_bytes, Dims &d, WsLayout &w) {
    int rc = make_dims(desc, d);
    if (rc) return rc;
    w = ws_layout(d, op);
    if (!ws) return CG_E_INVAL;
    if ((uint64_t)ws_bytes < w.total) return CG_E_WORKSPACE;
    if ((uintptr_t)ws % kWsAlign) return CG_E_INVAL;
    return CG_OK;
}

int clear_ws(void *ws, const WsLayout &w, hipStream_t s) {
    return hip_rc(launch_fill_u32(reinterpret_cast<uint32_t *>(ws), 0u, (int64_t)(w.clear_end / 4), s));
}

template <class T>
T *at(void *base, uint64_t off) {
    return reinterpret_cast<T *>(reinterpret_cast<uint8_t *>(base) + off);
}

void put_le(uint8_t *p, uint64_t v, int n) {
    for (int i = 0; i < n; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

uint64_t get_le(const uint8_t *p, int n) {
    uint64_t v = 0;
    for (int i = n - 1; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}

// Header bytes of a blob (the size field, bytes 40..47, is written by the
// encoder once the payload size is known).
void make_header(const cg_desc *desc, const Dims &d, const BlobLayout &b, HeaderBytes &hb) {
    memset(&hb, 0, sizeof hb);
    hb.n = (uint32_t)b.header_bytes;
    memcpy(hb.b, "CGMX", 4);
    put_le(hb.b + 4, 1, 2);
    put_le(hb.b + 6, 1, 2);
    put_le(hb.b + 8, (uint64_t)d.L, 4);
    put_le(hb.b + 12, (uint64_t)d.T, 4);
    put_le(hb.b + 16, (uint64_t)d.H, 4);
    put_le(hb.b + 20, (uint64_t)d.D, 4);
    put_le(hb.b + 24, (uint64_t)kChunk, 4);
    put_le(hb.b + 28, (uint64_t)d.NC, 4);
    put_le(hb.b + 32, (uint64_t)d.A, 4);
    put_le(hb.b + 36, (uint64_t)d.fmt, 4);
    memcpy(hb.b + kHdrFixed, desc->bins_k, (size_t)d.L);
    memcpy(hb.b + kHdrFixed + d.L, desc->bins_v, (size_t)d.L);
}

void fill_info(const Dims &d, const BlobLayout &b, cg_blob_info *out) {
    out->nlayers = d.L;
    out->ntokens = d.T;
    out->nheads = d.H;
    out->head_size = d.D;
    out->chunk_tokens = kChunk;
    out->nchunks = d.NC;
    out->alphabet = d.A;
    out->table_format = d.fmt;
    out->blob_size = 0;
    out->header_bytes = b.header_bytes;
    out->off_scales = b.off_scales;
    out->off_cdf = b.off_cdf;
    out->off_chunk_off = b.off_chunk_off;
    out->off_lengths = b.off_lengths;
    out->off_payload = b.off_payload;
}

// Quantise, tables and range coding of one call (or of a batch run as one
// call) into the blob sections `scales`, `wire` and `o`; the workspace is
// ws_layout(d, CG_OP_TO_BYTES). When one quantiser block covers a whole
// (K|V, layer) slab it builds the tables itself (no counts to clear, no
// k_cdf); the encoder reads the u16 tables from the blob. status_zeroed:
// the status word has been zeroed on the stream already (by the blob
// header's kernel), so only the counts, if used, need clearing.
int encode_call(const Dims &d, const MaxTable &mt, const void *kv, uint16_t *scales, uint16_t *wire,
                const EncodeOut &o, void *ws, const WsLayout &w, hipStream_t s, bool status_zeroed) {
    uint32_t *status = at<uint32_t>(ws, 0);
    uint32_t *counts = at<uint32_t>(ws, w.counts);
    uint32_t *wpre = d.fmt == CG_TABLES_PER_LAYER ? at<uint32_t>(ws, w.wpre) : nullptr;
    uint8_t *sym = at<uint8_t>(ws, w.sym);
    const uint16_t *kv16 = reinterpret_cast<const uint16_t *>(kv);
    const bool qh = quantize_hist_fits(d, kv, sym);
    const bool fused = qh && quantize_hist_fuses_cdf(d, wire);
    const bool packed = qh && encode_packs(d, mt);
    int rc = CG_OK;
    if (!(fused && status_zeroed) &&
        (rc = hip_rc(launch_fill_u32(status, 0u, (int64_t)((fused ? kWsAlign : w.clear_end) / 4), s))))
        return rc;
    if (wpre && (rc = hip_rc(launch_table_prefix(d, mt, wpre, s)))) return rc;
    if (qh) {
        rc = hip_rc(
            launch_quantize_hist(d, mt, kv16, sym, scales, counts, fused ? wire : nullptr, wpre, status, packed,
                                 packed && encode_nibbles(d, mt), s));
        if (rc) return rc;
    } else {
        if ((rc = hip_rc(launch_quantize(d, mt, kv16, sym, scales, status, s)))) return rc;
        if ((rc = hip_rc(launch_histogram(d, sym, counts, status, s)))) return rc;
    }
    if (!fused && (rc = hip_rc(launch_cdf(d, mt, counts, nullptr, wire, wpre, status, s)))) return rc;
    EncodeWs ew{at<WsHeader>(ws, 0),         at<uint32_t>(ws, w.tile_sum), at<uint8_t>(ws, w.tile_mode),
                at<uint64_t>(ws, w.tile_off), at<uint64_t>(ws, w.chunk_total),
                at<uint8_t>(ws, w.staging),   at<uint64_t>(ws, w.scan)};
    return hip_rc(launch_encode(d, mt, sym, nullptr, wire, wpre, o, ew, true, packed, s));
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CG_E_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CG_E_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CG_OK;
}

}  // namespace

extern "C" {

const char *cg_strerror(int code) {
    switch (code) {
    case CG_OK: return "ok";
    case CG_E_INVAL: return "invalid argument";
    case CG_E_SHAPE: return "shape out of range";
    case CG_E_CAPACITY: return "output buffer too small";
    case CG_E_CORRUPT: return "corrupt blob, stream, table or lengths";
    case CG_E_NONFINITE: return "non-finite value in the KV input";
    case CG_E_HIP: return "HIP runtime error";
    case CG_E_WORKSPACE: return "workspace too small";
    default: return "unknown status";
    }
}

int cg_version(void) { return 2; }

int cg_default_bins(int32_t nlayers, uint8_t *bins_k, uint8_t *bins_v) {
    if (!bins_k || !bins_v) return CG_E_INVAL;
    if (nlayers < 1 || nlayers > CG_MAX_LAYERS) return CG_E_SHAPE;
    for (int l = 0; l < nlayers; ++l) {
        if (nlayers < 10) {
            bins_k[l] = bins_v[l] = 32;
        } else {
            bins_k[l] = l < 10 ? 32 : 16;
            bins_v[l] = l < 2 ? 32 : 16;
        }
    }
    return CG_OK;
}

int cg_desc_check(const cg_desc *desc) {
    Dims d;
    return make_dims(desc, d);
}

int64_t cg_workspace_bytes(const cg_desc *desc, int op) {
    Dims d;
    const int rc = make_dims(desc, d);
    if (rc) return rc;
    if (op < CG_OP_QUANTIZE || op > CG_OP_FROM_BYTES) return CG_E_INVAL;
    return (int64_t)ws_layout(d, op).total;
}

int64_t cg_encode_bound(const cg_desc *desc) {
    Dims d;
    const int rc = make_dims(desc, d);
    if (rc) return rc;
    return d.NS * CG_MAX_STREAM_BYTES;
}

int64_t cg_blob_bound(const cg_desc *desc) {
    Dims d;
    const int rc = make_dims(desc, d);
    if (rc) return rc;
    return (int64_t)blob_layout(d).off_payload + d.NS * CG_MAX_STREAM_BYTES;
}

int cg_blob_layout(const cg_desc *desc, cg_blob_info *out) {
    Dims d;
    const int rc = make_dims(desc, d);
    if (rc) return rc;
    if (!out) return CG_E_INVAL;
    fill_info(d, blob_layout(d), out);
    return CG_OK;
}

int cg_blob_peek(const void *header, size_t n, cg_blob_info *out, uint8_t *bins_k,
                 uint8_t *bins_v, int32_t bins_cap) {
    if (!header || !out || !bins_k || !bins_v) return CG_E_INVAL;
    const uint8_t *h = reinterpret_cast<const uint8_t *>(header);
    if (n < kHdrFixed || memcmp(h, "CGMX", 4) != 0 || get_le(h + 4, 2) != 1 || get_le(h + 6, 2) != 1)
        return CG_E_CORRUPT;
    const uint64_t L = get_le(h + 8, 4);
    if (L < 1 || L > CG_MAX_LAYERS || n < kHdrFixed + 2 * L) return CG_E_CORRUPT;
    if ((int64_t)L > bins_cap) return CG_E_CAPACITY;
    memcpy(bins_k, h + kHdrFixed, L);
    memcpy(bins_v, h + kHdrFixed + L, L);
    const uint64_t T = get_le(h + 12, 4), H = get_le(h + 16, 4), D = get_le(h + 20, 4);
    if (T < 1 || T > 0x7FFFFFFF || H < 1 || H > 0x7FFFFFFF || D < 1 || D > 0x7FFFFFFF)
        return CG_E_CORRUPT;
    const uint64_t fmt = get_le(h + 36, 4);
    if (fmt != CG_TABLES_SHARED && fmt != CG_TABLES_PER_LAYER) return CG_E_CORRUPT;
    cg_desc desc = {(int32_t)L, (int32_t)T, (int32_t)H, (int32_t)D, bins_k, bins_v, (int32_t)fmt, 0};
    Dims d;
    if (make_dims(&desc, d) != CG_OK) return CG_E_CORRUPT;
    if (get_le(h + 24, 4) != (uint64_t)kChunk || get_le(h + 28, 4) != (uint64_t)d.NC ||
        get_le(h + 32, 4) != (uint64_t)d.A)
        return CG_E_CORRUPT;
    const BlobLayout b = blob_layout(d);
    fill_info(d, b, out);
    out->blob_size = get_le(h + 40, 8);
    if (out->blob_size < b.off_payload) return CG_E_CORRUPT;
    return CG_OK;
}

int cg_read_status(const void *ws, void *stream) {
    if (!ws) return CG_E_INVAL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(s) != hipSuccess) return CG_E_HIP;
    uint32_t st = 0;
    if (hipMemcpy(&st, ws, sizeof st, hipMemcpyDeviceToHost) != hipSuccess) return CG_E_HIP;
    if (st & kStNonfinite) return CG_E_NONFINITE;
    if (st & kStCorrupt) return CG_E_CORRUPT;
    if (st & kStCapacity) return CG_E_CAPACITY;
    return CG_OK;
}

int cg_quantize(const cg_desc *desc, const void *kv, uint8_t *sym, uint16_t *scale, void *ws,
                size_t ws_bytes, void *stream) {
    Dims d;
    WsLayout w;
    int rc = prologue(desc, CG_OP_QUANTIZE, ws, ws_bytes, d, w);
    if (rc) return rc;
    if (!kv || !sym || !scale) return CG_E_INVAL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    MaxTable mt;
    make_max_table(desc, d, mt);
    if ((rc = clear_ws(ws, w, s))) return rc;
    return hip_rc(launch_quantize(d, mt, reinterpret_cast<const uint16_t *>(kv), sym, scale,
                                  at<uint32_t>(ws, 0), s));
}

int cg_build_cdf(const cg_desc *desc, const uint8_t *sym, int32_t *cdf, void *ws, size_t ws_bytes,
                 void *stream) {
    Dims d;
    WsLayout w;
    int rc = prologue(desc, CG_OP_BUILD_CDF, ws, ws_bytes, d, w);
    if (rc) return rc;
    if (!sym || !cdf) return CG_E_INVAL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if ((rc = clear_ws(ws, w, s))) return rc;
    uint32_t *status = at<uint32_t>(ws, 0);
    uint32_t *counts = at<uint32_t>(ws, w.counts);
    if ((rc = hip_rc(launch_histogram(d, sym, counts, status, s)))) return rc;
    MaxTable mt;
    make_max_table(desc, d, mt);
    return hip_rc(launch_cdf(d, mt, counts, cdf, nullptr, nullptr, status, s));
}

int cg_encode(const cg_desc *desc, const uint8_t *sym, const int32_t *cdf, uint8_t *payload,
              size_t cap, uint16_t *lengths, uint64_t *chunk_off, void *ws, size_t ws_bytes,
              void *stream) {
    Dims d;
    WsLayout w;
    int rc = prologue(desc, CG_OP_ENCODE, ws, ws_bytes, d, w);
    if (rc) return rc;
    if (!sym || !cdf || !lengths || !chunk_off || (!payload && cap)) return CG_E_INVAL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if ((rc = clear_ws(ws, w, s))) return rc;
    EncodeOut o{payload, (uint64_t)cap, lengths, chunk_off, nullptr, nullptr, 0};
    EncodeWs ew{at<WsHeader>(ws, 0),         at<uint32_t>(ws, w.tile_sum), at<uint8_t>(ws, w.tile_mode),
                at<uint64_t>(ws, w.tile_off), at<uint64_t>(ws, w.chunk_total),
                at<uint8_t>(ws, w.staging),   at<uint64_t>(ws, w.scan)};
    MaxTable mt;
    make_max_table(desc, d, mt);
    return hip_rc(launch_encode(d, mt, sym, cdf, nullptr, nullptr, o, ew, false, false, s));
}

int cg_decode(const cg_desc *desc, const uint8_t *payload, size_t payload_bytes,
              const uint16_t *lengths, const uint64_t *chunk_off, const int32_t *cdf,
              uint8_t *sym, void *ws, size_t ws_bytes, void *stream) {
    Dims d;
    WsLayout w;
    int rc = prologue(desc, CG_OP_DECODE, ws, ws_bytes, d, w);
    if (rc) return rc;
    if (!lengths || !chunk_off || !cdf || !sym || (!payload && payload_bytes)) return CG_E_INVAL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    MaxTable mt;
    make_max_table(desc, d, mt);
    DecodeIn in{payload, (uint64_t)payload_bytes, lengths, chunk_off, cdf, nullptr, nullptr};
    in.zero_status = true;
    DecodeOut out{sym, nullptr, nullptr};
    return hip_rc(launch_decode(d, mt, in, out, at<uint64_t>(ws, w.tile_off), at<uint64_t>(ws, w.scan),
                                at<uint32_t>(ws, 0), s));
}

int cg_dequantize(const cg_desc *desc, const uint8_t *sym, const uint16_t *scale, void *kv_out,
                  void *ws, size_t ws_bytes, void *stream) {
    Dims d;
    int rc = make_dims(desc, d);
    if (rc) return rc;
    if (!sym || !scale || !kv_out) return CG_E_INVAL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (ws) {
        if (ws_bytes < kWsAlign || (uintptr_t)ws % kWsAlign) return CG_E_WORKSPACE;
        WsLayout w;
        if ((rc = clear_ws(ws, w, s))) return rc;
    }
    MaxTable mt;
    make_max_table(desc, d, mt);
    return hip_rc(launch_dequantize(d, mt, sym, scale, reinterpret_cast<uint16_t *>(kv_out), s));
}

int cg_to_bytes(const cg_desc *desc, const void *kv, uint8_t *blob, size_t cap,
                uint64_t *blob_size_dev, void *ws, size_t ws_bytes, void *stream) {
    Dims d;
    WsLayout w;
    int rc = prologue(desc, CG_OP_TO_BYTES, ws, ws_bytes, d, w);
    if (rc) return rc;
    if (!kv || !blob || !blob_size_dev) return CG_E_INVAL;
    if ((uintptr_t)blob % 8) return CG_E_INVAL;
    const BlobLayout b = blob_layout(d);
    if ((uint64_t)cap < b.off_payload) return CG_E_CAPACITY;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    MaxTable mt;
    make_max_table(desc, d, mt);

    HeaderBytes hb;
    make_header(desc, d, b, hb);

    if ((rc = hip_rc(launch_blob_header(blob, hb, b, d, s, 1, 0, at<uint32_t>(ws, 0))))) return rc;
    EncodeOut o{blob + b.off_payload,
                (uint64_t)cap - b.off_payload,
                at<uint16_t>(blob, b.off_lengths),
                at<uint64_t>(blob, b.off_chunk_off),
                blob_size_dev,
                blob + 40,
                b.off_payload};
    return encode_call(d, mt, kv, at<uint16_t>(blob, b.off_scales), at<uint16_t>(blob, b.off_cdf), o, ws, w, s,
                       true);
}

int cg_from_bytes(const cg_desc *desc, const uint8_t *blob, size_t blob_size, void *kv_out,
                  void *ws, size_t ws_bytes, void *stream) {
    Dims d;
    WsLayout w;
    int rc = prologue(desc, CG_OP_FROM_BYTES, ws, ws_bytes, d, w);
    if (rc) return rc;
    if (!blob || !kv_out) return CG_E_INVAL;
    if ((uintptr_t)blob % 8) return CG_E_INVAL;
    const BlobLayout b = blob_layout(d);
    if ((uint64_t)blob_size < b.off_payload) return CG_E_CORRUPT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    MaxTable mt;
    make_max_table(desc, d, mt);
    DecodeIn in{blob + b.off_payload,
                (uint64_t)blob_size - b.off_payload,
                reinterpret_cast<const uint16_t *>(blob + b.off_lengths),
                reinterpret_cast<const uint64_t *>(blob + b.off_chunk_off),
                nullptr,
                reinterpret_cast<const uint16_t *>(blob + b.off_cdf),
                at<uint32_t>(ws, w.wpre)};
    in.zero_status = true;
    DecodeOut out{nullptr, reinterpret_cast<uint16_t *>(kv_out),
                  reinterpret_cast<const uint16_t *>(blob + b.off_scales)};
    return hip_rc(launch_decode(d, mt, in, out, at<uint64_t>(ws, w.tile_off), at<uint64_t>(ws, w.scan),
                                at<uint32_t>(ws, 0), s));
}

int cg_from_bytes_noalloc(const cg_desc *desc, const uint8_t *blob, size_t blob_size, void *kv_out,
                          uint32_t *status_dev, void *stream) {
    Dims d;
    int rc = make_dims(desc, d);
    if (rc) return rc;
    if (!blob || !kv_out || !status_dev) return CG_E_INVAL;
    if ((uintptr_t)blob % 8 || (uintptr_t)status_dev % 4) return CG_E_INVAL;
    const WsLayout w = ws_layout(d, CG_OP_FROM_BYTES);
    if (w.total > kNoAllocScratchBytes) return CG_E_WORKSPACE;
    const BlobLayout b = blob_layout(d);
    if ((uint64_t)blob_size < b.off_payload) return CG_E_CORRUPT;
    void *ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    MaxTable mt;
    make_max_table(desc, d, mt);
    DecodeIn in{blob + b.off_payload,
                (uint64_t)blob_size - b.off_payload,
                reinterpret_cast<const uint16_t *>(blob + b.off_lengths),
                reinterpret_cast<const uint64_t *>(blob + b.off_chunk_off),
                nullptr,
                reinterpret_cast<const uint16_t *>(blob + b.off_cdf),
                at<uint32_t>(ws, w.wpre)};
    // The status word is the caller's; nothing in the scratch needs to start
    // at zero (tile offsets and scan partials are written before they are
    // read).
    in.zero_status = true;
    DecodeOut out{nullptr, reinterpret_cast<uint16_t *>(kv_out),
                  reinterpret_cast<const uint16_t *>(blob + b.off_scales)};
    return hip_rc(launch_decode(d, mt, in, out, at<uint64_t>(ws, w.tile_off), at<uint64_t>(ws, w.scan),
                                status_dev, s));
}

int cg_from_bytes_chunks(const cg_desc *desc, const uint8_t *blob, size_t blob_size, int32_t chunk_begin,
                         int32_t chunk_end, void *kv_out, void *ws, size_t ws_bytes, void *stream) {
    Dims d;
    WsLayout w;
    int rc = prologue(desc, CG_OP_FROM_BYTES, ws, ws_bytes, d, w);
    if (rc) return rc;
    if (!blob || !kv_out) return CG_E_INVAL;
    if ((uintptr_t)blob % 8) return CG_E_INVAL;
    if (chunk_begin < 0 || chunk_end > d.NC || chunk_begin >= chunk_end) return CG_E_INVAL;
    const BlobLayout b = blob_layout(d);
    if ((uint64_t)blob_size < b.off_payload) return CG_E_CORRUPT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    MaxTable mt;
    make_max_table(desc, d, mt);
    DecodeIn in{blob + b.off_payload,
                (uint64_t)blob_size - b.off_payload,
                reinterpret_cast<const uint16_t *>(blob + b.off_lengths),
                reinterpret_cast<const uint64_t *>(blob + b.off_chunk_off),
                nullptr,
                reinterpret_cast<const uint16_t *>(blob + b.off_cdf),
                at<uint32_t>(ws, w.wpre),
                chunk_begin,
                chunk_end};
    in.zero_status = true;
    DecodeOut out{nullptr, reinterpret_cast<uint16_t *>(kv_out),
                  reinterpret_cast<const uint16_t *>(blob + b.off_scales)};
    return hip_rc(launch_decode(d, mt, in, out, at<uint64_t>(ws, w.tile_off), at<uint64_t>(ws, w.scan),
                                at<uint32_t>(ws, 0), s));
}

int64_t cg_workspace_bytes_batch(const cg_desc *desc, int32_t batch, size_t blob_stride, int op) {
    Dims d, vd;
    const int rc = make_dims_batch(desc, batch, (uint64_t)blob_stride, d, vd);
    if (rc) return rc;
    if (op != CG_OP_TO_BYTES && op != CG_OP_FROM_BYTES) return CG_E_INVAL;
    return (int64_t)ws_layout(vd, op).total;
}

// A batch runs as one call of batch * L layers (vd) whose kernels write and
// read each call's blob sections in place, blob_stride bytes apart.
int cg_to_bytes_batch(const cg_desc *desc, int32_t batch, const void *kv, uint8_t *blobs, size_t blob_stride,
                      uint64_t *blob_sizes_dev, void *ws, size_t ws_bytes, void *stream) {
    Dims d, vd;
    int rc = make_dims_batch(desc, batch, (uint64_t)blob_stride, d, vd);
    if (rc) return rc;
    if (!kv || !blobs || !blob_sizes_dev || !ws) return CG_E_INVAL;
    if ((uintptr_t)blobs % 8 || blob_stride % 8 || (uintptr_t)ws % kWsAlign) return CG_E_INVAL;
    const BlobLayout lay = blob_layout(d);
    if ((uint64_t)blob_stride < lay.off_payload) return CG_E_CAPACITY;
    const WsLayout w = ws_layout(vd, CG_OP_TO_BYTES);
    if ((uint64_t)ws_bytes < w.total) return CG_E_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    MaxTable mt;
    make_max_table(desc, d, mt);
    HeaderBytes hb;
    make_header(desc, d, lay, hb);
    if ((rc = hip_rc(launch_blob_header(blobs, hb, lay, d, s, batch, blob_stride, at<uint32_t>(ws, 0))))) return rc;
    EncodeOut o{blobs + lay.off_payload,
                (uint64_t)blob_stride - lay.off_payload,
                at<uint16_t>(blobs, lay.off_lengths),
                at<uint64_t>(blobs, lay.off_chunk_off),
                blob_sizes_dev,
                blobs + 40,
                lay.off_payload};
    return encode_call(vd, mt, kv, at<uint16_t>(blobs, lay.off_scales), at<uint16_t>(blobs, lay.off_cdf), o, ws, w,
                       s, true);
}

int cg_from_bytes_batch(const cg_desc *desc, int32_t batch, const uint8_t *blobs, size_t blob_stride,
                        const uint64_t *blob_sizes_dev, void *kv_out, void *ws, size_t ws_bytes, void *stream) {
    Dims d, vd;
    int rc = make_dims_batch(desc, batch, (uint64_t)blob_stride, d, vd);
    if (rc) return rc;
    if (!blobs || !blob_sizes_dev || !kv_out || !ws) return CG_E_INVAL;
    if ((uintptr_t)blobs % 8 || blob_stride % 8 || (uintptr_t)ws % kWsAlign) return CG_E_INVAL;
    const BlobLayout lay = blob_layout(d);
    if ((uint64_t)blob_stride < lay.off_payload) return CG_E_INVAL;
    const WsLayout w = ws_layout(vd, CG_OP_FROM_BYTES);
    if ((uint64_t)ws_bytes < w.total) return CG_E_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    MaxTable mt;
    make_max_table(desc, d, mt);
    HeaderBytes hb;
    make_header(desc, d, lay, hb);
    uint32_t *status = at<uint32_t>(ws, 0);
    if ((rc = clear_ws(ws, w, s))) return rc;
    if ((rc = hip_rc(launch_batch_check(blobs, blob_stride, batch, blob_sizes_dev, hb, lay.off_payload, status, s))))
        return rc;
    DecodeIn in{blobs + lay.off_payload,
                (uint64_t)blob_stride - lay.off_payload,
                reinterpret_cast<const uint16_t *>(blobs + lay.off_lengths),
                reinterpret_cast<const uint64_t *>(blobs + lay.off_chunk_off),
                nullptr,
                reinterpret_cast<const uint16_t *>(blobs + lay.off_cdf),
                at<uint32_t>(ws, w.wpre)};
    in.call_sizes = blob_sizes_dev;
    in.payload_off = lay.off_payload;
    DecodeOut out{nullptr, reinterpret_cast<uint16_t *>(kv_out),
                  reinterpret_cast<const uint16_t *>(blobs + lay.off_scales)};
    return hip_rc(launch_decode(vd, mt, in, out, at<uint64_t>(ws, w.tile_off), at<uint64_t>(ws, w.scan), status, s));
}

int cg_from_bytes_paged(const cg_desc *desc, const uint8_t *blob, size_t blob_size, void *kv_cache,
                        int64_t layer_stride, int64_t kv_stride, int32_t block_size,
                        const int32_t *block_table, int32_t num_blocks, void *ws, size_t ws_bytes,
                        void *stream) {
    Dims d;
    WsLayout w;
    int rc = prologue(desc, CG_OP_FROM_BYTES, ws, ws_bytes, d, w);
    if (rc) return rc;
    if (!blob || !kv_cache || !block_table) return CG_E_INVAL;
    if ((uintptr_t)blob % 8 || (uintptr_t)kv_cache % 2) return CG_E_INVAL;
    if (block_size < 4 || (block_size & (block_size - 1)) || num_blocks < 1) return CG_E_INVAL;
    if (layer_stride < 0 || kv_stride < 0) return CG_E_INVAL;
    // One (layer, K|V) region, plus a block of slack for dropped rows, is
    // addressed with 32-bit byte offsets.
    if (((uint64_t)num_blocks + 1) * (uint64_t)block_size * (uint64_t)d.C * 2 >= (1ull << 32)) return CG_E_SHAPE;
    const BlobLayout b = blob_layout(d);
    if ((uint64_t)blob_size < b.off_payload) return CG_E_CORRUPT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    MaxTable mt;
    make_max_table(desc, d, mt);
    DecodeIn in{blob + b.off_payload,
                (uint64_t)blob_size - b.off_payload,
                reinterpret_cast<const uint16_t *>(blob + b.off_lengths),
                reinterpret_cast<const uint64_t *>(blob + b.off_chunk_off),
                nullptr,
                reinterpret_cast<const uint16_t *>(blob + b.off_cdf),
                at<uint32_t>(ws, w.wpre)};
    in.zero_status = true;
    int log2_bs = 0;
    while ((1 << log2_bs) < block_size) ++log2_bs;
    DecodeOut out{nullptr, nullptr, reinterpret_cast<const uint16_t *>(blob + b.off_scales),
                  PagedOut{reinterpret_cast<uint16_t *>(kv_cache), layer_stride, kv_stride, log2_bs,
                           block_table, num_blocks}};
    return hip_rc(launch_decode(d, mt, in, out, at<uint64_t>(ws, w.tile_off), at<uint64_t>(ws, w.scan),
                                at<uint32_t>(ws, 0), s));
}

}  // extern "C"
