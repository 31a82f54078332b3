// Batches of to_bytes / from_bytes calls of one shape on gfx950.
//
// LMCache CacheGen page (0539edu.com/news/4720135), end-to-end benchmark:
// KV is encoded per LMCache chunk (64..768 tokens), each call with its own
// tables. B such calls of one shape [L,2,T,H,D] are laid out as [B*L,2,T,H,D]
// and coded as one call of B*L layers whose slabs are numbered call by call
// (CallMap): every kernel writes (and the decoder reads) call b's scales,
// tables, lengths, chunk offsets and payload in place in call b's blob, so
// a batch moves no blob bytes beyond those of the calls themselves. The
// encoder's tile scan runs per (chunk, call), and k_chunk_scan turns each
// call's chunk totals into its chunk offsets and size.
//
// What remains here is the decode side's check of each blob's header
// against the batch's shape; the chunk offsets of each call are checked
// against its lengths by the tile scan, as for a single call.
#include "cg_internal.hpp"

namespace cg {

// Block b checks call b: header bytes (but the size field, bytes 40..47),
// the size field against sizes_dev[b], and that size against the stride
// and the header and sections' end.
__global__ __launch_bounds__(256) void k_batch_check(const uint8_t *__restrict__ blobs, uint64_t stride,
                                                     const uint64_t *__restrict__ sizes_dev, HeaderBytes hdr,
                                                     uint64_t off_payload, uint32_t *__restrict__ status) {
    __shared__ int bad_call;
    const int b = blockIdx.x, tid = threadIdx.x;
    const uint8_t *blob = blobs + (uint64_t)b * stride;
    if (tid == 0) bad_call = 0;
    __syncthreads();
    const uint64_t size = sizes_dev[b];
    bool bad = size < off_payload || size > stride;
    for (uint32_t i = tid; i < hdr.n; i += 256)
        if ((i < 40 || i >= 48) && blob[i] != hdr.b[i]) bad = true;
    if (tid < 8 && blob[40 + tid] != (uint8_t)(size >> (8 * tid))) bad = true;
    if (bad) atomicOr(&bad_call, 1);
    __syncthreads();
    if (tid == 0 && bad_call) atomicOr(status, kStCorrupt);
}

hipError_t launch_batch_check(const uint8_t *blobs, uint64_t stride, int B, const uint64_t *sizes_dev,
                              const HeaderBytes &hdr, uint64_t off_payload, uint32_t *status, hipStream_t s) {
    hipLaunchKernelGGL(k_batch_check, dim3((unsigned)B), dim3(256), 0, s, blobs, stride, sizes_dev, hdr,
                       off_payload, status);
    return hipGetLastError();
}

}  // namespace cg
