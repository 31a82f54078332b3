"""Decode of chunk ranges (cg_from_bytes_chunks) and the pipelined load that
decodes each piece of a blob as it arrives, on the GPU.

Every chunk decodes on its own once the front sections are there, so a range
decode must write exactly the tokens of its chunks, bit for bit as the whole
decode writes them, must not need (or read) the payload after its last chunk,
and the pieces of a pipelined load together must give the whole decode.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import to_dev, to_np
from kv_cache_compression_layer_amd import cachegen as cgb
from kv_cache_compression_layer_amd import streaming
from kv_cache_compression_layer_amd.synth import generate_kv

pytestmark = pytest.mark.gpu

SENTINEL = 0x7F7F


def _encode(shape, seed):
    import torch

    L, T, H, D = shape
    kv = generate_kv(L, T, H, D, outlier_frac=0.02, outlier_scale=10.0, seed=seed)
    bk, bv = oracle.default_bins(L)
    blob = cgb.to_bytes(to_dev(kv).view(torch.bfloat16), bk, bv)
    desc = cgb.Desc(L, T, H, D, bk, bv)
    full = to_np(cgb.from_bytes(blob).view(torch.int16), np.uint16).reshape(L, 2, T, H * D)
    lay = cgb.cg_blob_layout(desc)
    nc = desc.nchunks
    chunk_off = to_np(blob[lay["off_chunk_off"] : lay["off_chunk_off"] + 8 * (nc + 1)]).view(np.uint64)
    return kv, desc, blob, full, lay, chunk_off


@pytest.mark.parametrize("shape", [(2, 700, 1, 96), (3, 1024, 2, 64)])
def test_chunk_ranges_write_exactly_their_tokens(shape):
    import torch

    L, T, H, D = shape
    _, desc, blob, full, lay, chunk_off = _encode(shape, seed=61)
    nc = desc.nchunks
    ranges = [(0, 1), (nc - 1, nc), (0, nc)] + ([(1, nc - 1)] if nc > 2 else [])
    for j0, j1 in ranges:
        # Only the bytes up to the end of chunk j1 - 1 are there; the rest of
        # the buffer holds bytes that are not the blob's.
        need = int(lay["off_payload"] + chunk_off[j1])
        part = torch.full((blob.numel(),), 0xAB, dtype=torch.uint8, device="cuda:0")
        part[:need] = blob[:need]
        out = torch.full((L * 2 * T * H * D,), SENTINEL, dtype=torch.int16, device="cuda:0")
        ws = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES)
        cgb.cg_from_bytes_chunks(desc, part, need, j0, j1, out, ws)
        assert cgb.cg_read_status(ws) == cgb.CG_OK, (j0, j1)
        got = to_np(out, np.uint16).reshape(L, 2, T, H * D)
        t0, t1 = 256 * j0, min(T, 256 * j1)
        np.testing.assert_array_equal(got[:, :, t0:t1], full[:, :, t0:t1])
        assert np.all(got[:, :, :t0] == SENTINEL) and np.all(got[:, :, t1:] == SENTINEL)


def test_chunk_range_errors():
    import torch

    _, desc, blob, _, lay, chunk_off = _encode((2, 700, 1, 64), seed=62)
    nc = desc.nchunks
    out = torch.empty(desc.nlayers * 2 * desc.ntokens * desc.nchannels, dtype=torch.int16, device="cuda:0")
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES)
    for j0, j1 in [(1, 1), (2, 1), (-1, 1), (0, nc + 1)]:
        with pytest.raises(cgb.CacheGenValueError):
            cgb.cg_from_bytes_chunks(desc, blob, blob.numel(), j0, j1, out, ws)
    # The payload of the last chunk of the range has not fully arrived.
    short = int(lay["off_payload"] + chunk_off[2]) - 1
    cgb.cg_from_bytes_chunks(desc, blob, short, 0, 2, out, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_E_CORRUPT
    # ... which does not matter to the chunks before it.
    cgb.cg_from_bytes_chunks(desc, blob, short, 0, 1, out, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_OK


@pytest.mark.parametrize("chunks_per_piece", [1, 3])
def test_pipelined_load_equals_whole_decode(chunks_per_piece):
    import torch

    shape = (4, 2048 + 100, 8, 128)  # nine chunks, the last one short; C = 1024
    L, T, H, D = shape
    _, desc, blob, full, lay, chunk_off = _encode(shape, seed=63)
    host = torch.empty(blob.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(blob.cpu())
    dev_blob = torch.zeros(blob.numel(), dtype=torch.uint8, device="cuda:0")
    out = torch.full((L * 2 * T * H * D,), SENTINEL, dtype=torch.int16, device="cuda:0")
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES)
    pieces = streaming.plan_pieces(int(lay["off_payload"]), chunk_off, chunks_per_piece)
    assert pieces[-1].byte_end == blob.numel()
    copy_s, dec_s = torch.cuda.Stream(), torch.cuda.Stream()
    streaming.enqueue_pipelined_load(desc, host, dev_blob, out, ws, pieces, copy_s, dec_s)
    torch.cuda.synchronize()
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    np.testing.assert_array_equal(to_np(out, np.uint16).reshape(L, 2, T, H * D), full)

