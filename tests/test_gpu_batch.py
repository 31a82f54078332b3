"""Batches of to_bytes / from_bytes calls of one shape (cg_to_bytes_batch,
cg_from_bytes_batch) on the GPU.

Each call of a batch has its own scales, histograms and tables, so the blob a
batch writes for call b must be byte for byte the oracle's to_bytes of call b
alone, and the batch decode of those blobs must equal the per-call decode and the
oracle's decode bit for bit.
The cases cover ragged token counts, several chunks, channel counts that are
not a multiple of 64, calls with constant or zero KV, layer counts that vary
their bins, and batches of more than 1024 layers in total (the device looks
the layer constants up by the layer within its call).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import assert_bf16_equal, to_dev, to_np
from kv_cache_compression_layer_amd import cachegen as cgb
from kv_cache_compression_layer_amd.synth import generate_kv

pytestmark = pytest.mark.gpu


def _batch_kv(B, L, T, H, D, seed, specials=True):
    """[B, L, 2, T, H, D] uint16: seeded calls, some with outliers; with
    `specials`, call 1 is all zeros and call 2 a constant."""
    calls = []
    for b in range(B):
        if specials and b == 1:
            calls.append(np.zeros((L, 2, T, H, D), np.uint16))
        elif specials and b == 2:
            calls.append(np.full((L, 2, T, H, D), 0x3F80, np.uint16))  # 1.0
        else:
            calls.append(generate_kv(L, T, H, D, outlier_frac=0.02 * (b % 3), outlier_scale=8.0,
                                     seed=seed + b))
    return np.stack(calls)


def _stride(desc, extra=0):
    """A stride of a multiple of 16 bytes (plus `extra`): blobs whose stride
    is not one take the path where the tables are built apart from the
    quantiser."""
    return (cgb.cg_blob_bound(desc) + 15) // 16 * 16 + extra


def _to_bytes_batch(kv, bk, bv, stride=None, fmt=0, extra=0):
    import torch

    B, L, _, T, H, D = kv.shape
    desc = cgb.Desc(L, T, H, D, bk, bv, fmt)
    stride = _stride(desc, extra) if stride is None else stride
    blobs = torch.zeros(B * stride, dtype=torch.uint8, device="cuda:0")
    sizes = torch.zeros(B, dtype=torch.int64, device="cuda:0")
    ws = cgb.alloc_workspace_batch(desc, B, stride, cgb.CG_OP_TO_BYTES)
    cgb.cg_to_bytes_batch(desc, B, to_dev(kv), blobs, stride, sizes, ws)
    return desc, stride, blobs, sizes, cgb.cg_read_status(ws)


def _from_bytes_batch(desc, B, blobs, stride, sizes):
    import torch

    out = torch.empty(B * 2 * desc.nlayers * desc.ntokens * desc.nchannels, dtype=torch.int16, device="cuda:0")
    ws = cgb.alloc_workspace_batch(desc, B, stride, cgb.CG_OP_FROM_BYTES)
    cgb.cg_from_bytes_batch(desc, B, blobs, stride, sizes, out, ws)
    return to_np(out, np.uint16), cgb.cg_read_status(ws)


def _blob(blobs_np, stride, sizes_np, b):
    return blobs_np[b * stride : b * stride + int(sizes_np[b])].tobytes()


def _per_call_decode(blob_bytes):
    import torch

    blob = torch.from_numpy(np.frombuffer(blob_bytes, np.uint8).copy()).to("cuda:0")
    return to_np(cgb.from_bytes(blob).view(torch.int16), np.uint16).reshape(-1)


@pytest.mark.parametrize(
    "B,shape,extra",
    [
        (3, (2, 300, 1, 96), 0),   # ragged T over two chunks, C not a multiple of 64
        (5, (3, 64, 2, 64), 8),    # one short chunk per call
        (4, (1, 700, 1, 40), 0),   # three chunks, C < 64
        (1, (2, 256, 1, 64), 0),   # a batch of one is the plain call
        (3, (2, 256, 4, 128), 0),  # C = 512: the quantiser builds the tables (one block per slab)
        (3, (2, 256, 4, 128), 8),  # the same with a stride of 16k + 8: tables from the counts
        (2, (3, 200, 8, 128), 0),  # C = 1024, ragged T, tables built by the quantiser
        (2, (3, 200, 8, 128), 8),
        (2, (2, 300, 8, 128), 0),  # C = 1024, two chunks: tables from the counts
        (9, (2, 256, 8, 128), 0),  # 2L * 9 slabs of one chunk each, as LMCache's 256-token chunks
        (4, (2, 256, 2, 128), 0),  # C = 256: tables built by the quantiser eight entries at a time
        (3, (2, 256, 6, 128), 0),  # C = 768
    ],
)
def test_batch_blobs_equal_oracle_per_call(B, shape, extra):
    L, T, H, D = shape
    kv = _batch_kv(B, L, T, H, D, seed=900 + B)
    bk, bv = oracle.default_bins(L)
    desc, stride, blobs, sizes, status = _to_bytes_batch(kv, bk, bv, extra=extra)
    assert status == cgb.CG_OK
    blobs_np, sizes_np = to_np(blobs), to_np(sizes)
    for b in range(B):
        want = oracle.to_bytes(kv[b], bk, bv)
        assert int(sizes_np[b]) == len(want), f"call {b}"
        assert _blob(blobs_np, stride, sizes_np, b) == want, f"call {b}"

    got, st = _from_bytes_batch(desc, B, blobs, stride, sizes)
    assert st == cgb.CG_OK
    n = 2 * L * T * H * D
    for b in range(B):
        blob_b = _blob(blobs_np, stride, sizes_np, b)
        np.testing.assert_array_equal(got[b * n : (b + 1) * n], _per_call_decode(blob_b))
        ref = np.asarray(oracle.from_bytes(blob_b)).view(np.uint16).reshape(-1)
        assert_bf16_equal(got[b * n : (b + 1) * n], ref)


@pytest.mark.parametrize(
    "B,L,H,D,fmt",
    [
        (1100, 1, 1, 64, 0),   # 1100 layers in total: every call has one layer
        (150, 7, 1, 64, 0),    # 1050 layers, period 7
        (100, 12, 1, 64, 0),   # 1200 layers, bins differ across a call's layers
        (40, 32, 8, 128, 0),   # 1280 layers of C = 1024 (tables built by the quantiser)
        (100, 12, 1, 64, 1),   # the same with per-layer tables (widths of the layer within its call)
        (40, 32, 8, 128, 1),
    ],
)
def test_batch_many_layers(B, L, H, D, fmt):
    import torch

    T = 16
    kv = _batch_kv(B, L, T, H, D, seed=1300 + L, specials=False)
    bk, bv = oracle.default_bins(L)
    desc, stride, blobs, sizes, status = _to_bytes_batch(kv, bk, bv, fmt=fmt)
    assert status == cgb.CG_OK
    blobs_np, sizes_np = to_np(blobs), to_np(sizes)
    # Every call equals the plain GPU call; a sample also equals the oracle.
    kv_d = to_dev(kv).view(torch.bfloat16)
    for b in range(B):
        one = to_np(cgb.to_bytes(kv_d[b], bk, bv, table_format=fmt)).tobytes()
        assert _blob(blobs_np, stride, sizes_np, b) == one, f"call {b}"
    for b in (0, 1, B // 2, B - 1):
        assert _blob(blobs_np, stride, sizes_np, b) == oracle.to_bytes(kv[b], bk, bv, fmt), f"call {b}"

    got, st = _from_bytes_batch(desc, B, blobs, stride, sizes)
    assert st == cgb.CG_OK
    n = 2 * L * T * H * D
    for b in (0, 1, B // 2, B - 1):
        blob_b = _blob(blobs_np, stride, sizes_np, b)
        ref = np.asarray(oracle.from_bytes(blob_b)).view(np.uint16).reshape(-1)
        assert_bf16_equal(got[b * n : (b + 1) * n], ref)
    for b in range(B):
        np.testing.assert_array_equal(got[b * n : (b + 1) * n],
                                      _per_call_decode(_blob(blobs_np, stride, sizes_np, b)))


def test_batch_whole_slab_tiles_of_hundreds_of_tokens():
    """150 calls of 2 layers, 520 tokens, C = 512: 600 (K|V, layer) slabs in
    all, so the quantiser gives each slab one block over all its 520 tokens
    and builds the tables itself (packed symbols, three chunks with a ragged
    tail), while one such call alone takes three blocks per slab and the
    counts + k_cdf path. Every call equals the plain GPU call; a sample also
    equals the oracle, and decodes to the oracle's KV."""
    import torch

    B, L, T, H, D = 150, 2, 520, 4, 128
    kv = _batch_kv(B, L, T, H, D, seed=1500)
    bk, bv = oracle.default_bins(L)
    desc, stride, blobs, sizes, status = _to_bytes_batch(kv, bk, bv)
    assert status == cgb.CG_OK
    blobs_np, sizes_np = to_np(blobs), to_np(sizes)
    kv_d = to_dev(kv).view(torch.bfloat16)
    for b in range(B):
        one = to_np(cgb.to_bytes(kv_d[b], bk, bv)).tobytes()
        assert _blob(blobs_np, stride, sizes_np, b) == one, f"call {b}"
    got, st = _from_bytes_batch(desc, B, blobs, stride, sizes)
    assert st == cgb.CG_OK
    n = 2 * L * T * H * D
    for b in (0, 1, 2, 77, B - 1):
        blob_b = _blob(blobs_np, stride, sizes_np, b)
        assert blob_b == oracle.to_bytes(kv[b], bk, bv), f"call {b}"
        ref = np.asarray(oracle.from_bytes(blob_b)).view(np.uint16).reshape(-1)
        assert_bf16_equal(got[b * n : (b + 1) * n], ref)


def test_batch_at_the_layer_limit():
    """32767 one-layer calls: 65534 (K|V, layer) slabs, the largest grid
    dimension the per-slab kernels take. Every call equals the plain GPU
    call; a sample also equals the oracle."""
    import torch

    B, L, T, H, D = 32767, 1, 8, 1, 64
    rng = np.random.default_rng(32767)
    kv = (rng.standard_normal((B, L, 2, T, H, D)).astype(np.float32)
          * rng.lognormal(0.0, 1.0, (B, 1, 1, 1, 1, 1)).astype(np.float32))
    u = kv.view(np.uint32)
    kv = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # bf16, nearest even
    bk, bv = oracle.default_bins(L)
    desc, stride, blobs, sizes, status = _to_bytes_batch(kv, bk, bv)
    assert status == cgb.CG_OK
    blobs_np, sizes_np = to_np(blobs), to_np(sizes)
    got, st = _from_bytes_batch(desc, B, blobs, stride, sizes)
    assert st == cgb.CG_OK
    n = 2 * L * T * H * D
    kv_d = to_dev(kv).view(torch.bfloat16)
    for b in list(range(0, B, 4099)) + [B - 1]:
        one = to_np(cgb.to_bytes(kv_d[b], bk, bv)).tobytes()
        assert _blob(blobs_np, stride, sizes_np, b) == one, f"call {b}"
        assert one == oracle.to_bytes(kv[b], bk, bv), f"call {b}"
        ref = np.asarray(oracle.from_bytes(one)).view(np.uint16).reshape(-1)
        assert_bf16_equal(got[b * n : (b + 1) * n], ref)


def test_batch_corrupt_call_is_reported_and_isolated():
    import torch

    B, L, T, H, D = 4, 2, 300, 1, 64
    kv = _batch_kv(B, L, T, H, D, seed=77)
    bk, bv = oracle.default_bins(L)
    desc, stride, blobs, sizes, status = _to_bytes_batch(kv, bk, bv)
    assert status == cgb.CG_OK
    blobs_np, sizes_np = to_np(blobs), to_np(sizes)
    n = 2 * L * T * H * D

    # A header byte of call 1 (its token count) no longer matches the batch.
    bad = blobs.clone()
    bad[1 * stride + 12] ^= 1
    got, st = _from_bytes_batch(desc, B, bad, stride, sizes)
    assert st == cgb.CG_E_CORRUPT
    for b in (0, 2, 3):
        np.testing.assert_array_equal(got[b * n : (b + 1) * n],
                                      _per_call_decode(_blob(blobs_np, stride, sizes_np, b)))

    # A chunk offset of call 2 that disagrees with its lengths.
    lay = cgb.cg_blob_layout(desc)
    bad = blobs.clone()
    bad[2 * stride + lay["off_chunk_off"] + 8] ^= 1
    got, st = _from_bytes_batch(desc, B, bad, stride, sizes)
    assert st == cgb.CG_E_CORRUPT
    for b in (0, 1, 3):
        np.testing.assert_array_equal(got[b * n : (b + 1) * n],
                                      _per_call_decode(_blob(blobs_np, stride, sizes_np, b)))

    # A size that disagrees with the header of call 3.
    bad_sizes = sizes.clone()
    bad_sizes[3] -= 1
    _, st = _from_bytes_batch(desc, B, blobs, stride, bad_sizes)
    assert st == cgb.CG_E_CORRUPT
    # A size beyond the stride.
    bad_sizes = sizes.clone()
    bad_sizes[0] = stride + 8
    _, st = _from_bytes_batch(desc, B, blobs, stride, bad_sizes)
    assert st == cgb.CG_E_CORRUPT
    del torch


def test_batch_small_stride_reports_capacity():
    B, L, T, H, D = 3, 2, 300, 1, 64
    kv = _batch_kv(B, L, T, H, D, seed=31)
    bk, bv = oracle.default_bins(L)
    desc = cgb.Desc(L, T, H, D, bk, bv)
    want = [oracle.to_bytes(kv[b], bk, bv) for b in range(B)]
    # Room for the smallest call (the all-zero one) only.
    stride = (min(len(w) for w in want) + 7) // 8 * 8
    assert stride < max(len(w) for w in want)
    _, _, blobs, sizes, status = _to_bytes_batch(kv, bk, bv, stride=stride)
    assert status == cgb.CG_E_CAPACITY
    # Each call's size is the size it needs, whether or not it fitted.
    assert [int(x) for x in to_np(sizes)] == [len(w) for w in want]
    # A batch with room enough after the failed one is whole again.
    desc2, stride2, blobs2, sizes2, status2 = _to_bytes_batch(kv, bk, bv)
    assert status2 == cgb.CG_OK
    blobs_np, sizes_np = to_np(blobs2), to_np(sizes2)
    for b in range(B):
        assert _blob(blobs_np, stride2, sizes_np, b) == want[b]
    del desc, desc2


def test_batch_bad_arguments():
    import torch

    L, T, H, D = 2, 64, 1, 64
    bk, bv = oracle.default_bins(L)
    desc = cgb.Desc(L, T, H, D, bk, bv)
    lay = cgb.cg_blob_layout(desc)
    with pytest.raises(cgb.CacheGenValueError):
        cgb.cg_workspace_bytes_batch(desc, 0, 4096, cgb.CG_OP_TO_BYTES)
    with pytest.raises(cgb.CacheGenValueError):
        cgb.cg_workspace_bytes_batch(desc, 20000, 4096, cgb.CG_OP_TO_BYTES)  # 40000 layers
    kv = torch.zeros(2 * 2 * L * T * H * D, dtype=torch.bfloat16, device="cuda:0")
    sizes = torch.zeros(2, dtype=torch.int64, device="cuda:0")
    stride = _stride(desc)
    ws = cgb.alloc_workspace_batch(desc, 2, stride, cgb.CG_OP_TO_BYTES)
    blobs = torch.zeros(2 * stride + 8, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(cgb.CacheGenValueError):  # stride not a multiple of 8
        cgb.cg_to_bytes_batch(desc, 2, kv, blobs, stride - 4, sizes, ws)
    small = int(lay["off_payload"]) - 8
    ws_small = cgb.alloc_workspace_batch(desc, 2, small, cgb.CG_OP_TO_BYTES)
    with pytest.raises(cgb.CacheGenValueError):  # no room for the sections
        cgb.cg_to_bytes_batch(desc, 2, kv, blobs, small, sizes, ws_small)


@pytest.mark.parametrize("shape", [(2, 256, 8, 128), (3, 100, 4, 128)])
def test_table_build_in_quantiser_equals_counts_path(shape):
    """The quantiser builds the tables itself only into a 16-byte aligned
    blob; an 8-byte aligned one takes the counts + k_cdf path. Both give the
    oracle's bytes."""
    import torch

    L, T, H, D = shape
    kv = generate_kv(L, T, H, D, outlier_frac=0.01, outlier_scale=20.0, seed=4242)
    bk, bv = oracle.default_bins(L)
    want = oracle.to_bytes(kv, bk, bv)
    desc = cgb.Desc(L, T, H, D, bk, bv)
    bound = cgb.cg_blob_bound(desc)
    kv_d = to_dev(kv)
    got = []
    for off in (0, 8):
        raw = torch.zeros(bound + 64, dtype=torch.uint8, device="cuda:0")
        base = (-raw.data_ptr()) % 16
        blob = raw[base + off : base + off + bound]
        size = torch.zeros(1, dtype=torch.int64, device="cuda:0")
        ws = cgb.alloc_workspace(desc, cgb.CG_OP_TO_BYTES)
        cgb.cg_to_bytes(desc, kv_d, blob, size, ws)
        assert cgb.cg_read_status(ws) == cgb.CG_OK
        got.append(to_np(blob[: int(size.item())]).tobytes())
    assert got[0] == want
    assert got[1] == want
