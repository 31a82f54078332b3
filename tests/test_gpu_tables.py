"""The per-layer table format (CG_TABLES_PER_LAYER) on the GPU, against the
oracle.

Every (K|V, layer) table has its layer's own alphabet: the blobs must be
byte for byte the oracle's format-1 blobs (quantiser-built tables for
C = 512 / 1024 and short calls, tables from the counts otherwise, odd bins,
alphabets above 32), the stage calls must give the oracle's tables, payload
and symbols, and every decode path (whole, batch, paged, chunk ranges) must
give the same bf16 as the shared-table blob of the same KV.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import assert_bf16_equal, run_stages, to_dev, to_np
from kv_cache_compression_layer_amd import cachegen as cgb
from kv_cache_compression_layer_amd.synth import generate_kv

pytestmark = pytest.mark.gpu

PER_LAYER = cgb.CG_TABLES_PER_LAYER


def _bins(L, kind):
    if kind == "default":
        return oracle.default_bins(L)
    rng = np.random.default_rng(L + len(kind))
    hi = 33 if kind == "odd" else 100
    return rng.integers(4, hi, L).astype(np.uint8), rng.integers(4, hi, L).astype(np.uint8)


CASES = [
    ((12, 300, 1, 96), "default"),   # tables from the counts (C = 96)
    ((3, 64, 1, 40), "odd"),         # odd bins, one short chunk
    ((32, 256, 8, 128), "default"),  # C = 1024, one chunk: the quantiser builds the tables
    ((4, 700, 8, 128), "default"),   # C = 1024, three chunks: tables from the counts
    ((3, 256, 4, 128), "odd"),       # C = 512, quantiser-built tables, odd widths
    ((4, 256, 8, 128), "odd"),       # C = 1024, quantiser-built tables held whole, odd widths
    ((4, 264, 2, 128), "odd"),       # C = 256, quantiser-built tables, eight entries at a time
    ((3, 200, 6, 128), "default"),   # C = 768, quantiser-built tables
    ((2, 300, 1, 64), "wide"),       # alphabet above 32
]


@pytest.mark.parametrize("shape,kind", CASES)
def test_blob_equals_oracle(shape, kind):
    import torch

    L, T, H, D = shape
    kv = generate_kv(L, T, H, D, outlier_frac=0.02, outlier_scale=20.0, seed=31 + L + T)
    bk, bv = _bins(L, kind)
    want = oracle.to_bytes(kv, bk, bv, 1)
    kv_d = to_dev(kv).view(torch.bfloat16)
    blob = cgb.to_bytes(kv_d, bk, bv, table_format=PER_LAYER)
    assert to_np(blob).tobytes() == want
    out = to_np(cgb.from_bytes(blob).view(torch.int16), np.uint16)
    ref = np.asarray(oracle.from_bytes(want)).view(np.uint16)
    assert_bf16_equal(out.reshape(-1), ref.reshape(-1))
    # Same symbols as the shared-table blob, so the same decode bit for bit.
    shared = cgb.to_bytes(kv_d, bk, bv)
    np.testing.assert_array_equal(out, to_np(cgb.from_bytes(shared).view(torch.int16), np.uint16))
    if len(set(bk.tolist()) | set(bv.tolist())) > 1:
        assert blob.numel() < shared.numel()


@pytest.mark.parametrize("shape,kind", [((12, 300, 1, 96), "default"), ((3, 64, 2, 40), "odd")])
def test_stage_calls_equal_oracle(shape, kind):
    L, T, H, D = shape
    kv = generate_kv(L, T, H, D, outlier_frac=0.02, outlier_scale=20.0, seed=77 + L)
    bk, bv = _bins(L, kind)
    got = run_stages(kv, bk, bv, PER_LAYER)
    for k in ("quantize_status", "cdf_status", "encode_status", "decode_status"):
        assert got[k] == cgb.CG_OK, k
    sym, scale = oracle.quantize(kv, bk, bv)
    A = oracle.alphabet(bk, bv)
    widths = oracle.table_widths(bk, bv, 1)
    cdf = oracle.build_cdf(sym, A, widths)
    np.testing.assert_array_equal(got["cdf"], cdf)
    payload, lengths, chunk_off = oracle.encode(sym, cdf, widths)
    np.testing.assert_array_equal(got["lengths"], lengths)
    np.testing.assert_array_equal(got["chunk_off"], chunk_off)
    assert got["payload"].tobytes() == payload.tobytes()
    np.testing.assert_array_equal(got["sym_decoded"], sym)


def test_batch_paged_and_chunk_ranges():
    import torch

    B, L, T, H, D = 3, 12, 600, 2, 64
    bk, bv = oracle.default_bins(L)
    kv = np.stack([generate_kv(L, T, H, D, outlier_frac=0.02, outlier_scale=10.0, seed=500 + b) for b in range(B)])
    desc = cgb.Desc(L, T, H, D, bk, bv, PER_LAYER)
    stride = (cgb.cg_blob_bound(desc) + 7) // 8 * 8
    blobs = torch.zeros(B * stride, dtype=torch.uint8, device="cuda:0")
    sizes = torch.zeros(B, dtype=torch.int64, device="cuda:0")
    ws = cgb.alloc_workspace_batch(desc, B, stride, cgb.CG_OP_TO_BYTES)
    cgb.cg_to_bytes_batch(desc, B, to_dev(kv), blobs, stride, sizes, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    blobs_np, sizes_np = to_np(blobs), to_np(sizes)
    n = 2 * L * T * H * D
    out = torch.empty(B * n, dtype=torch.int16, device="cuda:0")
    ws = cgb.alloc_workspace_batch(desc, B, stride, cgb.CG_OP_FROM_BYTES)
    cgb.cg_from_bytes_batch(desc, B, blobs, stride, sizes, out, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    out_np = to_np(out, np.uint16)
    for b in range(B):
        blob_b = blobs_np[b * stride : b * stride + int(sizes_np[b])].tobytes()
        assert blob_b == oracle.to_bytes(kv[b], bk, bv, 1), f"call {b}"
        dev_b = torch.from_numpy(np.frombuffer(blob_b, np.uint8).copy()).to("cuda:0")
        whole = to_np(cgb.from_bytes(dev_b).view(torch.int16), np.uint16).reshape(-1)
        np.testing.assert_array_equal(out_np[b * n : (b + 1) * n], whole)
    # Paged and chunk-range decodes of call 0.
    blob0 = torch.from_numpy(np.frombuffer(blobs_np[: int(sizes_np[0])].tobytes(), np.uint8).copy()).to("cuda:0")
    whole = to_np(cgb.from_bytes(blob0).view(torch.int16), np.uint16).reshape(L, 2, T, H * D)
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES)
    part = torch.full((n,), 0x7F7F, dtype=torch.int16, device="cuda:0")
    cgb.cg_from_bytes_chunks(desc, blob0, blob0.numel(), 1, 3, part, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    got = to_np(part, np.uint16).reshape(L, 2, T, H * D)
    np.testing.assert_array_equal(got[:, :, 256:600], whole[:, :, 256:600])
    bs, nblk = 16, (T + 15) // 16
    table = np.random.default_rng(3).permutation(nblk + 4)[:nblk].astype(np.int32)
    cache = torch.zeros((L, 2, nblk + 4, bs, H * D), dtype=torch.int16, device="cuda:0")
    cgb.cg_from_bytes_paged(desc, blob0, blob0.numel(), cache, 2 * (nblk + 4) * bs * H * D,
                            (nblk + 4) * bs * H * D, bs, to_dev(table), nblk + 4, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    cache_np = to_np(cache, np.uint16)
    for i, phys in enumerate(table):
        t0, t1 = i * bs, min(T, (i + 1) * bs)
        np.testing.assert_array_equal(cache_np[:, :, phys, : t1 - t0], whole[:, :, t0:t1])


def test_corrupt_table_is_reported():
    import torch

    L, T, H, D = 12, 100, 1, 64
    kv = generate_kv(L, T, H, D, outlier_frac=0.0, outlier_scale=1.0, seed=12)
    bk, bv = oracle.default_bins(L)
    blob = bytearray(oracle.to_bytes(kv, bk, bv, 1))
    lay = cgb.cg_blob_layout(cgb.Desc(L, T, H, D, bk, bv, PER_LAYER))
    # Entry 1 of the first V table of layer 11 (width 16) made smaller than entry 0.
    widths = oracle.table_widths(bk, bv, 1).reshape(-1).astype(np.int64)
    e = int(widths[: L + 11].sum()) * H * D + 1
    pos = lay["off_cdf"] + 2 * e
    blob[pos] = blob[pos + 1] = 0
    dev = torch.from_numpy(np.frombuffer(bytes(blob), np.uint8).copy()).to("cuda:0")
    desc = cgb.Desc(L, T, H, D, bk, bv, PER_LAYER)
    out = torch.empty(2 * L * T * H * D, dtype=torch.int16, device="cuda:0")
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES)
    cgb.cg_from_bytes(desc, dev, dev.numel(), out, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_E_CORRUPT


@pytest.mark.parametrize("fmt", [0, 1])
def test_section_gaps_are_zero_in_a_dirty_buffer(fmt):
    """The blob is written into a buffer full of 0xAB: every byte the
    library does not fill with data (header padding, the gaps after each
    section, including the ragged table section) must still equal the
    oracle's zero padding."""
    import torch

    L, T, H, D = 5, 255, 1, 40
    rng = np.random.default_rng(2)
    bk = rng.integers(4, 129, L).astype(np.uint8)
    bv = rng.integers(4, 129, L).astype(np.uint8)
    kv = generate_kv(L, T, H, D, outlier_frac=0.0, outlier_scale=1.0, seed=13)
    want = oracle.to_bytes(kv, bk, bv, fmt)
    desc = cgb.Desc(L, T, H, D, bk, bv, fmt)
    blob = torch.full((cgb.cg_blob_bound(desc),), 0xAB, dtype=torch.uint8, device="cuda:0")
    size = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_TO_BYTES)
    cgb.cg_to_bytes(desc, to_dev(kv), blob, size, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    assert to_np(blob[: int(size.item())]).tobytes() == want
