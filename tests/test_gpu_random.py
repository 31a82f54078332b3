"""Seeded random sweep of shapes, bins and table formats through every
whole-blob path on the GPU, against the oracle; and two calls running at
once on two streams.

Each case draws L, T, H, D, per-layer bins in [4, 128] (or the default
rule), the table format and an outlier mix, then checks: the blob is the
oracle's byte for byte; the decode is the oracle's bit for bit; a
batch of two calls (this KV and a second draw) gives the two per-call blobs
and decodes; a random chunk range decodes exactly its tokens.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import assert_bf16_equal, to_dev, to_np
from kv_cache_compression_layer_amd import cachegen as cgb
from kv_cache_compression_layer_amd.synth import generate_kv

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 6))
    T = int(rng.choice([1, 17, 255, 256, 257, 511, 700, 1030]))
    H = int(rng.integers(1, 4))
    D = int(rng.choice([8, 40, 64, 96, 128]))
    if rng.random() < 0.3:
        bk, bv = oracle.default_bins(L)
    else:
        bk = rng.integers(4, 129, L).astype(np.uint8)
        bv = rng.integers(4, 129, L).astype(np.uint8)
    fmt = int(rng.integers(0, 2))
    frac = float(rng.choice([0.0, 0.02, 0.1]))
    return L, T, H, D, bk, bv, fmt, frac


@pytest.mark.parametrize("seed", range(12))
def test_random_case(seed):
    import torch

    L, T, H, D, bk, bv, fmt, frac = _draw(seed)
    kvs = [generate_kv(L, T, H, D, outlier_frac=frac, outlier_scale=15.0, seed=9000 + 2 * seed + i) for i in range(2)]
    want = [oracle.to_bytes(kv, bk, bv, fmt) for kv in kvs]
    ref = [np.asarray(oracle.from_bytes(w)).view(np.uint16).reshape(-1) for w in want]

    # Whole blob.
    blob = cgb.to_bytes(to_dev(kvs[0]).view(torch.bfloat16), bk, bv, table_format=fmt)
    assert to_np(blob).tobytes() == want[0], (L, T, H, D, fmt)
    out = to_np(cgb.from_bytes(blob).view(torch.int16), np.uint16).reshape(-1)
    assert_bf16_equal(out, ref[0])

    # Batch of two.
    desc = cgb.Desc(L, T, H, D, bk, bv, fmt)
    stride = (cgb.cg_blob_bound(desc) + 7) // 8 * 8
    blobs = torch.zeros(2 * stride, dtype=torch.uint8, device="cuda:0")
    sizes = torch.zeros(2, dtype=torch.int64, device="cuda:0")
    ws = cgb.alloc_workspace_batch(desc, 2, stride, cgb.CG_OP_TO_BYTES)
    cgb.cg_to_bytes_batch(desc, 2, to_dev(np.stack(kvs)), blobs, stride, sizes, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    b_np, s_np = to_np(blobs), to_np(sizes)
    for b in range(2):
        assert b_np[b * stride : b * stride + int(s_np[b])].tobytes() == want[b], f"call {b}"
    n = 2 * L * T * H * D
    bout = torch.empty(2 * n, dtype=torch.int16, device="cuda:0")
    ws = cgb.alloc_workspace_batch(desc, 2, stride, cgb.CG_OP_FROM_BYTES)
    cgb.cg_from_bytes_batch(desc, 2, blobs, stride, sizes, bout, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    bo = to_np(bout, np.uint16)
    np.testing.assert_array_equal(bo[:n], out)
    assert_bf16_equal(bo[n:], ref[1])

    # A random chunk range.
    rng = np.random.default_rng(seed + 77)
    nc = desc.nchunks
    j0 = int(rng.integers(0, nc))
    j1 = int(rng.integers(j0 + 1, nc + 1))
    part = torch.full((n,), 0x7F7F, dtype=torch.int16, device="cuda:0")
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES)
    cgb.cg_from_bytes_chunks(desc, blob, blob.numel(), j0, j1, part, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    got = to_np(part, np.uint16).reshape(L, 2, T, -1)
    full = out.reshape(L, 2, T, -1)
    t0, t1 = 256 * j0, min(T, 256 * j1)
    np.testing.assert_array_equal(got[:, :, t0:t1], full[:, :, t0:t1])
    assert np.all(got[:, :, :t0] == 0x7F7F) and np.all(got[:, :, t1:] == 0x7F7F)


def test_two_streams_at_once():
    """Calls on two streams with their own workspaces do not interfere."""
    import torch

    L, T, H, D = 4, 2048, 8, 128
    bk, bv = oracle.default_bins(L)
    kvs = [generate_kv(L, T, H, D, outlier_frac=0.01, outlier_scale=20.0, seed=4100 + i) for i in range(2)]
    want = [oracle.to_bytes(kv, bk, bv) for kv in kvs]
    desc = cgb.Desc(L, T, H, D, bk, bv)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    kv_d = [to_dev(kv) for kv in kvs]
    blobs = [torch.zeros(cgb.cg_blob_bound(desc), dtype=torch.uint8, device="cuda:0") for _ in range(2)]
    sizes = [torch.zeros(1, dtype=torch.int64, device="cuda:0") for _ in range(2)]
    wss = [cgb.alloc_workspace(desc, cgb.CG_OP_TO_BYTES) for _ in range(2)]
    outs = [torch.empty(2 * L * T * H * D, dtype=torch.int16, device="cuda:0") for _ in range(2)]
    wsd = [cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES) for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(3):
        for i in range(2):
            cgb.cg_to_bytes(desc, kv_d[i], blobs[i], sizes[i], wss[i], streams[i])
        for i in range(2):
            streams[i].synchronize()
            n = int(sizes[i].item())
            cgb.cg_from_bytes(desc, blobs[i], n, outs[i], wsd[i], streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert cgb.cg_read_status(wss[i], streams[i]) == cgb.CG_OK
            assert cgb.cg_read_status(wsd[i], streams[i]) == cgb.CG_OK
            n = int(sizes[i].item())
            assert to_np(blobs[i][:n]).tobytes() == want[i], (rep, i)
            ref = np.asarray(oracle.from_bytes(want[i])).view(np.uint16).reshape(-1)
            assert_bf16_equal(to_np(outs[i], np.uint16), ref)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize(
    "L,T,H,D",
    [
        (1024, 3, 1, 8),     # the largest layer count: every entry of the per-layer tables in use
        (1, 40, 64, 128),    # C = 8192: 128 channel blocks per slab, the generic quantiser
        (2, 300, 3, 1000),   # C = 3000, not a multiple of 64
    ],
)
def test_size_limits(L, T, H, D, fmt):
    import torch

    rng = np.random.default_rng(L + T + H)
    bk = rng.integers(4, 129, L).astype(np.uint8)
    bv = rng.integers(4, 129, L).astype(np.uint8)
    kv = generate_kv(L, T, H, D, outlier_frac=0.01, outlier_scale=10.0, seed=L * 7 + D)
    want = oracle.to_bytes(kv, bk, bv, fmt)
    blob = cgb.to_bytes(to_dev(kv).view(torch.bfloat16), bk, bv, table_format=fmt)
    assert to_np(blob).tobytes() == want
    out = to_np(cgb.from_bytes(blob).view(torch.int16), np.uint16).reshape(-1)
    ref = np.asarray(oracle.from_bytes(want)).view(np.uint16).reshape(-1)
    assert_bf16_equal(out, ref)

