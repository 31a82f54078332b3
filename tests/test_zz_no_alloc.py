"""cg_from_bytes_noalloc: the decode for callers that cannot allocate.

It runs the decode of cg_from_bytes with the library's fixed device
workspace instead of a caller's. Its output must equal cg_from_bytes's bit
for bit (and so the oracle's), call after call. Two calls run in a row, the
second with a smaller input (fewer tiles, other bins), because every call on
a GPU shares the one array and the second must not depend on what the first
left in it. A corrupt blob is reported through the caller's status word, and
a call whose workspace would exceed the fixed array is refused before
anything is launched.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import assert_bf16_equal, to_dev, to_np
from kv_cache_compression_layer_amd import cachegen as cgb
from kv_cache_compression_layer_amd.synth import generate_kv

pytestmark = pytest.mark.gpu


def _blob(shape, bins, seed, fmt=0):
    import torch

    L, T, H, D = shape
    kv = generate_kv(L, T, H, D, outlier_frac=0.02, outlier_scale=15.0, seed=seed)
    bk, bv = bins if bins is not None else oracle.default_bins(L)
    blob = cgb.to_bytes(to_dev(kv).view(torch.bfloat16), bk, bv, table_format=fmt)
    return kv, np.asarray(bk, np.uint8), np.asarray(bv, np.uint8), blob


def _decode_both(desc, blob, n):
    import torch

    status = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    out_na = torch.full((n,), 0x7F7F, dtype=torch.int16, device="cuda:0")
    cgb.cg_from_bytes_noalloc(desc, blob, blob.numel(), out_na, status)
    st = cgb.cg_read_status(status)
    out = torch.empty((n,), dtype=torch.int16, device="cuda:0")
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES)
    cgb.cg_from_bytes(desc, blob, blob.numel(), out, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    return st, to_np(out_na, np.uint16), to_np(out, np.uint16)


def test_two_calls_match_from_bytes():
    cases = [
        # A larger call first (17 chunks, 1024 channels, eight-wave blocks), then a smaller one
        # (3 chunks, 96 channels, per-layer tables) that reuses the same array.
        ((4, 4200, 8, 128), None, 11, 0),
        ((2, 700, 3, 32), ([32, 16], [8, 16]), 12, 1),
    ]
    for shape, bins, seed, fmt in cases:
        kv, bk, bv, blob = _blob(shape, bins, seed, fmt)
        L, T, H, D = shape
        desc = cgb.Desc(L, T, H, D, bk, bv, fmt)
        st, got, want = _decode_both(desc, blob, L * 2 * T * H * D)
        assert st == cgb.CG_OK, shape
        assert_bf16_equal(got, want, f"noalloc vs cg_from_bytes {shape}")
        ref = np.asarray(oracle.from_bytes(to_np(blob).tobytes())).view(np.uint16).reshape(-1)
        assert_bf16_equal(got, ref, f"noalloc vs oracle {shape}")


def test_corrupt_blob_sets_the_callers_status():
    import torch

    kv, bk, bv, blob = _blob((2, 600, 1, 64), None, 21)
    L, T, H, D = 2, 600, 1, 64
    desc = cgb.Desc(L, T, H, D, bk, bv)
    lay = cgb.cg_blob_layout(desc)
    bad = blob.clone()
    # Chunk offset 1 no longer matches the lengths of chunk 0.
    off = lay["off_chunk_off"] + 8
    v = int(to_np(bad[off : off + 8]).view(np.uint64)[0]) + 1
    bad[off : off + 8] = torch.from_numpy(np.array([v], np.uint64).view(np.uint8)).to("cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    out = torch.empty(L * 2 * T * H * D, dtype=torch.int16, device="cuda:0")
    cgb.cg_from_bytes_noalloc(desc, bad, bad.numel(), out, status)
    assert cgb.cg_read_status(status) == cgb.CG_E_CORRUPT
    # The next good call starts from a clear status.
    cgb.cg_from_bytes_noalloc(desc, blob, blob.numel(), out, status)
    assert cgb.cg_read_status(status) == cgb.CG_OK


def test_too_large_is_refused():
    import torch

    # 64 layers x 4096 channels x 16384 tokens: 524288 tiles, whose offsets alone fill 4 MiB.
    L, T, H, D = 64, 16384, 32, 128
    bk, bv = oracle.default_bins(L)
    desc = cgb.Desc(L, T, H, D, bk, bv)
    assert cgb.cg_workspace_bytes(desc, cgb.CG_OP_FROM_BYTES) > 4 << 20
    import ctypes

    blob = torch.zeros(cgb.cg_blob_layout(desc)["off_payload"] + 64, dtype=torch.uint8, device="cuda:0")
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda:0")
    out = torch.empty(8, dtype=torch.int16, device="cuda:0")  # never touched: the call is refused first
    rc = cgb.lib().cg_from_bytes_noalloc(desc.ptr, ctypes.c_void_p(blob.data_ptr()), blob.numel(),
                                         ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(status.data_ptr()), None)
    assert rc == cgb.CG_E_WORKSPACE
    torch.cuda.synchronize()
    assert int(status.item()) == 7  # nothing was launched
