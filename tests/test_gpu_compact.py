"""Compaction of tiles whose streams outgrew the encoder's LDS stage, and the
forms of the tile-offset scan.

Such a tile leaves the encoder in rows (byte i of every stream at row i of
its staging slot) and is put in stream order by the compaction kernel: in
LDS when the grid has at most 4096 tiles, a byte at a time otherwise. Both
forms must write the oracle's blob byte for byte. Independent Gaussian
tokens (rho = 0) at 32 bins give streams of about 100 bytes, so nearly every
tile of 64 streams is far beyond the stage (1.8 or 2.8 KiB).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import assert_bf16_equal, to_dev, to_np
from kv_cache_compression_layer_amd import cachegen as cgb
from kv_cache_compression_layer_amd.synth import generate_kv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize(
    "L,T,H,why",
    [
        (2, 256, 8, "64 tiles: ordered in LDS"),
        (4, 1000, 8, "512 tiles in four chunks, the last ragged: ordered in LDS"),
        (16, 2304, 8, "4608 tiles: a byte at a time"),
    ],
)
def test_rows_tiles_match_oracle(L, T, H, why):
    import torch

    D = 128
    kv = generate_kv(L, T, H, D, rho=0.0, outlier_frac=0.02, outlier_scale=8.0, seed=900 + L + T)
    bins = np.full(L, 32, np.uint8)
    want = oracle.to_bytes(kv, bins, bins)
    info, _, _ = cgb.cg_blob_peek(want[:4096])  # the header holds every layer's bins
    # The payload averages well above the larger stage per tile.
    payload = len(want) - info["off_payload"]
    ntiles = ((T + 255) // 256) * 2 * L * ((H * D + 63) // 64)
    assert payload > 2 * 2816 * ntiles // 3, "streams too short to leave the stage"
    blob = cgb.to_bytes(to_dev(kv).view(torch.bfloat16), bins, bins)
    got = to_np(blob).tobytes()
    assert len(got) == len(want), why
    assert got == want, why
    out = to_np(cgb.from_bytes(blob).view(torch.int16), np.uint16)
    assert_bf16_equal(out.reshape(-1), oracle.from_bytes(want).reshape(-1))


@pytest.mark.parametrize(
    "L,T,why",
    [
        (2, 256, "one chunk: one block per call scans it (and the chunk pass)"),
        (2, 1500, "six chunks of 64 tiles: a block per chunk, then the chunk pass"),
        (33, 600, "1056 tiles per chunk: the three-pass scan"),
    ],
)
def test_scan_forms_match_oracle(L, T, why):
    """The tile-offset scan takes one of three forms by the tiles per chunk
    and the chunks per call; each must give the oracle's blob and decode it."""
    import torch

    kv = generate_kv(L, T, 8, 128, outlier_frac=0.02, outlier_scale=8.0, seed=950 + L + T)
    bk, bv = oracle.default_bins(L)
    want = oracle.to_bytes(kv, bk, bv)
    blob = cgb.to_bytes(to_dev(kv).view(torch.bfloat16), bk, bv)
    got = to_np(blob).tobytes()
    assert got == want, why
    out = to_np(cgb.from_bytes(blob).view(torch.int16), np.uint16)
    assert_bf16_equal(out.reshape(-1), oracle.from_bytes(want).reshape(-1))
