"""Host-side planning of a pipelined load and the link-time model (no GPU)."""

from __future__ import annotations

import numpy as np
import pytest

from kv_cache_compression_layer_amd import streaming


def test_plan_pieces_cover_every_chunk_once():
    chunk_off = np.array([0, 10, 25, 25, 40, 41], np.uint64)  # five chunks, one empty
    for cpp in (1, 2, 3, 5, 9):
        pieces = streaming.plan_pieces(1000, chunk_off, cpp)
        assert pieces[0].chunk_begin == 0 and pieces[-1].chunk_end == 5
        for a, b in zip(pieces, pieces[1:]):
            assert a.chunk_end == b.chunk_begin and a.byte_end <= b.byte_end
        for p in pieces:
            assert p.chunk_end - p.chunk_begin <= cpp
            assert p.byte_end == 1000 + int(chunk_off[p.chunk_end])
    with pytest.raises(ValueError):
        streaming.plan_pieces(0, chunk_off, 0)


def test_link_model_arithmetic():
    raw, blob = 32 << 20, 5 << 20
    (r,) = streaming.link_model(raw_bytes=raw, blob_bytes=blob, decode_ms=2.0, last_piece_decode_ms=0.5, mbps=(100,))
    assert r["raw_transfer_s"] == pytest.approx(raw * 8 / 100e6)
    assert r["blob_transfer_s"] == pytest.approx(blob * 8 / 100e6)
    assert r["serial_load_s"] == pytest.approx(blob * 8 / 100e6 + 0.002)
    assert r["pipelined_load_s"] == pytest.approx(blob * 8 / 100e6 + 0.0005)
    assert r["speedup_vs_raw"] == pytest.approx(r["raw_transfer_s"] / r["pipelined_load_s"])
