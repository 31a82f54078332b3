"""The C ABI on the CPU: the library loads, exports every declared symbol, and
its host-side logic (bins rule, descriptor checks, sizes, blob layout, header
parsing) agrees with independent expectations. No device call is made."""

import math
import os
import re

import numpy as np
import pytest

import oracle
from kv_cache_compression_layer_amd import cachegen as cgb
from kv_cache_compression_layer_amd.build import LIB_PATH
from kv_cache_compression_layer_amd.synth import generate_kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "cachegen.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cg_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(LIB_PATH):
        from kv_cache_compression_layer_amd.build import build

        build()


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 17
    lib = cgb.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(cgb._SIGNATURES) == set(names)
    assert lib.cg_version() == 2


def test_default_bins_matches_oracle():
    for L in [1, 2, 9, 10, 11, 12, 32, 40, 1024]:
        bk, bv = cgb.cg_default_bins(L)
        ok, ov = oracle.default_bins(L)
        np.testing.assert_array_equal(bk, ok)
        np.testing.assert_array_equal(bv, ov)


def test_desc_validation():
    with pytest.raises(ValueError):
        cgb.Desc(0, 10, 1, 1)
    with pytest.raises(ValueError):
        cgb.Desc(2, 0, 1, 1)
    with pytest.raises(ValueError):
        cgb.Desc(2, 10, 1, 8, bins_k=[3, 32], bins_v=[32, 32])  # bins < 4
    with pytest.raises(ValueError):
        cgb.Desc(2, 10, 1, 8, bins_k=[32, 129], bins_v=[32, 32])  # bins > 128
    with pytest.raises(ValueError):
        cgb.Desc(1025, 10, 1, 1)
    d = cgb.Desc(2, 10, 1, 8, bins_k=[4, 128], bins_v=[32, 5])
    assert d.alphabet == 128


def _layout(L, T, C, A):
    up = lambda x: (x + 63) // 64 * 64
    NC = math.ceil(T / 256)
    o = {}
    o["header_bytes"] = up(48 + 2 * L)
    o["off_scales"] = o["header_bytes"]
    o["off_cdf"] = o["off_scales"] + up(4 * L * T)
    o["off_chunk_off"] = o["off_cdf"] + up(4 * L * C * A)
    o["off_lengths"] = o["off_chunk_off"] + up(8 * (NC + 1))
    o["off_payload"] = o["off_lengths"] + up(4 * NC * L * C)
    return o


@pytest.mark.parametrize("L,T,H,D", [(12, 64, 12, 64), (32, 32768, 8, 128), (1, 1, 1, 1), (3, 513, 5, 26)])
def test_sizes_and_layout(L, T, H, D):
    d = cgb.Desc(L, T, H, D)
    C, A = H * D, d.alphabet
    NC = math.ceil(T / 256)
    NS = NC * 2 * L * C
    assert cgb.cg_encode_bound(d) == NS * 513
    lay = cgb.cg_blob_layout(d)
    for k, v in _layout(L, T, C, A).items():
        assert lay[k] == v, k
    assert cgb.cg_blob_bound(d) == lay["off_payload"] + NS * 513
    tiles = NC * 2 * L * math.ceil(C / 64)
    assert cgb.cg_workspace_bytes(d, cgb.CG_OP_QUANTIZE) == 256
    assert cgb.cg_workspace_bytes(d, cgb.CG_OP_ENCODE) >= 256 + 12 * tiles
    assert cgb.cg_workspace_bytes(d, cgb.CG_OP_TO_BYTES) >= 2 * L * T * C
    with pytest.raises(ValueError):
        cgb.cg_workspace_bytes(d, 99)


def test_peek_parses_an_oracle_blob():
    L, T, H, D = 3, 300, 2, 16
    kv = generate_kv(L, T, H, D, seed=4)
    bk = np.array([32, 16, 8], np.uint8)
    bv = np.array([128, 4, 16], np.uint8)
    blob = oracle.to_bytes(kv, bk, bv)
    info, pk, pv = cgb.cg_blob_peek(blob[:48 + 2 * L])
    assert (info["nlayers"], info["ntokens"], info["nheads"], info["head_size"]) == (L, T, H, D)
    assert info["nchunks"] == 2 and info["alphabet"] == 128 and info["chunk_tokens"] == 256
    assert info["blob_size"] == len(blob)
    np.testing.assert_array_equal(pk, bk)
    np.testing.assert_array_equal(pv, bv)
    lay = cgb.cg_blob_layout(cgb.Desc(L, T, H, D, bk, bv))
    for k in ["off_scales", "off_cdf", "off_chunk_off", "off_lengths", "off_payload"]:
        assert info[k] == lay[k]


def test_peek_rejects_bad_headers():
    kv = generate_kv(2, 10, 1, 8, seed=1)
    bk, bv = oracle.default_bins(2)
    blob = bytearray(oracle.to_bytes(kv, bk, bv))
    good = bytes(blob[:52])
    cgb.cg_blob_peek(good)
    for pos, val in [(0, ord("X")), (4, 2), (6, 7), (8, 0), (24, 128), (28, 9), (32, 31), (36, 2), (48, 3)]:
        bad = bytearray(good)
        bad[pos] = val
        with pytest.raises(ValueError):
            cgb.cg_blob_peek(bytes(bad))
    with pytest.raises(ValueError):
        cgb.cg_blob_peek(good[:50])  # bins cut off


def test_per_layer_tables_layout_and_peek():
    """The per-layer table format: the library's layout and header parse
    agree with an oracle blob parsed independently."""
    from blob_format import parse

    L, T, H, D = 12, 300, 2, 16
    kv = generate_kv(L, T, H, D, seed=8)
    bk, bv = oracle.default_bins(L)
    blob = oracle.to_bytes(kv, bk, bv, 1)
    p = parse(blob)
    info, pk, pv = cgb.cg_blob_peek(blob[:48 + 2 * L])
    assert info["table_format"] == 1 and info["blob_size"] == len(blob)
    d = cgb.Desc(L, T, H, D, bk, bv, cgb.CG_TABLES_PER_LAYER)
    lay = cgb.cg_blob_layout(d)
    assert lay["table_format"] == 1
    for k in ["off_scales", "off_cdf", "off_chunk_off", "off_lengths", "off_payload"]:
        assert info[k] == lay[k], k
    assert lay["off_payload"] == len(blob) - len(p["payload"])
    assert lay["off_chunk_off"] - lay["off_cdf"] == (2 * H * D * int(p["widths"].sum()) + 63) // 64 * 64
    shared = cgb.cg_blob_layout(cgb.Desc(L, T, H, D, bk, bv))
    assert shared["table_format"] == 0 and shared["off_payload"] > lay["off_payload"]
    with pytest.raises(ValueError):
        cgb.Desc(L, T, H, D, bk, bv, 2)


def test_strerror():
    assert "workspace" in cgb.strerror(cgb.CG_E_WORKSPACE)
    assert cgb.strerror(0) == "ok"


def test_shape_limits_are_rejected():
    bk, bv = oracle.default_bins(2)
    for shape in [(2, 0, 1, 8), (0, 4, 1, 8), (2, 4, 0, 8), (1025, 4, 1, 8)]:
        L = shape[0]
        b = np.full(max(L, 1), 16, np.uint8)
        with pytest.raises(ValueError):
            cgb.Desc(*shape, b[:L], b[:L])
    with pytest.raises(ValueError):  # one (K|V, layer) slab of 2^31 elements
        cgb.Desc(2, 1 << 21, 8, 128, bk, bv)
    with pytest.raises(ValueError):  # batch beyond 32767 layers
        cgb.cg_workspace_bytes_batch(cgb.Desc(32, 16, 1, 64), 1024, 1 << 20, cgb.CG_OP_TO_BYTES)
