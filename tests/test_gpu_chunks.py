"""Oracle parity at the chunk counts where the coders change launch shape.

The encoder takes four-wave blocks from 8 chunks on. The fused, stage,
paged and chunk-range decoders take four-wave blocks at 8..15 chunks and
eight-wave blocks from 16 on, counted over the chunks they decode. These
cases reach 9, 12, 16 and 17 chunks (most with a short last chunk) at small
layer and channel counts. Each case runs every entry point and checks it
against the oracle bit for bit:

- cg_to_bytes (the blob) and cg_from_bytes (the decode of the oracle's own
  blob);
- the stage calls cg_quantize, cg_build_cdf, cg_encode, cg_decode and
  cg_dequantize;
- cg_from_bytes_paged through a shuffled block table;
- cg_from_bytes_chunks over ranges of 1, 8, 9 and 16+ chunks;
- the pipelined load in pieces of 8 and 16 chunks.

The cases mix 16- and 32-bin slabs. They include all-16 and all-32 bins
with C = 256 and T % 8 == 0 (the fused quantiser's packed nibble and byte
layouts), a channel count that is not a multiple of 64, and per-layer
tables.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import assert_bf16_equal, run_stages, to_dev, to_np
from kv_cache_compression_layer_amd import cachegen as cgb
from kv_cache_compression_layer_amd import streaming
from kv_cache_compression_layer_amd.synth import generate_kv

pytestmark = pytest.mark.gpu

SENTINEL = 0x7F7F  # a bf16 bit pattern no decode produces

CASES = [
    # name, L, T, H, D, bins_k, bins_v, table format
    ("c9_mixed_c128", 2, 2148, 1, 128, [32, 16], [16, 16], 0),
    ("c17_mixed_c128", 2, 4200, 1, 128, [32, 16], [16, 16], 0),
    ("c16_nibbles_c256", 2, 4096, 2, 128, [16, 16], [16, 16], 0),
    ("c9_bytes_c256", 2, 2304, 2, 128, [32, 32], [32, 32], 0),
    ("c17_mixed_c256", 2, 4104, 2, 128, [32, 16], [16, 16], 0),
    ("c17_c96_per_layer", 2, 4200, 3, 32, [32, 16], [16, 8], 1),
    ("c12_c1024_default", 3, 3000, 8, 128, None, None, 0),
]


def _case(case):
    name, L, T, H, D, bk, bv, fmt = case
    kv = generate_kv(L, T, H, D, outlier_frac=0.02, outlier_scale=15.0, seed=5000 + T + 7 * H)
    if bk is None:
        bk, bv = oracle.default_bins(L)
    return kv, np.array(bk, np.uint8), np.array(bv, np.uint8), fmt


@pytest.fixture(scope="module", params=CASES, ids=[c[0] for c in CASES])
def case(request):
    kv, bk, bv, fmt = _case(request.param)
    print(f"[{request.param[0]}] oracle on {kv.shape}", flush=True)
    want = oracle.to_bytes(kv, bk, bv, fmt)
    ref = np.asarray(oracle.from_bytes(want)).view(np.uint16)
    return dict(kv=kv, bk=bk, bv=bv, fmt=fmt, want=want, ref=ref, name=request.param[0])


def test_whole_blob_both_ways(case):
    import torch

    kv, bk, bv, fmt = case["kv"], case["bk"], case["bv"], case["fmt"]
    blob = cgb.to_bytes(to_dev(kv).view(torch.bfloat16), bk, bv, table_format=fmt)
    got = to_np(blob).tobytes()
    assert len(got) == len(case["want"]) and got == case["want"]
    # Decode the oracle's blob (the same bytes) on the device.
    dev_blob = to_dev(np.frombuffer(case["want"], np.uint8).copy())
    out = to_np(cgb.from_bytes(dev_blob).view(torch.int16), np.uint16)
    assert_bf16_equal(out, case["ref"], "cg_from_bytes")


def test_stage_calls(case):
    kv, bk, bv, fmt = case["kv"], case["bk"], case["bv"], case["fmt"]
    g = run_stages(kv, bk, bv, fmt)
    for k in ("quantize_status", "cdf_status", "encode_status", "decode_status"):
        assert g[k] == cgb.CG_OK, k
    sym, scale = oracle.quantize(kv, bk, bv)
    np.testing.assert_array_equal(g["scale"], scale)
    np.testing.assert_array_equal(g["sym"], sym)
    A = oracle.alphabet(bk, bv)
    widths = oracle.table_widths(bk, bv, fmt)
    cdf = oracle.build_cdf(sym, A, widths)
    np.testing.assert_array_equal(g["cdf"], cdf)
    payload, lengths, chunk_off = oracle.encode(sym, cdf, widths)
    np.testing.assert_array_equal(g["lengths"], lengths)
    np.testing.assert_array_equal(g["chunk_off"], chunk_off)
    assert g["payload"].size == payload.size
    np.testing.assert_array_equal(g["payload"], payload)
    np.testing.assert_array_equal(g["sym_decoded"], sym)
    L, T, C = kv.shape[0], kv.shape[2], kv.shape[3] * kv.shape[4]
    assert_bf16_equal(g["kv_out"], case["ref"].reshape(L, 2, T, C), "cg_dequantize")


@pytest.mark.parametrize("bs", [16, 256])
def test_paged(case, bs):
    import torch

    kv, bk, bv, fmt = case["kv"], case["bk"], case["bv"], case["fmt"]
    L, _, T, H, D = kv.shape
    C = H * D
    desc = cgb.Desc(L, T, H, D, bk, bv, fmt)
    blob = to_dev(np.frombuffer(case["want"], np.uint8).copy())
    nblk = (T + bs - 1) // bs
    num_blocks = nblk + 3
    table = np.random.default_rng(bs + T).permutation(num_blocks)[:nblk].astype(np.int32)
    cache = torch.full((L, 2, num_blocks, bs, C), SENTINEL, dtype=torch.int16, device="cuda:0")
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES)
    cgb.cg_from_bytes_paged(desc, blob, len(case["want"]), cache, 2 * num_blocks * bs * C, num_blocks * bs * C,
                            bs, to_dev(table), num_blocks, ws)
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    got_cache = to_np(cache, np.uint16)
    got = np.concatenate([got_cache[:, :, table[b], : min(bs, T - b * bs), :] for b in range(nblk)], axis=2)
    assert_bf16_equal(got, case["ref"].reshape(L, 2, T, C), f"paged bs={bs}")
    used = np.zeros(num_blocks, bool)
    used[table] = True
    assert np.all(got_cache[:, :, ~used] == SENTINEL)


def test_chunk_ranges(case):
    import torch

    kv, bk, bv, fmt = case["kv"], case["bk"], case["bv"], case["fmt"]
    L, _, T, H, D = kv.shape
    C = H * D
    desc = cgb.Desc(L, T, H, D, bk, bv, fmt)
    nc = desc.nchunks
    lay = cgb.cg_blob_layout(desc)
    want = np.frombuffer(case["want"], np.uint8).copy()
    chunk_off = want[lay["off_chunk_off"] : lay["off_chunk_off"] + 8 * (nc + 1)].view(np.uint64)
    ref = case["ref"].reshape(L, 2, T, C)
    ranges = {(0, nc), (0, min(8, nc)), (1, nc), (max(0, nc - 9), nc), (nc - 1, nc), (2, min(nc, 18))}
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES)
    for j0, j1 in sorted(ranges):
        need = int(lay["off_payload"] + chunk_off[j1])
        part = torch.full((want.size,), 0xAB, dtype=torch.uint8, device="cuda:0")
        part[:need] = to_dev(want[:need])
        out = torch.full((L * 2 * T * C,), SENTINEL, dtype=torch.int16, device="cuda:0")
        cgb.cg_from_bytes_chunks(desc, part, need, j0, j1, out, ws)
        assert cgb.cg_read_status(ws) == cgb.CG_OK, (j0, j1)
        got = to_np(out, np.uint16).reshape(L, 2, T, C)
        t0, t1 = 256 * j0, min(T, 256 * j1)
        assert_bf16_equal(got[:, :, t0:t1], ref[:, :, t0:t1], f"chunks [{j0}, {j1})")
        assert np.all(got[:, :, :t0] == SENTINEL) and np.all(got[:, :, t1:] == SENTINEL)


@pytest.mark.parametrize("chunks_per_piece", [8, 16])
def test_pipelined_load(case, chunks_per_piece):
    import torch

    kv, bk, bv, fmt = case["kv"], case["bk"], case["bv"], case["fmt"]
    L, _, T, H, D = kv.shape
    desc = cgb.Desc(L, T, H, D, bk, bv, fmt)
    lay = cgb.cg_blob_layout(desc)
    want = np.frombuffer(case["want"], np.uint8).copy()
    nc = desc.nchunks
    chunk_off = want[lay["off_chunk_off"] : lay["off_chunk_off"] + 8 * (nc + 1)].view(np.uint64)
    host = torch.empty(want.size, dtype=torch.uint8, pin_memory=True)
    host.copy_(torch.from_numpy(want))
    dev_blob = torch.zeros(want.size, dtype=torch.uint8, device="cuda:0")
    out = torch.full((L * 2 * T * H * D,), SENTINEL, dtype=torch.int16, device="cuda:0")
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES)
    pieces = streaming.plan_pieces(int(lay["off_payload"]), chunk_off, chunks_per_piece)
    copy_s, dec_s = torch.cuda.Stream(), torch.cuda.Stream()
    streaming.enqueue_pipelined_load(desc, host, dev_blob, out, ws, pieces, copy_s, dec_s)
    torch.cuda.synchronize()
    assert cgb.cg_read_status(ws) == cgb.CG_OK
    assert_bf16_equal(to_np(out, np.uint16), case["ref"], f"pipelined, {chunks_per_piece} chunks per piece")
