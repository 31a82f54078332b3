"""Helpers for the GPU tests: run every stage of the HIP library through the
C ABI on seeded inputs and bring the results back to numpy, plus the bf16 ulp
distance used for the dequantised output. Test-only."""

from __future__ import annotations

import numpy as np

from kv_cache_compression_layer_amd import cachegen as cgb


def torch_mod():
    import torch

    return torch


def to_dev(a: np.ndarray):
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda:0")


def to_np(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """|a - b| in units of bf16 ulps (signed-magnitude mapped to a line)."""

    def line(b):
        b = b.astype(np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)

    return np.abs(line(a_bits.view(np.uint16)) - line(b_bits.view(np.uint16)))


def assert_bf16_equal(got_bits: np.ndarray, want_bits: np.ndarray, what: str = "") -> None:
    """Bit-for-bit equality of two bf16 arrays (so +0 and -0 differ too); on a
    mismatch the message gives the count and the largest ulp distance."""
    g = np.asarray(got_bits).view(np.uint16).reshape(-1)
    w = np.asarray(want_bits).view(np.uint16).reshape(-1)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = g != w
    if bad.any():
        i = int(np.argmax(bad))
        raise AssertionError(f"{what}: {int(bad.sum())} of {g.size} bf16 values differ, largest "
                             f"{int(bf16_ulp_distance(g[bad], w[bad]).max())} ulp; first at {i}: "
                             f"{g[i]:#06x} vs {w[i]:#06x}")


def run_stages(kv_bits: np.ndarray, bins_k, bins_v, table_format=0):
    """All stage calls on the GPU. kv_bits: uint16 [L,2,T,H,D]."""
    torch = torch_mod()
    desc = cgb.Desc.for_kv(kv_bits.shape, bins_k, bins_v, table_format)
    L, T, C, A = desc.nlayers, desc.ntokens, desc.nchannels, desc.alphabet
    kv = to_dev(kv_bits)
    dev = kv.device
    out = {}
    sym = torch.empty(2 * L * T * C, dtype=torch.uint8, device=dev)
    scale = torch.empty(2 * L * T, dtype=torch.int16, device=dev)
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_QUANTIZE)
    cgb.cg_quantize(desc, kv, sym, scale, ws)
    out["quantize_status"] = cgb.cg_read_status(ws)
    cdf = torch.empty(2 * L * C * (A + 1), dtype=torch.int32, device=dev)
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_BUILD_CDF)
    cgb.cg_build_cdf(desc, sym, cdf, ws)
    out["cdf_status"] = cgb.cg_read_status(ws)
    payload = torch.empty(cgb.cg_encode_bound(desc), dtype=torch.uint8, device=dev)
    lengths = torch.empty(desc.nstreams, dtype=torch.int16, device=dev)
    chunk_off = torch.empty(desc.nchunks + 1, dtype=torch.int64, device=dev)
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_ENCODE)
    cgb.cg_encode(desc, sym, cdf, payload, lengths, chunk_off, ws)
    out["encode_status"] = cgb.cg_read_status(ws)
    nbytes = int(chunk_off[-1].item())
    sym2 = torch.full_like(sym, 255)
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_DECODE)
    cgb.cg_decode(desc, payload, nbytes, lengths, chunk_off, cdf, sym2, ws)
    out["decode_status"] = cgb.cg_read_status(ws)
    kv_out = torch.empty(2 * L * T * C, dtype=torch.int16, device=dev)
    cgb.cg_dequantize(desc, sym2, scale, kv_out)
    torch.cuda.synchronize()
    NC = desc.nchunks
    out.update(
        sym=to_np(sym).reshape(2, L, T, C),
        scale=to_np(scale, np.uint16).reshape(2, L, T),
        cdf=to_np(cdf).reshape(2, L, C, A + 1),
        payload=to_np(payload[:nbytes]),
        lengths=to_np(lengths, np.uint16).reshape(NC, 2 * L, C),
        chunk_off=to_np(chunk_off, np.uint64),
        sym_decoded=to_np(sym2).reshape(2, L, T, C),
        kv_out=to_np(kv_out, np.uint16).reshape(L, 2, T, C),
    )
    return out


def run_coder(sym_np: np.ndarray, cdf_np: np.ndarray, desc):
    """cg_encode then cg_decode on given symbols [2,L,T,C] and tables [2,L,C,A+1]."""
    torch = torch_mod()
    sym = to_dev(np.ascontiguousarray(sym_np, np.uint8)).reshape(-1)
    cdf = to_dev(np.ascontiguousarray(cdf_np, np.int32)).reshape(-1)
    payload = torch.empty(cgb.cg_encode_bound(desc), dtype=torch.uint8, device="cuda:0")
    lengths = torch.empty(desc.nstreams, dtype=torch.int16, device="cuda:0")
    chunk_off = torch.empty(desc.nchunks + 1, dtype=torch.int64, device="cuda:0")
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_ENCODE)
    cgb.cg_encode(desc, sym, cdf, payload, lengths, chunk_off, ws)
    enc_status = cgb.cg_read_status(ws)
    nbytes = int(chunk_off[-1].item())
    out = torch.full_like(sym, 255)
    ws = cgb.alloc_workspace(desc, cgb.CG_OP_DECODE)
    cgb.cg_decode(desc, payload, nbytes, lengths, chunk_off, cdf, out, ws)
    dec_status = cgb.cg_read_status(ws)
    NC = desc.nchunks
    return dict(
        encode_status=enc_status,
        decode_status=dec_status,
        payload=to_np(payload[:nbytes]),
        lengths=to_np(lengths, np.uint16).reshape(NC, 2 * desc.nlayers, desc.nchannels),
        chunk_off=to_np(chunk_off, np.uint64),
        sym_decoded=to_np(out).reshape(sym_np.shape),
    )
