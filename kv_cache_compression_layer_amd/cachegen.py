"""Python binding of libcachegen_mi355x.so (see include/cachegen.h).

Argument marshalling only: every step of the codec runs in the library's HIP
kernels. torch supplies device memory and the current stream. The functions
named ``cg_*`` mirror the C entry points one to one; :func:`to_bytes` and
:func:`from_bytes` are conveniences that allocate their buffers with torch and
wait for the result.

The library must be built (``python -m kv_cache_compression_layer_amd.build``).
If it is missing, loading raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import numpy as np

from .build import LIB_PATH

# Status codes (include/cachegen.h).
CG_OK = 0
CG_E_INVAL = -1
CG_E_SHAPE = -2
CG_E_CAPACITY = -3
CG_E_CORRUPT = -4
CG_E_NONFINITE = -5
CG_E_HIP = -6
CG_E_WORKSPACE = -7

CG_OP_QUANTIZE = 0
CG_OP_BUILD_CDF = 1
CG_OP_ENCODE = 2
CG_OP_DECODE = 3
CG_OP_DEQUANTIZE = 4
CG_OP_TO_BYTES = 5
CG_OP_FROM_BYTES = 6

CG_TABLES_SHARED = 0
CG_TABLES_PER_LAYER = 1

CHUNK_TOKENS = 256
MAX_LAYERS = 1024
MAX_STREAM_BYTES = 513
WS_ALIGN = 256


class CgDescC(ctypes.Structure):
    _fields_ = [
        ("nlayers", ctypes.c_int32),
        ("ntokens", ctypes.c_int32),
        ("nheads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("bins_k", ctypes.c_void_p),
        ("bins_v", ctypes.c_void_p),
        ("table_format", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class CgBlobInfoC(ctypes.Structure):
    _fields_ = [
        ("nlayers", ctypes.c_int32),
        ("ntokens", ctypes.c_int32),
        ("nheads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("chunk_tokens", ctypes.c_int32),
        ("nchunks", ctypes.c_int32),
        ("alphabet", ctypes.c_int32),
        ("table_format", ctypes.c_int32),
        ("blob_size", ctypes.c_uint64),
        ("header_bytes", ctypes.c_uint64),
        ("off_scales", ctypes.c_uint64),
        ("off_cdf", ctypes.c_uint64),
        ("off_chunk_off", ctypes.c_uint64),
        ("off_lengths", ctypes.c_uint64),
        ("off_payload", ctypes.c_uint64),
    ]


class CacheGenError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})")


class CacheGenValueError(CacheGenError, ValueError):
    """Bad argument, shape, blob or input values (the pages raise ValueError)."""


_lib = None

# name -> (restype, argtypes)
_P, _SZ, _I32, _I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
_SIGNATURES = {
    "cg_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "cg_version": (ctypes.c_int, []),
    "cg_default_bins": (ctypes.c_int, [_I32, _P, _P]),
    "cg_desc_check": (ctypes.c_int, [_P]),
    "cg_workspace_bytes": (_I64, [_P, ctypes.c_int]),
    "cg_encode_bound": (_I64, [_P]),
    "cg_blob_bound": (_I64, [_P]),
    "cg_blob_layout": (ctypes.c_int, [_P, _P]),
    "cg_blob_peek": (ctypes.c_int, [_P, _SZ, _P, _P, _P, _I32]),
    "cg_read_status": (ctypes.c_int, [_P, _P]),
    "cg_quantize": (ctypes.c_int, [_P, _P, _P, _P, _P, _SZ, _P]),
    "cg_build_cdf": (ctypes.c_int, [_P, _P, _P, _P, _SZ, _P]),
    "cg_encode": (ctypes.c_int, [_P, _P, _P, _P, _SZ, _P, _P, _P, _SZ, _P]),
    "cg_decode": (ctypes.c_int, [_P, _P, _SZ, _P, _P, _P, _P, _P, _SZ, _P]),
    "cg_dequantize": (ctypes.c_int, [_P, _P, _P, _P, _P, _SZ, _P]),
    "cg_to_bytes": (ctypes.c_int, [_P, _P, _P, _SZ, _P, _P, _SZ, _P]),
    "cg_from_bytes": (ctypes.c_int, [_P, _P, _SZ, _P, _P, _SZ, _P]),
    "cg_from_bytes_noalloc": (ctypes.c_int, [_P, _P, _SZ, _P, _P, _P]),
    "cg_from_bytes_paged": (ctypes.c_int, [_P, _P, _SZ, _P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                           _P, ctypes.c_int32, _P, _SZ, _P]),
    "cg_from_bytes_chunks": (ctypes.c_int, [_P, _P, _SZ, _I32, _I32, _P, _P, _SZ, _P]),
    "cg_workspace_bytes_batch": (_I64, [_P, _I32, _SZ, ctypes.c_int]),
    "cg_to_bytes_batch": (ctypes.c_int, [_P, _I32, _P, _P, _SZ, _P, _P, _SZ, _P]),
    "cg_from_bytes_batch": (ctypes.c_int, [_P, _I32, _P, _SZ, _P, _P, _P, _SZ, _P]),
}


def lib():
    """Load libcachegen_mi355x.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m kv_cache_compression_layer_amd.build`"
            )
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().cg_strerror(code).decode()


def _check(rc: int, what: str) -> int:
    if rc < 0:
        if rc in (CG_E_HIP,):
            raise CacheGenError(rc, what)
        raise CacheGenValueError(rc, what)
    return rc


# ------------------------------------------------------------------ desc


class Desc:
    """A cg_desc plus the host bins arrays it points to."""

    def __init__(self, nlayers, ntokens, nheads, head_size, bins_k=None, bins_v=None,
                 table_format=CG_TABLES_SHARED):
        if bins_k is None or bins_v is None:
            dk, dv = cg_default_bins(nlayers)
            bins_k = dk if bins_k is None else bins_k
            bins_v = dv if bins_v is None else bins_v
        self.bins_k = np.ascontiguousarray(bins_k, dtype=np.uint8)
        self.bins_v = np.ascontiguousarray(bins_v, dtype=np.uint8)
        if self.bins_k.shape != (nlayers,) or self.bins_v.shape != (nlayers,):
            raise ValueError("bins_k and bins_v need one entry per layer")
        self.c = CgDescC(nlayers, ntokens, nheads, head_size,
                         self.bins_k.ctypes.data, self.bins_v.ctypes.data, int(table_format), 0)
        _check(lib().cg_desc_check(self.ptr), "cg_desc_check")

    @classmethod
    def for_kv(cls, shape, bins_k=None, bins_v=None, table_format=CG_TABLES_SHARED):
        L, two, T, H, D = shape
        if two != 2:
            raise ValueError("KV must be [nlayers, 2, ntokens, nheads, head_size]")
        return cls(L, T, H, D, bins_k, bins_v, table_format)

    @property
    def table_format(self):
        return self.c.table_format

    @property
    def ptr(self):
        return ctypes.addressof(self.c)

    @property
    def nlayers(self):
        return self.c.nlayers

    @property
    def ntokens(self):
        return self.c.ntokens

    @property
    def nchannels(self):
        return self.c.nheads * self.c.head_size

    @property
    def alphabet(self):
        return int(max(self.bins_k.max(), self.bins_v.max()))

    @property
    def nchunks(self):
        return (self.c.ntokens + CHUNK_TOKENS - 1) // CHUNK_TOKENS

    @property
    def kv_shape(self):
        return (self.c.nlayers, 2, self.c.ntokens, self.c.nheads, self.c.head_size)

    @property
    def nstreams(self):
        return self.nchunks * 2 * self.nlayers * self.nchannels


# ------------------------------------------------------------ host calls


def cg_default_bins(nlayers: int):
    bk = np.zeros(nlayers, np.uint8)
    bv = np.zeros(nlayers, np.uint8)
    _check(lib().cg_default_bins(nlayers, bk.ctypes.data, bv.ctypes.data), "cg_default_bins")
    return bk, bv


def cg_workspace_bytes(desc: Desc, op: int) -> int:
    return _check(lib().cg_workspace_bytes(desc.ptr, op), "cg_workspace_bytes")


def cg_encode_bound(desc: Desc) -> int:
    return _check(lib().cg_encode_bound(desc.ptr), "cg_encode_bound")


def cg_blob_bound(desc: Desc) -> int:
    return _check(lib().cg_blob_bound(desc.ptr), "cg_blob_bound")


def _info_dict(info: CgBlobInfoC) -> dict:
    return {name: getattr(info, name) for name, _ in CgBlobInfoC._fields_}


def cg_blob_layout(desc: Desc) -> dict:
    info = CgBlobInfoC()
    _check(lib().cg_blob_layout(desc.ptr, ctypes.addressof(info)), "cg_blob_layout")
    return _info_dict(info)


def cg_blob_peek(header: bytes):
    """Parse a blob header held in host memory -> (info dict, bins_k, bins_v)."""
    buf = np.frombuffer(bytes(header), np.uint8).copy()
    info = CgBlobInfoC()
    bk = np.zeros(MAX_LAYERS, np.uint8)
    bv = np.zeros(MAX_LAYERS, np.uint8)
    _check(lib().cg_blob_peek(buf.ctypes.data, buf.size, ctypes.addressof(info), bk.ctypes.data,
                              bv.ctypes.data, MAX_LAYERS), "cg_blob_peek")
    d = _info_dict(info)
    return d, bk[: d["nlayers"]].copy(), bv[: d["nlayers"]].copy()


# ---------------------------------------------------------- device calls


def _torch():
    import torch

    return torch


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t, name, dtype=None, numel=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _ws(ws, desc, op):
    need = cg_workspace_bytes(desc, op)
    if ws is None:
        raise ValueError("workspace required")
    p = _dev(ws, "ws")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, needs {need}")
    return p, ws.numel() * ws.element_size()


def alloc_workspace(desc: Desc, op: int, device="cuda"):
    """A uint8 device tensor of cg_workspace_bytes(op), 256-byte aligned."""
    torch = _torch()
    need = cg_workspace_bytes(desc, op)
    raw = torch.empty(need + WS_ALIGN, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % WS_ALIGN
    return raw[off : off + need]


def cg_read_status(ws, stream=None) -> int:
    return lib().cg_read_status(_dev(ws, "ws"), _stream_handle(stream))


def cg_quantize(desc, kv, sym, scale, ws, stream=None):
    torch = _torch()
    T, C, L = desc.ntokens, desc.nchannels, desc.nlayers
    p, n = _ws(ws, desc, CG_OP_QUANTIZE)
    _check(lib().cg_quantize(desc.ptr, _dev(kv, "kv", (torch.bfloat16, torch.uint16, torch.int16), 2 * L * T * C),
                             _dev(sym, "sym", torch.uint8, 2 * L * T * C),
                             _dev(scale, "scale", (torch.bfloat16, torch.uint16, torch.int16), 2 * L * T),
                             p, n, _stream_handle(stream)), "cg_quantize")


def cg_build_cdf(desc, sym, cdf, ws, stream=None):
    torch = _torch()
    L, T, C, A = desc.nlayers, desc.ntokens, desc.nchannels, desc.alphabet
    p, n = _ws(ws, desc, CG_OP_BUILD_CDF)
    _check(lib().cg_build_cdf(desc.ptr, _dev(sym, "sym", torch.uint8, 2 * L * T * C),
                              _dev(cdf, "cdf", torch.int32, 2 * L * C * (A + 1)), p, n,
                              _stream_handle(stream)), "cg_build_cdf")


def cg_encode(desc, sym, cdf, payload, lengths, chunk_off, ws, stream=None):
    torch = _torch()
    L, T, C, A = desc.nlayers, desc.ntokens, desc.nchannels, desc.alphabet
    p, n = _ws(ws, desc, CG_OP_ENCODE)
    _check(lib().cg_encode(desc.ptr, _dev(sym, "sym", torch.uint8, 2 * L * T * C),
                           _dev(cdf, "cdf", torch.int32, 2 * L * C * (A + 1)),
                           _dev(payload, "payload", torch.uint8), payload.numel(),
                           _dev(lengths, "lengths", (torch.int16, torch.uint16), desc.nstreams),
                           _dev(chunk_off, "chunk_off", (torch.int64, torch.uint64), desc.nchunks + 1),
                           p, n, _stream_handle(stream)), "cg_encode")


def cg_decode(desc, payload, payload_bytes, lengths, chunk_off, cdf, sym, ws, stream=None):
    torch = _torch()
    L, T, C, A = desc.nlayers, desc.ntokens, desc.nchannels, desc.alphabet
    if payload_bytes > payload.numel():
        raise ValueError("payload_bytes exceeds the payload tensor")
    p, n = _ws(ws, desc, CG_OP_DECODE)
    _check(lib().cg_decode(desc.ptr, _dev(payload, "payload", torch.uint8), payload_bytes,
                           _dev(lengths, "lengths", (torch.int16, torch.uint16), desc.nstreams),
                           _dev(chunk_off, "chunk_off", (torch.int64, torch.uint64), desc.nchunks + 1),
                           _dev(cdf, "cdf", torch.int32, 2 * L * C * (A + 1)),
                           _dev(sym, "sym", torch.uint8, 2 * L * T * C), p, n,
                           _stream_handle(stream)), "cg_decode")


def cg_dequantize(desc, sym, scale, kv_out, ws=None, stream=None):
    torch = _torch()
    L, T, C = desc.nlayers, desc.ntokens, desc.nchannels
    if ws is not None:
        p, n = _dev(ws, "ws"), ws.numel() * ws.element_size()
    else:
        p, n = None, 0
    _check(lib().cg_dequantize(desc.ptr, _dev(sym, "sym", torch.uint8, 2 * L * T * C),
                               _dev(scale, "scale", (torch.bfloat16, torch.uint16, torch.int16), 2 * L * T),
                               _dev(kv_out, "kv_out", (torch.bfloat16, torch.uint16, torch.int16), 2 * L * T * C),
                               p, n, _stream_handle(stream)), "cg_dequantize")


def cg_to_bytes(desc, kv, blob, blob_size_dev, ws, stream=None):
    torch = _torch()
    L, T, C = desc.nlayers, desc.ntokens, desc.nchannels
    p, n = _ws(ws, desc, CG_OP_TO_BYTES)
    _check(lib().cg_to_bytes(desc.ptr, _dev(kv, "kv", (torch.bfloat16, torch.uint16, torch.int16), 2 * L * T * C),
                             _dev(blob, "blob", torch.uint8), blob.numel(),
                             _dev(blob_size_dev, "blob_size_dev", (torch.int64, torch.uint64), 1),
                             p, n, _stream_handle(stream)), "cg_to_bytes")


def cg_from_bytes(desc, blob, blob_size, kv_out, ws, stream=None):
    torch = _torch()
    L, T, C = desc.nlayers, desc.ntokens, desc.nchannels
    if blob_size > blob.numel():
        raise ValueError("blob_size exceeds the blob tensor")
    p, n = _ws(ws, desc, CG_OP_FROM_BYTES)
    _check(lib().cg_from_bytes(desc.ptr, _dev(blob, "blob", torch.uint8), blob_size,
                               _dev(kv_out, "kv_out", (torch.bfloat16, torch.uint16, torch.int16), 2 * L * T * C),
                               p, n, _stream_handle(stream)), "cg_from_bytes")


def cg_from_bytes_noalloc(desc, blob, blob_size, kv_out, status, stream=None):
    """cg_from_bytes with the library's own fixed workspace (no allocation);
    status: a device int32/uint32 tensor of at least one element that
    receives the status word (read it with cg_read_status(status))."""
    torch = _torch()
    L, T, C = desc.nlayers, desc.ntokens, desc.nchannels
    if blob_size > blob.numel():
        raise ValueError("blob_size exceeds the blob tensor")
    _check(lib().cg_from_bytes_noalloc(desc.ptr, _dev(blob, "blob", torch.uint8), blob_size,
                                       _dev(kv_out, "kv_out", (torch.bfloat16, torch.uint16, torch.int16),
                                            2 * L * T * C),
                                       _dev(status, "status", (torch.int32, torch.uint32), 1),
                                       _stream_handle(stream)), "cg_from_bytes_noalloc")


def cg_from_bytes_chunks(desc, blob, blob_size, chunk_begin, chunk_end, kv_out, ws, stream=None):
    """Decode chunks [chunk_begin, chunk_end) of a blob whose first blob_size
    bytes have arrived; writes those tokens of kv_out [L,2,T,H,D]."""
    torch = _torch()
    L, T, C = desc.nlayers, desc.ntokens, desc.nchannels
    if blob_size > blob.numel():
        raise ValueError("blob_size exceeds the blob tensor")
    p, n = _ws(ws, desc, CG_OP_FROM_BYTES)
    _check(lib().cg_from_bytes_chunks(desc.ptr, _dev(blob, "blob", torch.uint8), blob_size, chunk_begin, chunk_end,
                                      _dev(kv_out, "kv_out", (torch.bfloat16, torch.uint16, torch.int16),
                                           2 * L * T * C),
                                      p, n, _stream_handle(stream)), "cg_from_bytes_chunks")


def cg_from_bytes_paged(desc, blob, blob_size, kv_cache, layer_stride, kv_stride, block_size, block_table,
                        num_blocks, ws, stream=None):
    """from_bytes into a paged cache: token t of (layer l, K|V kv) goes to row
    block_table[t // block_size] * block_size + t % block_size of the (l, kv)
    region kv_cache[l*layer_stride + kv*kv_stride:] (strides in elements)."""
    torch = _torch()
    T = desc.ntokens
    if blob_size > blob.numel():
        raise ValueError("blob_size exceeds the blob tensor")
    if block_size < 4 or block_size & (block_size - 1):
        raise CacheGenValueError(CG_E_INVAL, "block_size must be a power of two >= 4")
    nblk = (T + block_size - 1) // block_size
    C = desc.nchannels
    need = (desc.nlayers - 1) * layer_stride + kv_stride + num_blocks * block_size * C
    p, n = _ws(ws, desc, CG_OP_FROM_BYTES)
    _check(lib().cg_from_bytes_paged(desc.ptr, _dev(blob, "blob", torch.uint8), blob_size,
                                     _dev(kv_cache, "kv_cache", (torch.bfloat16, torch.uint16, torch.int16), need),
                                     layer_stride, kv_stride, block_size,
                                     _dev(block_table, "block_table", torch.int32, nblk), num_blocks,
                                     p, n, _stream_handle(stream)), "cg_from_bytes_paged")


def cg_workspace_bytes_batch(desc: Desc, batch: int, blob_stride: int, op: int) -> int:
    return _check(lib().cg_workspace_bytes_batch(desc.ptr, batch, blob_stride, op), "cg_workspace_bytes_batch")


def alloc_workspace_batch(desc: Desc, batch: int, blob_stride: int, op: int, device="cuda"):
    """A uint8 device tensor of cg_workspace_bytes_batch(...), 256-byte aligned."""
    torch = _torch()
    need = cg_workspace_bytes_batch(desc, batch, blob_stride, op)
    raw = torch.empty(need + WS_ALIGN, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % WS_ALIGN
    return raw[off : off + need]


def _ws_batch(ws, desc, batch, blob_stride, op):
    need = cg_workspace_bytes_batch(desc, batch, blob_stride, op)
    if ws is None:
        raise ValueError("workspace required")
    p = _dev(ws, "ws")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, needs {need}")
    return p, ws.numel() * ws.element_size()


def cg_to_bytes_batch(desc, batch, kv, blobs, blob_stride, blob_sizes_dev, ws, stream=None):
    """`batch` calls of one shape: kv [batch, L, 2, T, H, D] -> blob b at
    blobs[b * blob_stride:], its size in blob_sizes_dev[b]."""
    torch = _torch()
    L, T, C = desc.nlayers, desc.ntokens, desc.nchannels
    p, n = _ws_batch(ws, desc, batch, blob_stride, CG_OP_TO_BYTES)
    _check(lib().cg_to_bytes_batch(desc.ptr, batch,
                                   _dev(kv, "kv", (torch.bfloat16, torch.uint16, torch.int16), batch * 2 * L * T * C),
                                   _dev(blobs, "blobs", torch.uint8, batch * blob_stride), blob_stride,
                                   _dev(blob_sizes_dev, "blob_sizes_dev", (torch.int64, torch.uint64), batch),
                                   p, n, _stream_handle(stream)), "cg_to_bytes_batch")


def cg_from_bytes_batch(desc, batch, blobs, blob_stride, blob_sizes_dev, kv_out, ws, stream=None):
    """Decode `batch` blobs of one shape (blob b at blobs[b * blob_stride:],
    size blob_sizes_dev[b]) -> kv_out [batch, L, 2, T, H, D]."""
    torch = _torch()
    L, T, C = desc.nlayers, desc.ntokens, desc.nchannels
    p, n = _ws_batch(ws, desc, batch, blob_stride, CG_OP_FROM_BYTES)
    _check(lib().cg_from_bytes_batch(desc.ptr, batch, _dev(blobs, "blobs", torch.uint8, batch * blob_stride),
                                     blob_stride,
                                     _dev(blob_sizes_dev, "blob_sizes_dev", (torch.int64, torch.uint64), batch),
                                     _dev(kv_out, "kv_out", (torch.bfloat16, torch.uint16, torch.int16),
                                          batch * 2 * L * T * C),
                                     p, n, _stream_handle(stream)), "cg_from_bytes_batch")


# ------------------------------------------------------- conveniences


def check_status(ws, stream=None, what="device status"):
    _check(cg_read_status(ws, stream), what)


def to_bytes(kv, bins_k=None, bins_v=None, stream=None, table_format=CG_TABLES_SHARED):
    """Encode bf16 KV [L,2,T,H,D] on the device -> uint8 device tensor (the blob)."""
    torch = _torch()
    desc = Desc.for_kv(tuple(kv.shape), bins_k, bins_v, table_format)
    blob = torch.empty(cg_blob_bound(desc), dtype=torch.uint8, device=kv.device)
    size = torch.zeros(1, dtype=torch.int64, device=kv.device)
    ws = alloc_workspace(desc, CG_OP_TO_BYTES, kv.device)
    cg_to_bytes(desc, kv.contiguous(), blob, size, ws, stream)
    check_status(ws, stream, "cg_to_bytes")
    return blob[: int(size.item())]


def peek(blob):
    """Read the header of a device or host blob -> (info, bins_k, bins_v)."""
    head = blob[:48]
    head = head.cpu().numpy().tobytes() if hasattr(head, "cpu") else bytes(head)
    L = int.from_bytes(head[8:12], "little")
    n = min(48 + 2 * max(L, 0), len(blob))
    h = blob[:n]
    return cg_blob_peek(h.cpu().numpy().tobytes() if hasattr(h, "cpu") else bytes(h))


def from_bytes(blob, stream=None, out=None):
    """Decode a device blob -> bf16 KV [L,2,T,H,D] on the same device."""
    torch = _torch()
    info, bk, bv = peek(blob)
    if info["blob_size"] != blob.numel():
        raise CacheGenValueError(CG_E_CORRUPT, "blob size disagrees with its header")
    desc = Desc(info["nlayers"], info["ntokens"], info["nheads"], info["head_size"], bk, bv, info["table_format"])
    if out is None:
        out = torch.empty(desc.kv_shape, dtype=torch.bfloat16, device=blob.device)
    ws = alloc_workspace(desc, CG_OP_FROM_BYTES, blob.device)
    cg_from_bytes(desc, blob, blob.numel(), out, ws, stream)
    check_status(ws, stream, "cg_from_bytes")
    return out
