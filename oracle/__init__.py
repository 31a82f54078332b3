"""CacheGen KV-cache codec -- CPU oracle (Python wrapper).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` import this.
The product library never links, loads or calls it, and this wrapper never
imports the product package.

The arithmetic lives in ``cachegen_oracle.c`` (plain scalar C, built with
``gcc -O2 -ffp-contract=off``); ``cachegen_oracle_mt.c`` only runs its
one-layer calls on several threads (``threads=`` below) and moves the results
into place. This module only builds, loads and marshals.
All arrays are numpy arrays in C order; bf16 tensors are ``uint16`` bit
patterns.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cachegen_oracle.c")
_SRC_MT = os.path.join(_HERE, "cachegen_oracle_mt.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libcachegen_oracle.so")
_lib = None

CHUNK_TOKENS = 256


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile the oracle shared library with gcc."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall", "-pthread",
               "-fPIC", "-shared", "-o", tmp, _SRC, _SRC_MT, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        sig = {
            "ocg_default_bins": (i32, [i32, p, p]),
            "ocg_quantize": (i32, [i32, i32, i32, p, p, p, p, p]),
            "ocg_histogram": (i32, [i32, i32, i32, i32, p, p]),
            "ocg_cdf": (i32, [i32, i32, i32, i32, p, p]),
            "ocg_cdf_w": (i32, [i32, i32, i32, i32, p, p, p]),
            "ocg_encode_w": (i64, [i32, i32, i32, i32, p, p, p, p, i64, p, p]),
            "ocg_decode_w": (i32, [i32, i32, i32, i32, p, p, i64, p, p, p, p]),
            "ocg_to_bytes_fmt": (i64, [i32, i32, i32, i32, p, p, i32, p, p, i64]),
            "ocg_encode_stream": (i64, [p, i32, p, i32, p, i64]),
            "ocg_decode_stream": (i32, [p, i64, i32, p, i32, p]),
            "ocg_encode": (i64, [i32, i32, i32, i32, p, p, p, i64, p, p]),
            "ocg_decode": (i32, [i32, i32, i32, i32, p, i64, p, p, p, p]),
            "ocg_dequantize": (i32, [i32, i32, i32, p, p, p, p, p]),
            "ocg_blob_bound": (i64, [i32, i32, i32, i32, p, p]),
            "ocg_to_bytes": (i64, [i32, i32, i32, i32, p, p, p, p, i64]),
            "ocg_blob_header": (i32, [p, i64, p, p, p, i32]),
            "ocg_from_bytes": (i32, [p, i64, p]),
            "ocg_quantize_mt": (i32, [i32, i32, i32, p, p, p, p, p, i32]),
            "ocg_to_bytes_mt": (i64, [i32, i32, i32, i32, p, p, i32, p, p, i64, i32]),
            "ocg_from_bytes_mt": (i32, [p, i64, p, i32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc < 0:
        raise OracleError(f"{what} failed with code {rc}")
    return rc


def _u8(a):
    return np.ascontiguousarray(a, dtype=np.uint8)


def default_bins(nlayers: int):
    bk = np.zeros(nlayers, np.uint8)
    bv = np.zeros(nlayers, np.uint8)
    _check(lib().ocg_default_bins(nlayers, _p(bk), _p(bv)), "default_bins")
    return bk, bv


def alphabet(bins_k, bins_v) -> int:
    return int(max(np.max(bins_k), np.max(bins_v)))


def quantize(kv: np.ndarray, bins_k, bins_v, threads: int = 1):
    """kv: uint16 [L,2,T,H,D] or [L,2,T,C] -> (sym uint8 [2,L,T,C], scale uint16 [2,L,T]).
    threads > 1: the same result, layers spread over that many threads."""
    L, two, T = kv.shape[:3]
    assert two == 2
    C = int(np.prod(kv.shape[3:]))
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    bk, bv = _u8(bins_k), _u8(bins_v)
    sym = np.empty((2, L, T, C), np.uint8)
    scale = np.empty((2, L, T), np.uint16)
    if threads > 1:
        _check(lib().ocg_quantize_mt(L, T, C, _p(bk), _p(bv), _p(kv), _p(sym), _p(scale), int(threads)),
               "quantize_mt")
    else:
        _check(lib().ocg_quantize(L, T, C, _p(bk), _p(bv), _p(kv), _p(sym), _p(scale)), "quantize")
    return sym, scale


def histogram(sym: np.ndarray, A: int):
    _, L, T, C = sym.shape
    sym = _u8(sym)
    cnt = np.empty((2, L, C, A), np.uint32)
    _check(lib().ocg_histogram(L, T, C, A, _p(sym), _p(cnt)), "histogram")
    return cnt


def table_widths(bins_k, bins_v, table_format: int = 0):
    """Width of the tables of each (kv, layer) -> uint8 [2, L]: the call's
    alphabet for format 0, the layer's bins for format 1."""
    bk, bv = _u8(bins_k), _u8(bins_v)
    if table_format == 0:
        A = alphabet(bk, bv)
        return np.full((2, len(bk)), A, np.uint8)
    if table_format == 1:
        return np.ascontiguousarray(np.stack([bk, bv]))
    raise ValueError("table_format must be 0 or 1")


def cdf_from_counts(cnt: np.ndarray, T: int, widths=None):
    """-> int32 [2,L,C,A+1]; widths (uint8 [2,L]) gives each table its own
    alphabet (entries past a table's end hold 2^16)."""
    _, L, C, A = cnt.shape
    cnt = np.ascontiguousarray(cnt, dtype=np.uint32)
    cdf = np.empty((2, L, C, A + 1), np.int32)
    if widths is None:
        _check(lib().ocg_cdf(L, T, C, A, _p(cnt), _p(cdf)), "cdf")
    else:
        w = _u8(widths).reshape(2 * L)
        _check(lib().ocg_cdf_w(L, T, C, A, _p(w), _p(cnt), _p(cdf)), "cdf_w")
    return cdf


def build_cdf(sym: np.ndarray, A: int, widths=None):
    return cdf_from_counts(histogram(sym, A), sym.shape[2], widths)


def encode_stream(symbols, cdf_row) -> bytes:
    s = _u8(symbols)
    tab = np.ascontiguousarray(cdf_row, dtype=np.int32)
    A = tab.shape[0] - 1
    out = np.empty(4 * max(1, len(s)) + 8, np.uint8)
    n = _check(lib().ocg_encode_stream(_p(s), len(s), _p(tab), A, _p(out), out.size), "encode_stream")
    return out[:n].tobytes()


def decode_stream(data: bytes, n: int, cdf_row) -> np.ndarray:
    buf = np.frombuffer(bytes(data) + b"\0", np.uint8).copy()
    tab = np.ascontiguousarray(cdf_row, dtype=np.int32)
    A = tab.shape[0] - 1
    out = np.empty(max(1, n), np.uint8)
    _check(lib().ocg_decode_stream(_p(buf), len(data), n, _p(tab), A, _p(out)), "decode_stream")
    return out[:n]


def nchunks(T: int) -> int:
    return (T + CHUNK_TOKENS - 1) // CHUNK_TOKENS


def encode(sym: np.ndarray, cdf: np.ndarray, widths=None):
    """-> (payload bytes as uint8 array, lengths uint16 [NC,2L,C], chunk_off uint64 [NC+1])."""
    _, L, T, C = sym.shape
    A = cdf.shape[-1] - 1
    NC = nchunks(T)
    sym = _u8(sym)
    cdf = np.ascontiguousarray(cdf, dtype=np.int32)
    cap = NC * 2 * L * C * 4 * CHUNK_TOKENS
    payload = np.empty(max(cap, 1), np.uint8)
    lengths = np.empty((NC, 2 * L, C), np.uint16)
    chunk_off = np.empty(NC + 1, np.uint64)
    if widths is None:
        n = _check(lib().ocg_encode(L, T, C, A, _p(sym), _p(cdf), _p(payload), cap, _p(lengths), _p(chunk_off)),
                   "encode")
    else:
        w = _u8(widths).reshape(2 * L)
        n = _check(lib().ocg_encode_w(L, T, C, A, _p(w), _p(sym), _p(cdf), _p(payload), cap, _p(lengths),
                                      _p(chunk_off)), "encode_w")
    return payload[:n].copy(), lengths, chunk_off


def decode(payload: np.ndarray, lengths: np.ndarray, chunk_off: np.ndarray, cdf: np.ndarray, T: int,
           widths=None):
    NC, twoL, C = lengths.shape
    L = twoL // 2
    A = cdf.shape[-1] - 1
    pay = np.ascontiguousarray(np.concatenate([_u8(payload), np.zeros(1, np.uint8)]))
    lengths = np.ascontiguousarray(lengths, dtype=np.uint16)
    chunk_off = np.ascontiguousarray(chunk_off, dtype=np.uint64)
    cdf = np.ascontiguousarray(cdf, dtype=np.int32)
    sym = np.empty((2, L, T, C), np.uint8)
    if widths is None:
        _check(lib().ocg_decode(L, T, C, A, _p(pay), len(payload), _p(lengths), _p(chunk_off), _p(cdf), _p(sym)),
               "decode")
    else:
        w = _u8(widths).reshape(2 * L)
        _check(lib().ocg_decode_w(L, T, C, A, _p(w), _p(pay), len(payload), _p(lengths), _p(chunk_off), _p(cdf),
                                  _p(sym)), "decode_w")
    return sym


def dequantize(sym: np.ndarray, scale: np.ndarray, bins_k, bins_v):
    """-> bf16 bits uint16 [L,2,T,C]."""
    _, L, T, C = sym.shape
    sym = _u8(sym)
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    bk, bv = _u8(bins_k), _u8(bins_v)
    out = np.empty((L, 2, T, C), np.uint16)
    _check(lib().ocg_dequantize(L, T, C, _p(bk), _p(bv), _p(sym), _p(scale), _p(out)), "dequantize")
    return out


def to_bytes(kv: np.ndarray, bins_k, bins_v, table_format: int = 0, threads: int = 1) -> bytes:
    """The whole encode; threads > 1 spreads the layers over that many threads
    (the same bytes)."""
    L, two, T, H, D = kv.shape
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    bk, bv = _u8(bins_k), _u8(bins_v)
    cap = _check(lib().ocg_blob_bound(L, T, H, D, _p(bk), _p(bv)), "blob_bound")
    blob = np.empty(cap, np.uint8)
    if threads > 1:
        n = _check(lib().ocg_to_bytes_mt(L, T, H, D, _p(bk), _p(bv), int(table_format), _p(kv), _p(blob), cap,
                                         int(threads)), "to_bytes_mt")
    else:
        n = _check(lib().ocg_to_bytes_fmt(L, T, H, D, _p(bk), _p(bv), int(table_format), _p(kv), _p(blob), cap),
                   "to_bytes")
    return blob[:n].tobytes()


def blob_header(blob: bytes):
    """-> (dims dict, bins_k, bins_v)."""
    buf = np.frombuffer(blob, np.uint8).copy()
    dims = np.zeros(8, np.int32)
    bk = np.zeros(1024, np.uint8)
    bv = np.zeros(1024, np.uint8)
    _check(lib().ocg_blob_header(_p(buf), len(blob), _p(dims), _p(bk), _p(bv), 1024), "blob_header")
    names = ["nlayers", "ntokens", "nheads", "head_size", "chunk_tokens", "nchunks", "alphabet", "table_format"]
    d = dict(zip(names, map(int, dims)))
    return d, bk[: d["nlayers"]].copy(), bv[: d["nlayers"]].copy()


def from_bytes(blob, threads: int = 1) -> np.ndarray:
    """The whole decode -> bf16 bits [L,2,T,H,D]; blob: bytes or a uint8
    array. threads > 1 spreads the layers over that many threads."""
    d, _, _ = blob_header(blob)
    buf = np.ascontiguousarray(np.frombuffer(blob, np.uint8) if isinstance(blob, (bytes, bytearray)) else blob,
                               dtype=np.uint8)
    out = np.empty((d["nlayers"], 2, d["ntokens"], d["nheads"], d["head_size"]), np.uint16)
    if threads > 1:
        _check(lib().ocg_from_bytes_mt(_p(buf), buf.size, _p(out), int(threads)), "from_bytes_mt")
    else:
        _check(lib().ocg_from_bytes(_p(buf), buf.size, _p(out)), "from_bytes")
    return out
