"""Independent parse of the blob layout with struct/numpy (test-only).

Layout: header ("CGMX", u16 version, u16 dtype, u32 L, T, H, D, chunk, NC, A,
table format, u64 size, u8 bins_k[L], u8 bins_v[L]); then 64-byte aligned
sections: scales bf16 [2,L,T], cdf u16 (format 0: [2,L,C,A]; format 1: for
each (kv, layer) in turn, C tables of that layer's bins entries), chunk
offsets u64 [NC+1], lengths u16 [NC,2L,C], payload.
"""

import struct

import numpy as np


def parse(blob):
    buf = np.frombuffer(blob, np.uint8) if isinstance(blob, (bytes, bytearray)) else blob
    head = bytes(buf[:48])
    magic, ver, dt, L, T, H, D, chunk, NC, A, fmt, size = struct.unpack_from("<4sHH8IQ", head, 0)
    assert magic == b"CGMX" and ver == 1 and dt == 1 and chunk == 256 and fmt in (0, 1)
    C = H * D
    bins = np.stack([buf[48 : 48 + L], buf[48 + L : 48 + 2 * L]]).astype(np.int64)
    widths = bins if fmt == 1 else np.full((2, L), A, np.int64)
    up = lambda x: (x + 63) // 64 * 64
    o_sc = up(48 + 2 * L)
    o_cdf = o_sc + up(4 * L * T)
    tab_bytes = 2 * C * int(widths.sum())
    o_off = o_cdf + up(tab_bytes)
    o_len = o_off + up(8 * (NC + 1))
    o_pay = o_len + up(2 * NC * 2 * L * C)

    def view(dtype, count, offset):
        return buf[offset : offset + count * np.dtype(dtype).itemsize].view(dtype)

    # tables[kv][l]: u16 [C, W] (entries 0..W-1 of each channel's table).
    tables, e = [[None] * L for _ in range(2)], o_cdf
    for k in range(2):
        for l in range(L):
            w = int(widths[k, l])
            tables[k][l] = view("<u2", C * w, e).reshape(C, w)
            e += 2 * C * w

    return dict(
        L=L, T=T, H=H, D=D, C=C, NC=NC, A=A, size=size,
        bins_k=buf[48 : 48 + L].copy(), bins_v=buf[48 + L : 48 + 2 * L].copy(),
        scales=view("<u2", 2 * L * T, o_sc).reshape(2, L, T),
        fmt=fmt, widths=widths, tables=tables,
        cdf=view("<u2", 2 * L * C * A, o_cdf).reshape(2, L, C, A) if fmt == 0 else None,
        chunk_off=view("<u8", NC + 1, o_off),
        lengths=view("<u2", NC * 2 * L * C, o_len).reshape(NC, 2 * L, C),
        payload=buf[o_pay:],
        gaps=[(48 + 2 * L, o_sc), (o_sc + 4 * L * T, o_cdf), (o_cdf + tab_bytes, o_off),
              (o_off + 8 * (NC + 1), o_len), (o_len + 4 * NC * L * C, o_pay)],
    )


def stream_offsets(p):
    """Payload offset of every stream, [NC, 2L, C] int64, from the chunk offsets and lengths."""
    lens = p["lengths"].astype(np.int64).reshape(p["NC"], -1)
    excl = np.cumsum(lens, axis=1) - lens
    return (excl + p["chunk_off"].astype(np.int64)[:-1, None]).reshape(p["lengths"].shape)
