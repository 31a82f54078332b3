"""Loading a CacheGen blob while it arrives: decode chunk j while chunk j + 1
is still in transfer.

LMCache stores KV compressed so that loading it over a link is fast; the
CacheGen reproduction thread measures network transfer time against decode
time over simulated 100 / 500 / 1000 Mbps links. The codec makes every
256-token chunk decodable on its own once the sections in front of the
payload (scales, tables, chunk offsets, lengths) are there (LMCache CacheGen
page, sections 4 and 5), so a receiver can decode chunk by chunk as the
payload comes in. Here the link is the host-to-device copy: the blob sits in
pinned host memory, a copy stream moves the front sections and then the
payload piece by piece, and the decode stream waits for each piece and runs
cg_from_bytes_chunks on its chunk range. Nothing here computes a codec step;
the device work is the library's.
"""

from __future__ import annotations

from dataclasses import dataclass

from . import cachegen as cgb


@dataclass
class Piece:
    chunk_begin: int
    chunk_end: int
    byte_end: int  # blob bytes that must have arrived (front sections + payload up to chunk_end)


def plan_pieces(off_payload: int, chunk_off, chunks_per_piece: int):
    """Split the chunks into pieces of `chunks_per_piece` (the last may be
    shorter). chunk_off: the blob's chunk offsets (host, NC + 1 entries)."""
    nc = len(chunk_off) - 1
    if chunks_per_piece < 1:
        raise ValueError("chunks_per_piece must be >= 1")
    out = []
    for j0 in range(0, nc, chunks_per_piece):
        j1 = min(nc, j0 + chunks_per_piece)
        out.append(Piece(j0, j1, off_payload + int(chunk_off[j1])))
    return out


def enqueue_pipelined_load(desc, blob_host, blob_dev, kv_out, ws, pieces, copy_stream, decode_stream):
    """Enqueue the copies (on copy_stream) and the chunk-range decodes (on
    decode_stream, each after its piece has arrived). blob_host: pinned uint8
    host tensor holding the whole blob; blob_dev: uint8 device tensor at
    least as large. Returns the per-piece arrival events."""
    torch = cgb._torch()
    arrived = []
    start = 0
    for p in pieces:
        with torch.cuda.stream(copy_stream):
            blob_dev[start:p.byte_end].copy_(blob_host[start:p.byte_end], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(copy_stream)
        arrived.append(ev)
        start = p.byte_end
    for p, ev in zip(pieces, arrived):
        decode_stream.wait_event(ev)
        cgb.cg_from_bytes_chunks(desc, blob_dev, p.byte_end, p.chunk_begin, p.chunk_end, kv_out, ws,
                                 decode_stream)
    return arrived


def link_model(raw_bytes: int, blob_bytes: int, decode_ms: float, last_piece_decode_ms: float,
               mbps=(100, 500, 1000)):
    """Load time of the KV over a link of each bandwidth: the raw bf16 bytes
    sent as they are, against the blob sent and decoded after it arrives
    (serial) or while it arrives (pipelined: only the decode of the last
    piece remains once the link is done, as the decode runs far faster than
    the link delivers)."""
    rows = []
    for m in mbps:
        bps = m * 1e6 / 8
        raw_s = raw_bytes / bps
        blob_s = blob_bytes / bps
        rows.append({
            "link_mbps": m,
            "raw_transfer_s": raw_s,
            "blob_transfer_s": blob_s,
            "serial_load_s": blob_s + decode_ms * 1e-3,
            "pipelined_load_s": blob_s + last_piece_decode_ms * 1e-3,
            "speedup_vs_raw": raw_s / (blob_s + last_piece_decode_ms * 1e-3),
        })
    return rows
