#!/usr/bin/env python3
"""Benchmark of the CacheGen KV-cache codec on one MI355X.

One step = the whole hot path on one batch of synthetic KV already resident
in HBM: cg_to_bytes (quantise, histogram + CDF, range-encode, blob) followed
by cg_from_bytes (length scan, range-decode + dequantise) of that blob.

Default workload: Llama-3.1-8B-shaped long context, 32 layers x 8 KV heads x
128 = 1024 channels x 32768 tokens of bf16 (4 GiB of raw K+V), default
per-layer bins, seeded AR(1) generator with 1% outlier channels x20.

Prints ONE JSON line. ``value`` is the round-trip throughput: raw KV bytes /
(encode time + decode time). Encode and decode GB/s, the compression ratio,
per-stage times, the HBM roofline of each direction (whole entry-point calls
timed live with HIP events on the stream the library launches on; the one
furthest from its roofline is ``roofline``), and the CPU oracle on the same
input (all host cores on the whole tensor, one thread on a slab of it) are
reported beside it; the oracle's blob and decode also check the GPU's
(``verified``: SHA-256 of the blobs, count of differing decoded values).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "encode & decode GB/s of raw bf16 KV on 1 MI355X (32L×1024ch) + compression ratio"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD public spec


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama31_8b_t32k")
    ap.add_argument("--stage-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chunked-batch", action="store_true",
                    help="skip the 256-token-chunk batch measurement (e.g. under a profiler)")
    ap.add_argument("--no-streaming", action="store_true",
                    help="skip the pipelined host-to-device load measurement")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the encode/decode timing of the other model-shaped workloads")
    ap.add_argument("--cpu-slab-layers", type=int, default=4,
                    help="layers of the benchmark input the one-thread oracle timing takes")
    ap.add_argument("--json-out", default=None)
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_events(fn, reps, torch):
    """Average milliseconds of fn() over reps, HIP events on the current stream."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def source_hash():
    """SHA-256 over the library's device sources (every kernel)."""
    import glob
    import hashlib

    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "kv_cache_compression_layer_amd", "csrc", "*"))):
        if path.endswith((".hip", ".hpp")):
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload, entry_point):
    """HBM bytes per call of an entry point (its kernels' calibrated
    rocprofv3 FETCH_SIZE + WRITE_SIZE), from the summaries committed under
    profiles/, if they were taken on this workload and on the device sources
    as they are now; otherwise None."""
    import glob

    sha = source_hash()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith(f"traffic {entry_point} "):
                    continue
                kv = dict(item.split("=", 1) for item in line.split()[2:])
                if kv.get("workload") == workload and kv.get("source_sha256") == sha:
                    return int(kv["bytes_per_call"]), os.path.relpath(path, ROOT)
    return None


def other_workloads(torch, cgb, dev, skip, oracle_too):
    """Whole-blob encode and decode times of the other model-shaped workloads
    (one call each, inputs resident on the device, HIP events on the current
    stream): OPT-125m at 64 tokens (latency), Mistral-7B at 256 and 768
    tokens, GLM-4-9B at 16K tokens (its decode from a blob encoded before the
    timed region). Medians over the repetitions. With oracle_too, the CPU
    oracle is timed on each same input, on one thread and on all threads."""
    from kv_cache_compression_layer_amd.synth import WORKLOADS, generate_workload

    out = {}
    for name, reps in (("opt125m_t64", 100), ("mistral7b_t256", 100), ("mistral7b_t768", 100),
                       ("glm4_9b_t16k", 10)):
        if name == skip:
            continue
        w = WORKLOADS[name]
        kv_np = generate_workload(w)
        kv = torch.from_numpy(kv_np.view(np.int16)).to(dev).view(torch.bfloat16)
        desc = cgb.Desc.for_kv(tuple(kv.shape))
        blob = torch.empty(cgb.cg_blob_bound(desc), dtype=torch.uint8, device=dev)
        size_dev = torch.zeros(1, dtype=torch.int64, device=dev)
        ws_e = cgb.alloc_workspace(desc, cgb.CG_OP_TO_BYTES, dev)
        ws_d = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES, dev)
        kv_out = torch.empty_like(kv)

        def enc():
            cgb.cg_to_bytes(desc, kv, blob, size_dev, ws_e)

        enc()
        cgb.check_status(ws_e, what=f"cg_to_bytes {name}")
        nbytes = int(size_dev.item())

        def dec():
            cgb.cg_from_bytes(desc, blob, nbytes, kv_out, ws_d)

        dec()
        cgb.check_status(ws_d, what=f"cg_from_bytes {name}")

        def med(fn):
            for _ in range(max(3, reps // 5)):
                fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            torch.cuda.synchronize()
            ev[0].record()
            for i in range(reps):
                fn()
                ev[i + 1].record()
            torch.cuda.synchronize()
            return float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))

        enc_ms, dec_ms = med(enc), med(dec)
        raw = kv.numel() * 2
        out[name] = {"shape": list(kv.shape), "raw_bytes": raw, "blob_bytes": nbytes,
                     "compression_ratio": raw / nbytes, "encode_ms": enc_ms, "decode_ms": dec_ms,
                     "encode_GBps": raw / (enc_ms * 1e-3) / 1e9, "decode_GBps": raw / (dec_ms * 1e-3) / 1e9,
                     "reps": reps}
        if oracle_too:
            # The oracle on the same input, one thread and all threads.
            bk_np, bv_np = np.asarray(desc.bins_k, np.uint8), np.asarray(desc.bins_v, np.uint8)
            for threads in sorted({1, oracle_threads()}):
                te, td, _, _ = time_oracle(kv_np, bk_np, bv_np, threads)
                out[name][f"oracle_{threads}t"] = {"encode_GBps": raw / te / 1e9, "decode_GBps": raw / td / 1e9,
                                                   "round_trip_GBps": raw / (te + td) / 1e9, "threads": threads}
        log(f"{name}: {json.dumps({k: v for k, v in out[name].items() if k != 'shape'})}")
        del kv, kv_np, blob, ws_e, ws_d, kv_out
        torch.cuda.empty_cache()
    return out


def cpu_info():
    """CPU model, SMT state and core counts of this host."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    smt = None
    try:
        with open("/sys/devices/system/cpu/smt/active") as f:
            smt = "on" if f.read().strip() == "1" else "off"
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"cpu": model, "smt": smt, "nproc": os.cpu_count(), "affinity": affinity}


def oracle_threads():
    """Host threads for the multi-threaded oracle: all the cores this process
    may use, at most 16 (one GPU's share of a shared host)."""
    info = cpu_info()
    return max(1, min(16, info["affinity"] or 1))


def time_oracle(kv_np, bk, bv, threads):
    """to_bytes then from_bytes of the oracle on kv_np; seconds and outputs."""
    import oracle

    t0 = time.perf_counter()
    blob = oracle.to_bytes(kv_np, bk, bv, threads=threads)
    t1 = time.perf_counter()
    dec = oracle.from_bytes(blob, threads=threads)
    t2 = time.perf_counter()
    return t1 - t0, t2 - t1, blob, dec


def cpu_baseline(w, kv_np, bk, bv, gpu_blob, gpu_out, slab_layers):
    """The oracle (scalar C) on this host, on the benchmark's own input: all
    layers on all threads (which also checks the GPU's blob and decode), and a
    slab of the first `slab_layers` layers of the same tensor on one thread."""
    import hashlib

    threads = oracle_threads()
    raw = kv_np.nbytes
    log(f"cpu baseline: oracle on the whole input, {threads} threads")
    te, td, blob, dec = time_oracle(kv_np, bk, bv, threads)
    sha_o = hashlib.sha256(blob).hexdigest()
    sha_g = hashlib.sha256(gpu_blob).hexdigest()
    ndiff = int(np.count_nonzero(dec.reshape(-1) != gpu_out.reshape(-1)))
    verified = {"blob_sha256_gpu": sha_g, "blob_sha256_oracle": sha_o, "blob_equal": sha_g == sha_o,
                "decoded_values_differing": ndiff, "decoded_values": int(dec.size)}
    log(f"verified: {json.dumps(verified)}")
    del blob, dec
    sub = np.ascontiguousarray(kv_np[:slab_layers])
    sraw = sub.nbytes
    log(f"cpu baseline: oracle on layers 0-{slab_layers - 1}, 1 thread")
    te1, td1, _, _ = time_oracle(sub, bk[:slab_layers], bv[:slab_layers], 1)
    info = cpu_info()
    return {
        "value": raw / (te + td) / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the whole benchmark input ({w.name}, seed {w.seed}, {raw / 2**30:.0f} GiB of bf16 KV): "
                  f"to_bytes then from_bytes, {threads} threads over the layers",
        "encode_GBps": raw / te / 1e9,
        "decode_GBps": raw / td / 1e9,
        "seconds": te + td,
        "single_thread": {
            "value": sraw / (te1 + td1) / 1e9,
            "unit": "GB/s",
            "cores": 1,
            "sample": f"layers 0-{slab_layers - 1} of the same tensor as one {slab_layers}-layer call "
                      f"({sraw / 2**20:.0f} MiB; their bins): to_bytes then from_bytes",
            "encode_GBps": sraw / te1 / 1e9,
            "decode_GBps": sraw / td1 / 1e9,
            "seconds": te1 + td1,
        },
        **info,
    }, verified


def main():
    args = parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this codec runs on one GPU; multi-GPU runs are not part of this "
                                   "build (see DESIGN.md for how the work would shard)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    from kv_cache_compression_layer_amd import cachegen as cgb
    from kv_cache_compression_layer_amd.synth import WORKLOADS, generate_workload

    w = WORKLOADS[args.workload]
    L, T, H, D = w.nlayers, w.ntokens, w.nheads, w.head_size
    C = H * D
    N = 2 * L * T * C
    raw = 2 * N
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log(f"generating {w.name} {w.shape}")
    t0 = time.perf_counter()
    kv_np = generate_workload(w)
    log(f"generated in {time.perf_counter() - t0:.1f}s")
    kv = torch.from_numpy(kv_np.view(np.int16)).to(dev).view(torch.bfloat16)

    desc = cgb.Desc.for_kv(tuple(kv.shape))
    A = desc.alphabet
    blob = torch.empty(cgb.cg_blob_bound(desc), dtype=torch.uint8, device=dev)
    size_dev = torch.zeros(1, dtype=torch.int64, device=dev)
    ws_enc = cgb.alloc_workspace(desc, cgb.CG_OP_TO_BYTES, dev)
    ws_dec = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES, dev)
    kv_out = torch.empty_like(kv)

    def encode():
        cgb.cg_to_bytes(desc, kv, blob, size_dev, ws_enc)

    encode()
    cgb.check_status(ws_enc, what="cg_to_bytes")
    blob_size = int(size_dev.item())

    def decode():
        cgb.cg_from_bytes(desc, blob, blob_size, kv_out, ws_dec)

    decode()
    cgb.check_status(ws_dec, what="cg_from_bytes")
    info, _, _ = cgb.peek(blob[:blob_size])
    payload_bytes = blob_size - info["off_payload"]

    log(f"warmup {args.warmup}, steps {args.steps}")
    for _ in range(args.warmup):
        encode()
        decode()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps)]
    t_wall = time.perf_counter()
    for i in range(args.steps):
        ev[3 * i].record()
        encode()
        ev[3 * i + 1].record()
        decode()
        ev[3 * i + 2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    enc_steps = [ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(args.steps)]
    dec_steps = [ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(args.steps)]
    enc_ms = sum(enc_steps) / args.steps
    dec_ms = sum(dec_steps) / args.steps
    cgb.check_status(ws_dec, what="cg_from_bytes")
    step_ms = enc_ms + dec_ms
    log(f"encode {enc_ms:.3f} ms, decode {dec_ms:.3f} ms, wall/step {1e3 * wall / args.steps:.3f} ms")

    # Stage entry points, each timed on its own (same inputs, same stream).
    sym = torch.empty(N, dtype=torch.uint8, device=dev)
    scale = torch.empty(2 * L * T, dtype=torch.int16, device=dev)
    cdf = torch.empty(2 * L * C * (A + 1), dtype=torch.int32, device=dev)
    payload = torch.empty(max(payload_bytes, 1) + 1024, dtype=torch.uint8, device=dev)
    lengths = torch.empty(desc.nstreams, dtype=torch.int16, device=dev)
    chunk_off = torch.empty(desc.nchunks + 1, dtype=torch.int64, device=dev)
    ws_q = cgb.alloc_workspace(desc, cgb.CG_OP_QUANTIZE, dev)
    ws_c = cgb.alloc_workspace(desc, cgb.CG_OP_BUILD_CDF, dev)
    ws_e = cgb.alloc_workspace(desc, cgb.CG_OP_ENCODE, dev)
    ws_d = cgb.alloc_workspace(desc, cgb.CG_OP_DECODE, dev)
    sym2 = torch.empty_like(sym)
    kv_out2 = torch.empty_like(kv)
    stage_fns = {
        "quantize": lambda: cgb.cg_quantize(desc, kv, sym, scale, ws_q),
        "build_cdf": lambda: cgb.cg_build_cdf(desc, sym, cdf, ws_c),
        "encode": lambda: cgb.cg_encode(desc, sym, cdf, payload, lengths, chunk_off, ws_e),
        "decode": lambda: cgb.cg_decode(desc, payload, payload_bytes, lengths, chunk_off, cdf, sym2, ws_d),
        "dequantize": lambda: cgb.cg_dequantize(desc, sym2, scale, kv_out2),
    }
    stages_ms = {}
    for name, fn in stage_fns.items():
        fn()
        stages_ms[name] = time_events(fn, args.stage_reps, torch)
    for ws in (ws_q, ws_c, ws_e, ws_d):
        cgb.check_status(ws, what="stage calls")
    stages_ms["from_bytes"] = dec_ms
    stages_ms["to_bytes"] = enc_ms

    # Decode into a paged cache (16-token blocks, a shuffled block table with
    # 1% spare blocks), the layout a serving engine keeps.
    bs = 16
    nblk = (T + bs - 1) // bs
    num_blocks = nblk + nblk // 100 + 1
    gen = torch.Generator(device="cpu").manual_seed(1234)
    table = torch.randperm(num_blocks, generator=gen)[:nblk].to(torch.int32).to(dev)
    cache = torch.empty(L * 2 * num_blocks * bs * C, dtype=torch.int16, device=dev)
    ws_p = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES, dev)

    def paged():
        cgb.cg_from_bytes_paged(desc, blob, blob_size, cache, 2 * num_blocks * bs * C, num_blocks * bs * C,
                                bs, table, num_blocks, ws_p)

    paged()
    cgb.check_status(ws_p, what="cg_from_bytes_paged")
    stages_ms["from_bytes_paged"] = time_events(paged, args.stage_reps, torch)
    del cache
    log(f"stages (ms): {json.dumps({k: round(v, 4) for k, v in stages_ms.items()})}")

    # Loading the blob from host memory while it arrives: the host-to-device
    # copy of the payload piece by piece on one stream, the decode of each
    # piece's chunks on another as soon as it is there; against copying the
    # whole blob first. The link-time model prices 100/500/1000 Mbps links
    # with the measured decode times.
    streaming = None
    if not args.no_streaming:
        from kv_cache_compression_layer_amd import streaming as stm

        host_blob = torch.empty(blob_size, dtype=torch.uint8, pin_memory=True)
        host_blob.copy_(blob[:blob_size].cpu())
        dev_blob = torch.empty(blob_size, dtype=torch.uint8, device=dev)
        kv_s = torch.empty_like(kv)
        ws_s = cgb.alloc_workspace(desc, cgb.CG_OP_FROM_BYTES, dev)
        off_c = info["off_chunk_off"]
        chunk_off_h = blob[off_c:off_c + 8 * (desc.nchunks + 1)].cpu().numpy().view(np.uint64)
        cpp = max(1, desc.nchunks // 8)
        pieces = stm.plan_pieces(info["off_payload"], chunk_off_h, cpp)
        copy_s, dec_s = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)

        def wall_ms(fn, reps):
            best = []
            for _ in range(reps):
                torch.cuda.synchronize()
                t = time.perf_counter()
                fn()
                torch.cuda.synchronize()
                best.append(1e3 * (time.perf_counter() - t))
            return float(np.median(best))

        def serial():
            with torch.cuda.stream(copy_s):
                dev_blob.copy_(host_blob, non_blocking=True)
            cgb.cg_from_bytes(desc, dev_blob, blob_size, kv_s, ws_s, copy_s)

        def pipelined():
            stm.enqueue_pipelined_load(desc, host_blob, dev_blob, kv_s, ws_s, pieces, copy_s, dec_s)

        def copy_only():
            with torch.cuda.stream(copy_s):
                dev_blob.copy_(host_blob, non_blocking=True)

        pipelined()
        torch.cuda.synchronize()
        cgb.check_status(ws_s, what="pipelined cg_from_bytes_chunks")
        assert torch.equal(kv_s, kv_out), "pipelined load differs from the whole decode"
        copy_ms = wall_ms(copy_only, 5)
        serial_ms = wall_ms(serial, 5)
        pipe_ms = wall_ms(pipelined, 5)
        last = pieces[-1]
        last_ms = time_events(lambda: cgb.cg_from_bytes_chunks(desc, blob, blob_size, last.chunk_begin,
                                                               last.chunk_end, kv_s, ws_s), args.stage_reps, torch)
        streaming = {
            "pieces": len(pieces),
            "chunks_per_piece": cpp,
            "h2d_copy_ms": copy_ms,
            "h2d_GBps": blob_size / (copy_ms * 1e-3) / 1e9,
            "serial_copy_then_decode_ms": serial_ms,
            "pipelined_ms": pipe_ms,
            "last_piece_decode_ms": last_ms,
            "link_model": stm.link_model(raw, blob_size, dec_ms, last_ms),
        }
        log(f"streaming: copy {copy_ms:.3f} ms, serial {serial_ms:.3f} ms, pipelined {pipe_ms:.3f} ms, "
            f"last piece {last_ms:.3f} ms")
        del host_blob, dev_blob, kv_s

    # The same KV as LMCache stores it: one to_bytes call per 256-token chunk,
    # each with its own tables. All chunks as one batch call, against the
    # same calls made one by one on the same stream.
    ct = 256
    nb = T // ct
    batch = None

    # Batch calls (a few ms each) are averaged over at least 20 calls, after
    # two untimed ones.
    def time_batch(fn):
        fn()
        fn()
        return time_events(fn, max(args.stage_reps, 20), torch)

    if nb >= 2 and not args.no_chunked_batch:
        desc1 = cgb.Desc(L, ct, H, D, desc.bins_k, desc.bins_v)
        chunks = kv.view(L, 2, nb, ct, C).permute(2, 0, 1, 3, 4).contiguous()
        stride = (cgb.cg_blob_bound(desc1) + 15) // 16 * 16  # 16-byte multiple: tables written in place
        blobs = torch.empty(nb * stride, dtype=torch.uint8, device=dev)
        sizes = torch.zeros(nb, dtype=torch.int64, device=dev)
        ws_be = cgb.alloc_workspace_batch(desc1, nb, stride, cgb.CG_OP_TO_BYTES, dev)
        ws_bd = cgb.alloc_workspace_batch(desc1, nb, stride, cgb.CG_OP_FROM_BYTES, dev)
        chunks_out = torch.empty_like(chunks)

        def b_enc():
            cgb.cg_to_bytes_batch(desc1, nb, chunks, blobs, stride, sizes, ws_be)

        def b_dec():
            cgb.cg_from_bytes_batch(desc1, nb, blobs, stride, sizes, chunks_out, ws_bd)

        b_enc()
        cgb.check_status(ws_be, what="cg_to_bytes_batch")
        b_dec()
        cgb.check_status(ws_bd, what="cg_from_bytes_batch")
        b_enc_ms = time_batch(b_enc)
        b_dec_ms = time_batch(b_dec)
        sizes_h = [int(x) for x in sizes.cpu()]
        # One call per chunk (views prepared outside the timed region).
        ws1e = cgb.alloc_workspace(desc1, cgb.CG_OP_TO_BYTES, dev)
        ws1d = cgb.alloc_workspace(desc1, cgb.CG_OP_FROM_BYTES, dev)
        blobs2 = torch.empty_like(blobs)
        sizes2 = torch.zeros(nb, dtype=torch.int64, device=dev)
        views = [(chunks[b], blobs2[b * stride:(b + 1) * stride], sizes2[b:b + 1], chunks_out[b])
                 for b in range(nb)]

        def l_enc():
            for c_in, bl, sz, _ in views:
                cgb.cg_to_bytes(desc1, c_in, bl, sz, ws1e)

        def l_dec():
            for (_, bl, _, c_out), n in zip(views, sizes_h):
                cgb.cg_from_bytes(desc1, bl, n, c_out, ws1d)

        l_enc()
        cgb.check_status(ws1e, what="cg_to_bytes")
        assert torch.equal(sizes2, sizes), "batch and per-call blob sizes differ"
        l_dec()
        cgb.check_status(ws1d, what="cg_from_bytes")
        l_enc_ms = time_events(l_enc, 2, torch)
        l_dec_ms = time_events(l_dec, 2, torch)
        craw = chunks.numel() * 2
        batch = {
            "calls": nb,
            "tokens_per_call": ct,
            "to_bytes_ms": b_enc_ms,
            "from_bytes_ms": b_dec_ms,
            "to_bytes_GBps": craw / (b_enc_ms * 1e-3) / 1e9,
            "from_bytes_GBps": craw / (b_dec_ms * 1e-3) / 1e9,
            "per_call_to_bytes_ms": l_enc_ms,
            "per_call_from_bytes_ms": l_dec_ms,
            "per_call_to_bytes_GBps": craw / (l_enc_ms * 1e-3) / 1e9,
            "per_call_from_bytes_GBps": craw / (l_dec_ms * 1e-3) / 1e9,
            "compression_ratio": craw / sum(sizes_h),
        }
        del blobs2, ws1e, ws1d, views
        # The same batch with per-layer tables (every (K|V, layer) table has
        # its layer's bins): the tables are most of a 256-token blob.
        desc1p = cgb.Desc(L, ct, H, D, desc.bins_k, desc.bins_v, cgb.CG_TABLES_PER_LAYER)
        stride_p = (cgb.cg_blob_bound(desc1p) + 15) // 16 * 16
        ws_pe = cgb.alloc_workspace_batch(desc1p, nb, stride_p, cgb.CG_OP_TO_BYTES, dev)
        ws_pd = cgb.alloc_workspace_batch(desc1p, nb, stride_p, cgb.CG_OP_FROM_BYTES, dev)
        sizes_p = torch.zeros(nb, dtype=torch.int64, device=dev)
        out_p = torch.empty_like(chunks)

        def p_enc():
            cgb.cg_to_bytes_batch(desc1p, nb, chunks, blobs, stride_p, sizes_p, ws_pe)

        def p_dec():
            cgb.cg_from_bytes_batch(desc1p, nb, blobs, stride_p, sizes_p, out_p, ws_pd)

        p_enc()
        cgb.check_status(ws_pe, what="cg_to_bytes_batch (per-layer tables)")
        p_dec()
        cgb.check_status(ws_pd, what="cg_from_bytes_batch (per-layer tables)")
        assert torch.equal(out_p, chunks_out), "per-layer tables decode differently"
        batch["per_layer_tables"] = {
            "to_bytes_ms": time_batch(p_enc),
            "from_bytes_ms": time_batch(p_dec),
            "compression_ratio": craw / int(sizes_p.sum().item()),
        }
        log(f"batch of {nb} x {ct} tokens: {json.dumps(batch)}")
        del chunks, chunks_out, out_p, blobs, ws_be, ws_bd, ws_pe, ws_pd
        torch.cuda.empty_cache()
        # The pages' chunk-size sweep: the same KV cut into calls of 64, 128
        # and 768 tokens (768 takes the first 42 * 768 tokens), one batch call
        # each way.
        sweep = []
        for ct2 in (64, 128, 768):
            nb2 = T // ct2
            if nb2 < 2 or nb2 * L > 32767:
                continue
            d2 = cgb.Desc(L, ct2, H, D, desc.bins_k, desc.bins_v)
            ch2 = kv.view(L, 2, T, C)[:, :, : nb2 * ct2].reshape(L, 2, nb2, ct2, C).permute(2, 0, 1, 3, 4).contiguous()
            st2 = (cgb.cg_blob_bound(d2) + 15) // 16 * 16
            bl2 = torch.empty(nb2 * st2, dtype=torch.uint8, device=dev)
            sz2 = torch.zeros(nb2, dtype=torch.int64, device=dev)
            we2 = cgb.alloc_workspace_batch(d2, nb2, st2, cgb.CG_OP_TO_BYTES, dev)
            wd2 = cgb.alloc_workspace_batch(d2, nb2, st2, cgb.CG_OP_FROM_BYTES, dev)
            out2 = torch.empty_like(ch2)

            def e2():
                cgb.cg_to_bytes_batch(d2, nb2, ch2, bl2, st2, sz2, we2)

            def d2f():
                cgb.cg_from_bytes_batch(d2, nb2, bl2, st2, sz2, out2, wd2)

            e2()
            cgb.check_status(we2, what=f"cg_to_bytes_batch ({ct2}-token calls)")
            d2f()
            cgb.check_status(wd2, what=f"cg_from_bytes_batch ({ct2}-token calls)")
            r2 = ch2.numel() * 2
            te2 = time_batch(e2)
            td2 = time_batch(d2f)
            row = {"tokens_per_call": ct2, "calls": nb2, "to_bytes_ms": te2, "from_bytes_ms": td2,
                   "to_bytes_GBps": r2 / (te2 * 1e-3) / 1e9, "from_bytes_GBps": r2 / (td2 * 1e-3) / 1e9,
                   "compression_ratio": r2 / int(sz2.sum().item())}
            log(f"batch of {nb2} x {ct2} tokens: {json.dumps(row)}")
            sweep.append(row)
            del ch2, bl2, sz2, we2, wd2, out2
            torch.cuda.empty_cache()
        batch["chunk_size_sweep"] = sweep

    # Achievable copy bandwidth: a device-to-device copy of the raw KV
    # (read + write of 4 GiB), the practical ceiling beside the 8 TB/s spec.
    kv_copy = torch.empty_like(kv)
    copy_ms = time_events(lambda: kv_copy.copy_(kv), 5, torch)
    copy_GBps = 2 * raw / (copy_ms * 1e-3) / 1e9
    del kv_copy
    log(f"copy {copy_ms:.3f} ms = {copy_GBps:.0f} GB/s")

    # Roofline of each direction: the algorithmic bytes of the metric (read the
    # bf16 KV and write the blob, or read the blob and write the bf16 KV) over
    # the whole entry point's time. Each call is a short sequence of kernels
    # launched back to back on one stream; HIP events on that stream bracket
    # the call, averaged over the timed steps. The kernel split of one call is
    # in the rocprofv3 kernel trace under profiles/.
    def direction(entry, kernels, ms):
        alg = raw + blob_size
        ach = alg / (ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
             "traffic": None, "kernel": f"{entry}: {kernels}", "entry_point": entry,
             "algorithmic_bytes": alg, "avg_ms": ms,
             "timing": "whole entry-point call; HIP events on the stream the library launches on, "
                       "average over the timed steps",
             "frac_of_copy": ach / copy_GBps}
        rec = recorded_traffic(w.name, entry)
        if rec is not None:
            r["traffic"], r["traffic_source"] = rec
            r["traffic_ratio"] = rec[0] / alg
        return r

    directions = {
        "encode": direction("cg_to_bytes", "quantise + histogram (+ tables), range encode, offset scans, "
                                           "compaction", enc_ms),
        "decode": direction("cg_from_bytes", "length scan, range decode + dequantise", dec_ms),
    }
    # The contract's single entry: the direction furthest from its roofline.
    roofline = dict(min(directions.values(), key=lambda r: r["frac"]))

    enc_GBps = raw / (enc_ms * 1e-3) / 1e9
    dec_GBps = raw / (dec_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": raw / (step_ms * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "io_dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: bf16 KV [L,2,T,H,D]=[{L},2,{T},{H},{D}], default per-layer bins "
                        f"(K 32/16, V 32/16), AR(1) rho={w.rho} {w.innovations}, "
                        f"{w.outlier_frac:.0%} outlier channels x{w.outlier_scale:g}, seed {w.seed}",
            "raw_bytes": raw,
            "chunk_tokens": 256,
            "alphabet": A,
        },
        "encode_GBps": enc_GBps,
        "decode_GBps": dec_GBps,
        "encode_ms": enc_ms,
        "decode_ms": dec_ms,
        "encode_ms_median": float(np.median(enc_steps)),
        "encode_ms_min": min(enc_steps),
        "decode_ms_median": float(np.median(dec_steps)),
        "decode_ms_min": min(dec_steps),
        "copy_GBps": copy_GBps,
        "paged_decode_GBps": raw / (stages_ms["from_bytes_paged"] * 1e-3) / 1e9,
        "compression_ratio": raw / blob_size,
        "payload_ratio": raw / payload_bytes,
        "blob_bytes": blob_size,
        "encode_hbm_frac": (raw + blob_size) / (enc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "decode_hbm_frac": (raw + blob_size) / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "encode_copy_frac": (raw + blob_size) / (enc_ms * 1e-3) / 1e9 / copy_GBps,
        "decode_copy_frac": (raw + blob_size) / (dec_ms * 1e-3) / 1e9 / copy_GBps,
        "stages_ms": stages_ms,
        "chunked_batch": batch,
        "streaming": streaming,
        "roofline": roofline,
        "roofline_by_direction": directions,
        "cpu_baseline": None,
    }

    del sym, sym2, kv_out2, payload
    if not args.no_other_workloads:
        result["other_workloads"] = other_workloads(torch, cgb, dev, w.name, not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        gpu_blob = blob[:blob_size].cpu().numpy()
        gpu_out = kv_out.view(torch.int16).cpu().numpy().view(np.uint16)
        bk_np = np.asarray(desc.bins_k, np.uint8)
        bv_np = np.asarray(desc.bins_v, np.uint8)
        result["cpu_baseline"], result["verified"] = cpu_baseline(w, kv_np, bk_np, bv_np, gpu_blob, gpu_out,
                                                                 args.cpu_slab_layers)
        del gpu_blob, gpu_out
    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
