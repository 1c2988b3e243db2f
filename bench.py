#!/usr/bin/env python3
"""Benchmark of the PGKQ hot path on one MI355X.

Workload: the GQA decode cache of 16 sequences x 8 kv-heads (32 query heads)
x 32 768 tokens, head_dim 128, fp16 keys/values, bf16 queries, b_main 3 /
b_angle 2 with a 128-bit QJL sketch; its 4 194 304 keys are also the bulk
encode workload (with the channel reorder step).  Synthetic, seeded inputs
(synth/), resident in HBM before the timed region.

One step = the whole path: calibrate (channel sums, reorder, radius table) ->
encode every key -> decode attention for every (sequence, query head) over the
32k-token compressed cache (8 token splits).  A 512 MiB buffer is rewritten
between encode and decode so that the decode does not read the freshly written
codes out of the 256 MB Infinity Cache.  HIP events time each phase; the
library records events around the decode scan kernel itself (the roofline
figure).  The JSON line reports decode cache tokens/s as ``value``.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "decode_scan_gqa32k_b16_traffic.json")
SCAN_SOURCES = ["compressed_cache_decode_pgkq_amd/csrc/scan.hpp",
                "compressed_cache_decode_pgkq_amd/csrc/pgkq_internal.hpp",
                "compressed_cache_decode_pgkq_amd/csrc/host_iface.hpp",
                "compressed_cache_decode_pgkq_amd/csrc/coded_pv.hpp",
                "compressed_cache_decode_pgkq_amd/csrc/mfma_pv.hpp",
                "compressed_cache_decode_pgkq_amd/csrc/device_common.hpp"]


ENCODE_SOURCES = ["compressed_cache_decode_pgkq_amd/csrc/encode.hip",
                  "compressed_cache_decode_pgkq_amd/csrc/pgkq_internal.hpp",
                  "compressed_cache_decode_pgkq_amd/csrc/host_iface.hpp",
                  "compressed_cache_decode_pgkq_amd/csrc/device_common.hpp"]
PROFILE_UTIL = os.path.join(ROOT, "profiles", "utilization_gqa32k_b16.json")
ENCODE_KERNEL = "void encode_kernel<128, 3, true, 2, true>"
# vector ALU issue rate: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz (a
# wave64 instruction occupies its SIMD for 4 clocks); an fp64 FMA is one
# lane-operation, so this is also the published fp64 vector peak / 2
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9


def _source_hash(files) -> str:
    """Hash of the code of `files` (comments and blank space removed, so that a
    profile stays attached to kernels whose code has not changed)."""
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def scan_source_hash() -> str:
    return _source_hash(SCAN_SOURCES)


def encode_source_hash() -> str:
    return _source_hash(ENCODE_SOURCES)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def generate(cfg):
    from synth import make_inputs
    t = time.perf_counter()
    inp = make_inputs(cfg)
    log(f"[bench] generated {cfg.name} inputs in {time.perf_counter() - t:.1f} s")
    return inp


def host_cores() -> int:
    """Host cores the oracle may use: this process's CPU affinity, capped at 16
    (the host share of one GPU on a multi-GPU node)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def _oracle_encode_stream(cfg, inp, b, h, c, t, p):
    from oracle import calibrate, codebook, encode
    K = inp["K"][b, h]
    ss = calibrate.channel_sumsq(K)
    lv, th = codebook.scaled_table(c, t, calibrate.head_scale(ss, len(K)), cfg.head_dim)
    f = encode.encode_keys(K, inp["signs"][h], None, lv, th, inp["S"][h], p)
    # keep only the stored fields (the diagnostics of Fields are large)
    return {"rc": f.rc.astype(np.uint8), "ac": f.ac.astype(np.uint8), "bits": f.bits, "nu": f.nu}, lv


def _oracle_decode_stream(cfg, inp, b, h, fields, lv, p):
    from oracle import attn
    G = cfg.n_q // cfg.n_kv
    for g in range(G):
        s = attn.analytic_logits(inp["q"][b, h * G + g], fields, lv, inp["S"][h], inp["signs"][h],
                                 None, p)
        attn.attend(s, inp["V"][b, h], 1.0 / math.sqrt(cfg.head_dim))


def cpu_baseline(cfg, inp, one_core_streams: int = 4):
    """Time the float64 oracle, as it stands, on the host cores.

    All-core leg: the whole workload (every (sequence, kv-head) stream: encode
    of its keys, then decode of its G query heads over the oracle's codes),
    streams spread over `host_cores()` worker threads with one BLAS thread
    each (NumPy and BLAS release the GIL, so the threads run in parallel).
    One-core leg: the first `one_core_streams` streams on one thread."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    from oracle import codebook, encode

    p = encode.Params(cfg.head_dim, cfg.b_main, cfg.b_angle, cfg.qjl_m)
    G = cfg.n_q // cfg.n_kv
    c, t = codebook.lloyd_max_beta(cfg.head_dim, cfg.b_main)
    streams = [divmod(i, cfg.n_kv) for i in range(cfg.n_seq * cfg.n_kv)]
    cores = host_cores()

    def run(sel, workers):
        with threadpool_limits(limits=1):
            with cf.ThreadPoolExecutor(max_workers=workers) as ex:
                t0 = time.perf_counter()
                enc = list(ex.map(lambda bh: _oracle_encode_stream(cfg, inp, bh[0], bh[1], c, t, p), sel))
                t1 = time.perf_counter()
                list(ex.map(lambda a: _oracle_decode_stream(cfg, inp, a[0][0], a[0][1], a[1][0], a[1][1], p),
                            zip(sel, enc)))
                t2 = time.perf_counter()
        return t1 - t0, t2 - t1

    e1, d1 = run(streams[:one_core_streams], 1)
    log(f"[bench] oracle on 1 core: {one_core_streams} streams, encode {e1:.1f} s, decode {d1:.1f} s")
    eN, dN = run(streams, cores)
    log(f"[bench] oracle on {cores} cores: {len(streams)} streams, encode {eN:.1f} s, decode {dN:.1f} s")
    T = cfg.n_tokens
    # token-heads/s -> cache tokens/s (a cache token spans all n_kv kv-heads)
    dec = {"value": len(streams) * T / dN / cfg.n_kv, "unit": "cache tokens/s", "cores": cores,
           "kind": "oracle",
           "sample": f"the whole workload: {len(streams)} streams x {T} tokens x {G} query heads "
                     f"(decode of oracle-encoded codes, float64), {cores} worker threads with one "
                     f"BLAS thread each, {dN:.1f} s wall",
           "one_core": {"value": one_core_streams * T / d1 / cfg.n_kv, "unit": "cache tokens/s",
                        "sample": f"{one_core_streams} streams, {d1:.1f} s"}}
    enc = {"value": len(streams) * T / eN, "unit": "keys/s", "cores": cores, "kind": "oracle",
           "sample": f"all {len(streams) * T} keys, {cores} worker threads, {eN:.1f} s wall",
           "one_core": {"value": one_core_streams * T / e1, "unit": "keys/s",
                        "sample": f"{one_core_streams * T} keys, {e1:.1f} s"}}
    return {"decode": dec, "encode": enc}


def measure_copy(torch, dev, reps: int = 10) -> float:
    """Device-to-device copy bandwidth on this GPU (bytes read + written per
    second, GB/s), 1 GiB each way, beside the 8 TB/s spec figure."""
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.copy_(a)
    ts = []
    for _ in range(reps):
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del a, b
    return 2 * n / (float(np.median(ts)) * 1e-3) / 1e9


def measure_read(api, torch, dev, nbytes: int, flush, reps: int = 20) -> dict:
    """Read ceiling: the library's read probe (16-byte non-temporal buffer loads,
    the decode scans' load path, nothing else) over `nbytes` bytes, the
    Infinity Cache evicted before each read; median GB/s of the kernel alone."""
    nbytes = nbytes // 16 * 16
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    acc = torch.zeros(1, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for r in range(reps + 3):
        flush.fill_(r & 255)
        e0.record()
        api.pgkq_stream_read(buf, acc)
        e1.record()
        torch.cuda.synchronize()
        if r >= 3:
            ts.append(e0.elapsed_time(e1))
    del buf
    ms = float(np.median(ts))
    return {"bytes": nbytes, "ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "p10_ms": float(np.percentile(ts, 10)), "p90_ms": float(np.percentile(ts, 90))}


def run_controls(api, torch, dev, cfg, K, V, Vt, q, signs, S, flush, E, reps: int = 20):
    """The same decode workload on the RTN INT4 / INT3 key caches, with PGKQ-coded
    values as well (PGKQ-KV k3v3), and on the uncompressed fp16 cache (same
    keys, values, queries and split count): scan kernel time and its share of
    the HBM peak."""
    n_seq, n_kv, T, d = K.shape
    res = {}
    e0, e1 = E(), E()
    e0.record()
    e1.record()

    def timed(call):
        ts = []
        for r in range(reps + 3):
            flush.fill_(r & 255)
            call()
            torch.cuda.synchronize()
            if r >= 3:
                ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    out = torch.empty((n_seq, cfg.n_q, d), dtype=torch.float32, device=dev)
    for bits in (4, 3):
        rb = api.pgkq_rtn_record_bytes(d, bits)
        codes = api.pgkq_rtn_encode(K, bits)
        ws = torch.empty(api.pgkq_rtn_decode_workspace_bytes(d, n_seq, cfg.n_q, n_kv, T, cfg.n_splits),
                         dtype=torch.uint8, device=dev)
        ms = timed(lambda: api.pgkq_rtn_decode_attn(q, codes, Vt, bits, n_splits=cfg.n_splits, out=out,
                                                    workspace=ws, events=(e0, e1)))
        alg = n_seq * n_kv * T * (rb + 2 * d)
        res[f"rtn_int{bits}"] = {"record_bytes": rb, "scan_ms": ms,
                                 "cache_tokens_per_s_scan": n_seq * T / (ms * 1e-3),
                                 "scan_gbs": alg / (ms * 1e-3) / 1e9,
                                 "frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del codes, ws
    # PGKQ-KV k3v3: values coded too (key table and projection as in the main path)
    from synth.inputs import value_projection
    pk = api.PgkqParams(d, cfg.b_main, cfg.b_angle, cfg.qjl_m, 1)
    pv = api.PgkqParams(d, cfg.b_main, cfg.b_angle, cfg.qjl_m, 0)
    Sv = torch.from_numpy(value_projection(cfg)).to(dev)
    _, _, cbk = api.pgkq_calibrate(pk, K)
    _, _, cbv = api.pgkq_calibrate(pv, V)
    ck = api.pgkq_encode(pk, K, signs, None, cbk, S, capacity=T)
    cv = api.pgkq_encode(pv, V, signs, None, cbv, Sv, capacity=T)
    ws = torch.empty(api.pgkq_kv_decode_workspace_bytes(pk, pv, n_seq, cfg.n_q, n_kv, T, cfg.n_splits),
                     dtype=torch.uint8, device=dev)
    ms = timed(lambda: api.pgkq_kv_decode_attn(pk, pv, q, ck, cv, n_kv, T, signs, None, cbk, S, cbv,
                                               Sv, n_splits=cfg.n_splits, out=out, workspace=ws,
                                               events=(e0, e1)))
    rbk, rbv = api.pgkq_record_bytes(pk), api.pgkq_record_bytes(pv)
    alg = n_seq * n_kv * T * (rbk + rbv)
    res["pgkq_kv_k3v3"] = {"record_bytes": rbk + rbv, "scan_ms": ms,
                           "cache_tokens_per_s_scan": n_seq * T / (ms * 1e-3),
                           "scan_gbs": alg / (ms * 1e-3) / 1e9,
                           "frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "note": "VALU-bound: values decoded in the code domain"}
    del ck, cv, ws
    ws = torch.empty(max(api.pgkq_fp16_decode_workspace_bytes(d, n_seq, cfg.n_q, n_kv, T, cfg.n_splits), 256),
                     dtype=torch.uint8, device=dev)
    ms = timed(lambda: api.pgkq_fp16_decode_attn(q, K, Vt, n_splits=cfg.n_splits, out=out, workspace=ws,
                                                 events=(e0, e1)))
    alg = n_seq * n_kv * T * 4 * d
    res["fp16_cache"] = {"record_bytes": 2 * d, "scan_ms": ms,
                         "cache_tokens_per_s_scan": n_seq * T / (ms * 1e-3),
                         "scan_gbs": alg / (ms * 1e-3) / 1e9,
                         "frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return res


def run_decode_step(api, torch, dev, cfg, p, q, K, V, codes, Vt, signs, perm, cb, S, ws, flush, E,
                    reps: int = 20):
    """The fused append + decode step on the main workload: the token of slot
    T - 1 is encoded and written again (same key and value rows), then
    attention runs over the T cached tokens; whole call, caches evicted
    before each call.  Steps alternate with plain decode calls on the same
    cache, so that the two are timed under the same conditions."""
    n_seq, n_kv, T, d = K.shape
    k_new = K[:, :, T - 1].contiguous()
    v_new = V[:, :, T - 1].contiguous()
    out = torch.empty((n_seq, cfg.n_q, d), dtype=torch.float32, device=dev)
    c0, c1 = E(), E()
    ts = {"step": [], "call": []}
    for r in range(reps + 3):
        for kind in ("call", "step"):
            flush.fill_(r & 255)
            c0.record()
            if kind == "step":
                api.pgkq_decode_step(p, q, k_new, v_new, codes, Vt, T - 1, signs, perm, cb, S,
                                     n_splits=cfg.n_splits, out=out, workspace=ws)
            else:
                api.pgkq_decode_attn(p, q, codes, Vt, signs, perm, cb, S, n_splits=cfg.n_splits,
                                     out=out, workspace=ws)
            c1.record()
            torch.cuda.synchronize()
            if r >= 3:
                ts[kind].append(c0.elapsed_time(c1))
    ms = float(np.median(ts["step"]))
    return {"description": "append one token per stream (encode its key, write its value) and "
                           "decode over the 32768 cached tokens, one call",
            "call_ms": ms, "cache_tokens_per_s": n_seq * T / (ms * 1e-3),
            "plain_call_ms": float(np.median(ts["call"])),
            "note": "plain_call_ms: the decode call without the append, alternating with the steps"}


def run_nano_latency(api, torch, dev, E, reps: int = 50):
    """The NanoGPT-256 cache of one decode step (24 flattened layer-heads, 128
    tokens, d64, fp32 keys and query): latency of the whole decode call, all
    launches included; cache resident, no roofline claim."""
    from synth import CONFIGS, make_inputs
    cfg = CONFIGS["nano_t128"]
    inp = make_inputs(cfg)
    n_seq, n_kv, T, d = inp["K"].shape
    p = api.PgkqParams(d, cfg.b_main, cfg.b_angle, cfg.qjl_m, 1)
    K = torch.from_numpy(inp["K"]).to(dev)
    Vt = api.pgkq_pack_values(torch.from_numpy(inp["V"]).to(dev), capacity=(T + 31) // 32 * 32)
    q = torch.from_numpy(inp["q"]).to(dev)
    signs = torch.from_numpy(inp["signs"]).to(dev)
    S = torch.from_numpy(inp["S"]).to(dev)
    _, _, cb = api.pgkq_calibrate(p, K)
    codes = api.pgkq_encode(p, K, signs, None, cb, S, capacity=Vt.shape[2])
    out = torch.empty((n_seq, cfg.n_q, d), dtype=torch.float32, device=dev)
    ws = torch.empty(api.pgkq_decode_workspace_bytes(p, n_seq, cfg.n_q, n_kv, T), dtype=torch.uint8, device=dev)
    c0, c1 = E(), E()
    ts = []
    for r in range(reps + 5):
        c0.record()
        api.pgkq_decode_attn(p, q, codes, Vt, signs, None, cb, S, n_tokens=T, out=out, workspace=ws)
        c1.record()
        torch.cuda.synchronize()
        if r >= 5:
            ts.append(c0.elapsed_time(c1))
    us = np.array(ts) * 1e3
    return {"description": cfg.description, "latency_us_p50": float(np.median(us)),
            "latency_us_p10": float(np.percentile(us, 10)), "latency_us_p90": float(np.percentile(us, 90)),
            "note": "cache-resident, launch-bound: latency only"}


def decode_only(api, torch, dev, name: str, calls: int) -> dict:
    """Only the decode call of one named workload, `calls` times with the
    Infinity Cache evicted before each (for a rocprofv3 kernel trace of the
    call's launches: query preparation, scan, merge)."""
    from synth import CONFIGS, make_inputs
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    n_seq, n_kv, T, d = inp["K"].shape
    p = api.PgkqParams(d, cfg.b_main, cfg.b_angle, cfg.qjl_m, 1)
    K = torch.from_numpy(inp["K"]).to(dev)
    Vt = api.pgkq_pack_values(torch.from_numpy(inp["V"]).to(dev))
    q = torch.from_numpy(inp["q"]).to(dev)
    if cfg.q_dtype == "bf16":
        q = q.to(torch.bfloat16)
    signs = torch.from_numpy(inp["signs"]).to(dev)
    S = torch.from_numpy(inp["S"]).to(dev) if cfg.qjl_m else None
    _, _, cb = api.pgkq_calibrate(p, K)
    codes = api.pgkq_encode(p, K, signs, None, cb, S, capacity=T)
    del K
    out = torch.empty((n_seq, cfg.n_q, d), dtype=torch.float32, device=dev)
    ws = torch.empty(api.pgkq_decode_workspace_bytes(p, n_seq, cfg.n_q, n_kv, T, cfg.n_splits),
                     dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for r in range(calls + 3):
        flush.fill_(r & 255)
        e0.record()
        api.pgkq_decode_attn(p, q, codes, Vt, signs, None, cb, S, n_splits=cfg.n_splits, out=out,
                             workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        if r >= 3:
            ts.append(e0.elapsed_time(e1))
    return {"workload": name, "description": cfg.description, "calls": calls + 3,
            "call_ms_p50": float(np.median(ts))}


def run_other_workloads(api, torch, dev, flush, E, reps: int = 20):
    """Decode of the other configurations of the pages' workload list on this
    GPU (NanoGPT-256 context with and without QJL, the 131k-token single
    stream): whole decode call and scan kernel, keys encoded and values packed
    beforehand (inputs resident).  Cache tokens count every flattened layer.
    The NanoGPT-256 context is also decoded from the fp16 cache (the FP16
    comparator), with the fidelity of the PGKQ output against it."""
    from synth import CONFIGS, make_inputs
    res = {}
    for name in ("nano_b64_t512", "nano_b64_t512_b4", "gqa_b1_t131k"):
        cfg = CONFIGS[name]
        inp = make_inputs(cfg)
        n_seq, n_kv, T, d = inp["K"].shape
        p = api.PgkqParams(d, cfg.b_main, cfg.b_angle, cfg.qjl_m, 1)
        K = torch.from_numpy(inp["K"]).to(dev)
        Vt = api.pgkq_pack_values(torch.from_numpy(inp["V"]).to(dev))
        q = torch.from_numpy(inp["q"]).to(dev)
        if cfg.q_dtype == "bf16":
            q = q.to(torch.bfloat16)
        signs = torch.from_numpy(inp["signs"]).to(dev)
        S = torch.from_numpy(inp["S"]).to(dev) if cfg.qjl_m else None
        _, perm, cb = api.pgkq_calibrate(p, K)
        codes = api.pgkq_encode(p, K, signs, None, cb, S, capacity=T)
        out = torch.empty((n_seq, cfg.n_q, d), dtype=torch.float32, device=dev)
        ws = torch.empty(api.pgkq_decode_workspace_bytes(p, n_seq, cfg.n_q, n_kv, T, cfg.n_splits),
                         dtype=torch.uint8, device=dev)
        e0, e1, c0, c1 = E(), E(), E(), E()
        e0.record()
        e1.record()
        scan, call = [], []
        for r in range(reps + 3):   # whole call
            flush.fill_(r & 255)
            c0.record()
            api.pgkq_decode_attn(p, q, codes, Vt, signs, None, cb, S, n_splits=cfg.n_splits, out=out,
                                 workspace=ws)
            c1.record()
            torch.cuda.synchronize()
            if r >= 3:
                call.append(c0.elapsed_time(c1))
        for r in range(reps + 3):   # scan kernel (events recorded by the library)
            flush.fill_(r & 255)
            api.pgkq_decode_attn(p, q, codes, Vt, signs, None, cb, S, n_splits=cfg.n_splits, out=out,
                                 workspace=ws, events=(e0, e1))
            torch.cuda.synchronize()
            if r >= 3:
                scan.append(e0.elapsed_time(e1))
        scan_ms, call_ms = float(np.median(scan)), float(np.median(call))
        rb = api.pgkq_record_bytes(p)
        alg = n_seq * n_kv * T * (rb + 2 * d)
        res[name] = {"description": cfg.description, "record_bytes": rb,
                     "decode_call_ms": call_ms, "scan_ms": scan_ms,
                     "cache_tokens_per_s": n_seq * cfg.layers * T / (call_ms * 1e-3),
                     "scan_gbs": alg / (scan_ms * 1e-3) / 1e9,
                     "scan_frac": alg / (scan_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if name == "nano_b64_t512":
            # the FP16 comparator on the same keys (as fp16), values and queries
            K16 = K.to(torch.float16)
            out16 = torch.empty_like(out)
            ws16 = torch.empty(max(api.pgkq_fp16_decode_workspace_bytes(d, n_seq, cfg.n_q, n_kv, T), 256),
                               dtype=torch.uint8, device=dev)
            f16 = []
            for r in range(reps + 3):
                flush.fill_(r & 255)
                c0.record()
                api.pgkq_fp16_decode_attn(q, K16, Vt, out=out16, workspace=ws16)
                c1.record()
                torch.cuda.synchronize()
                if r >= 3:
                    f16.append(c0.elapsed_time(c1))
            f16_ms = float(np.median(f16))
            api.pgkq_decode_attn(p, q, codes, Vt, signs, None, cb, S, out=out, workspace=ws)
            torch.cuda.synchronize()
            a = out.double().flatten()
            ref = out16.double().flatten()
            res["nano_b64_t512_fp16"] = {
                "description": "the same NanoGPT-256 context from the fp16 cache (FP16 comparator)",
                "decode_call_ms": f16_ms,
                "cache_tokens_per_s": n_seq * cfg.layers * T / (f16_ms * 1e-3),
                "gbs": n_seq * n_kv * T * 4 * d / (f16_ms * 1e-3) / 1e9,
                "pgkq_vs_fp16": {"max_abs": float((a - ref).abs().max()),
                                 "rel_l2": float((a - ref).norm() / ref.norm()),
                                 "cosine": float(torch.dot(a, ref) / (a.norm() * ref.norm())),
                                 "note": "fidelity of the method on these synthetic inputs (the "
                                         "float64 oracle gives the same figures), not a parity measure"}}
            del K16, out16, ws16
        del K, Vt, q, codes, ws, inp
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration for rocprofv3)")
    ap.add_argument("--decode-only", metavar="WORKLOAD", default=None,
                    help="run only the decode call of one named workload (e.g. gqa_b1_t131k), "
                         "--steps times, for a rocprofv3 kernel trace of its launches")
    ap.add_argument("--read-probe", action="store_true",
                    help="run only the library's read probe over the decode scan's algorithmic "
                         "bytes, --steps times (the read ceiling, for rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; use --gpus 1"}))
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")

    if args.copy_probe:
        n = 1 << 30
        a = torch.ones(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_per_launch": n, "launches": args.steps}))
        return

    import compressed_cache_decode_pgkq_amd as api
    from synth import CONFIGS

    if args.decode_only:
        print(json.dumps(decode_only(api, torch, dev, args.decode_only, args.steps)))
        return

    if args.read_probe:
        c = CONFIGS["gqa_b16_t32k"]
        rbp = api.pgkq_record_bytes(api.PgkqParams(c.head_dim, c.b_main, c.b_angle, c.qjl_m, 1))
        nbytes = c.n_seq * c.n_kv * c.n_tokens * (rbp + 2 * c.head_dim)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        res = measure_read(api, torch, dev, nbytes, flush, reps=args.steps)
        print(json.dumps({"read_probe": res, "launches": args.steps + 3}))
        return

    cfg = CONFIGS["gqa_b16_t32k"]           # decode workload
    ecfg = CONFIGS["gqa_b16_t32k_encode"]          # the same keys, encoded with the reorder step
    inp = generate(cfg)
    p = api.PgkqParams(cfg.head_dim, cfg.b_main, cfg.b_angle, cfg.qjl_m, 1)
    n_seq, n_kv, T, d = inp["K"].shape
    K = torch.from_numpy(inp["K"]).to(dev)
    V = torch.from_numpy(inp["V"]).to(dev)      # value rows (encoded as keys by the PGKQ-KV control)
    Vt = api.pgkq_pack_values(V)                  # the fp16 value cache, 32-token tiles
    q = torch.from_numpy(inp["q"]).to(torch.bfloat16).to(dev)
    signs = torch.from_numpy(inp["signs"]).to(dev)
    S = torch.from_numpy(inp["S"]).to(dev)
    rb = api.pgkq_record_bytes(p)
    codes = torch.zeros((n_seq, n_kv, T * rb), dtype=torch.uint8, device=dev)
    out = torch.empty((n_seq, cfg.n_q, d), dtype=torch.float32, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ws = torch.empty(api.pgkq_decode_workspace_bytes(p, n_seq, cfg.n_q, n_kv, T, cfg.n_splits),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident: K {K.numel() * 2 / 2**30:.2f} GiB, V {V.numel() * 2 / 2**30:.2f} GiB, "
        f"codes {codes.numel() / 2**20:.1f} MiB")

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(ev=None):
        if ev:
            ev[0].record()
        _, perm, cb = api.pgkq_calibrate(p, K, reorder=ecfg.reorder)
        if ev:
            ev[1].record()
        api.pgkq_encode(p, K, signs, perm, cb, S, codes=codes, capacity=T)
        if ev:
            ev[2].record()
        flush.fill_(1)
        if ev:
            ev[3].record()
        api.pgkq_decode_attn(p, q, codes, Vt, signs, perm, cb, S, n_splits=cfg.n_splits, out=out,
                             workspace=ws)
        if ev:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[E() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the scan kernel alone: the same decode call (caches evicted first) with the
    # library recording events around the scan launch on its stream; kept out
    # of the timed steps, whose decode phase is the plain call
    sev = [(E(), E()) for _ in range(args.steps)]
    for e in sev:  # torch creates the HIP event on first record; the library re-records them
        e[0].record()
        e[1].record()
    _, perm, cb = api.pgkq_calibrate(p, K, reorder=ecfg.reorder)
    for e in sev:
        flush.fill_(1)
        api.pgkq_decode_attn(p, q, codes, Vt, signs, perm, cb, S, n_splits=cfg.n_splits, out=out,
                             workspace=ws, events=e)
    torch.cuda.synchronize()
    ph = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[3].elapsed_time(e[4]),
                    f[0].elapsed_time(f[1])] for e, f in zip(evs, sev)])  # ms
    cal_ms, enc_ms, dec_ms, scan_ms = (float(np.median(ph[:, k])) for k in range(4))
    scan_mean = float(np.mean(ph[:, 3]))
    pct = lambda k: {"p10": float(np.percentile(ph[:, k], 10)), "p50": float(np.median(ph[:, k])),  # noqa: E731
                     "p90": float(np.percentile(ph[:, k], 90))}
    copy_gbs = measure_copy(torch, dev)
    read = measure_read(api, torch, dev, n_seq * n_kv * T * (rb + 2 * d), flush)
    step_res = run_decode_step(api, torch, dev, cfg, p, q, K, V, codes, Vt, signs, perm, cb, S, ws,
                               flush, E)
    controls = run_controls(api, torch, dev, cfg, K, V, Vt, q, signs, S, flush, E)
    others = run_other_workloads(api, torch, dev, flush, E)
    others["nano_t128_latency"] = run_nano_latency(api, torch, dev, E)

    token_heads = n_seq * n_kv * T
    alg_bytes = token_heads * (rb + 2 * d)
    cache_tokens = n_seq * T
    value = cache_tokens / (dec_ms * 1e-3)
    achieved = alg_bytes / (scan_mean * 1e-3) / 1e9
    traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        with open(PROFILE_TRAFFIC) as f:
            tr = json.load(f)
        if tr.get("source_hash") == scan_source_hash():
            traffic = tr.get("bytes_per_launch")
    n_keys = n_seq * n_kv * T
    # the encoder's binding resource is the vector ALU: issued lane-operations
    # per key from the committed instruction-count profile of the same sources
    enc_valu = None
    if os.path.exists(PROFILE_UTIL):
        with open(PROFILE_UTIL) as f:
            ut = json.load(f)
        kern = ut.get("kernels", {}).get(ENCODE_KERNEL)
        if ut.get("encode_source_hash") == encode_source_hash() and kern:
            enc_valu = kern["valu_instr_per_unit"] * 64.0
    enc_flops = n_keys * 2.0 * cfg.qjl_m * d
    enc_gbs = n_keys * (2 * d + rb) / (enc_ms * 1e-3) / 1e9
    result = {
        "metric": "decode-attn cache tokens/s/GPU + % HBM roofline; PGKQ encode keys/s",
        "value": value,
        "unit": "cache tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; keys with log-normal channel scales and 4 outlier channels x10)",
        "config": {
            "workload": "GQA decode 32q/8kv, head_dim 128, 32768-token cache, batch 16, "
                        f"b_main 3 / b_angle 2, QJL m 128, {cfg.n_splits} token splits; encode of "
                        "its 4194304 fp16 keys with the channel reorder step",
            "n_seq": n_seq, "n_q": cfg.n_q, "n_kv": n_kv, "n_tokens": T, "head_dim": d,
            "b_main": cfg.b_main, "b_angle": cfg.b_angle, "qjl_m": cfg.qjl_m,
            "n_splits": cfg.n_splits, "record_bytes": rb,
        },
        "phases_ms": {"calibrate": cal_ms, "encode": enc_ms, "decode_attn": dec_ms,
                      "decode_scan_kernel": scan_ms},
        "phase_percentiles_ms": {"decode_attn": pct(2), "decode_scan_kernel": pct(3),
                                 "encode": pct(1)},
        "decode": {"cache_tokens_per_s": value, "token_heads_per_s": token_heads / (dec_ms * 1e-3),
                   "algorithmic_bytes": alg_bytes,
                   "gbs_whole_call": alg_bytes / (dec_ms * 1e-3) / 1e9},
        "encode": {"keys_per_s": n_keys / (enc_ms * 1e-3),
                   "keys_per_s_with_calibrate": n_keys / ((enc_ms + cal_ms) * 1e-3),
                   "hbm_gbs": enc_gbs,
                   "projection_tflops": enc_flops / (enc_ms * 1e-3) / 1e12,
                   # against the method's work: HBM bytes (fp16 keys in, records
                   # out) over the 8 TB/s peak, and the projection's three
                   # split-fp16 products against the 2.5 PFLOP/s fp16 MFMA peak;
                   # both ceilings are ~165 us for this workload.  The vector-ALU
                   # issue rate is a diagnostic of the kernel, not of the method
                   "roofline": {"bound": "hbm", "achieved": enc_gbs, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": enc_gbs / HBM_PEAK_GBS,
                                "algorithmic_bytes_per_key": 2 * d + rb,
                                "mfma_frac": enc_flops * 3 / (enc_ms * 1e-3) / 2.5e15,
                                "mfma_flops_per_key": 3 * 2 * cfg.qjl_m * d,
                                "valu_issue_frac": (enc_valu * n_keys / (enc_ms * 1e-3) / VALU_PEAK_LANE_OPS) if enc_valu else None,
                                "valu_lane_ops_per_key": enc_valu,
                                "note": "frac: (2 d + record) bytes per key over the HBM peak; "
                                        "mfma_frac: three split-fp16 products per projection flop "
                                        "over the fp16 MFMA peak; valu_issue_frac: profiled VALU "
                                        "lane-operations per key (profiles/utilization_gqa32k_b16.json) "
                                        "over the issue rate of 256 CUs x 64 lanes x 2.4 GHz"}},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "decode_scan_kernel<128,3,QJL,G=4>", "launch_ms": scan_mean,
                     "measured_copy_gbs": copy_gbs,
                     # the same byte count read by the read probe (the scans'
                     # load path and nothing else): the ceiling measured here
                     "measured_read_gbs": read["gbs"],
                     "frac_of_measured_read": achieved / read["gbs"]},
        "decode_step": step_res,
        "controls": controls,
        "other_workloads": others,
    }
    if not args.no_cpu_baseline:
        cb_res = cpu_baseline(cfg, inp)
        result["cpu_baseline"] = cb_res["decode"]
        result["cpu_baseline_encode"] = cb_res["encode"]
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
