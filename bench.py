"""Benchmark: compress / decompress throughput of the bf16 exponent codec.

One step = one pass of the whole path over one buffer resident in HBM:
zc_compress of every chunk, then zc_decompress of every stream.  The default
workload is the FSDP parameter all-gather shard (64 chunks x 4 Mi bf16,
sigma log-uniform in [0.005, 0.05]); --workload picks another (1..5).

Throughput is GB/s of uncompressed input (2 bytes per value).  Each call is
timed with HIP events on the stream the library launches on; a 1 GiB write
evicts the 256 MB Infinity Cache before each call, outside the timed
intervals.  The oracle (plain C, test infrastructure) is timed on the host
cores over the same workload for the cpu_baseline field.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("compress / decompress GB/s (uncompressed input) on 1 MI355X; "
          "% HBM peak; ratio")
HBM_PEAK_GBPS = 8000.0


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def cpu_baseline(w, counts, threads):
    """The oracle over every chunk, chunks spread over `threads` threads."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle
    oracle.build(force=False)
    vo = np.concatenate([[0], np.cumsum(counts)])

    def comp(c):
        return oracle.compress_chunk(w[vo[c]:vo[c + 1]])

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        streams = list(ex.map(comp, range(len(counts))))
    t1 = time.perf_counter()

    def dec(c):
        r, back = oracle.decompress_chunk(streams[c], int(counts[c]))
        return r == 0 and np.array_equal(back, w[vo[c]:vo[c + 1]])

    with ThreadPoolExecutor(threads) as ex:
        ok = all(ex.map(dec, range(len(counts))))
    t2 = time.perf_counter()
    comp_bytes = sum(s.size for s in streams)
    return t1 - t0, t2 - t1, comp_bytes, ok


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=16)
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU "
              "path (the codec is per-GPU; collectives are out of scope), so "
              "--gpus %d is not supported." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from lossless_bf16_tensor_sign_amd import synth, zc

    dev = torch.device("cuda:0")
    seed = synth.default_seed(args.workload)
    log("generating workload %d" % args.workload)
    w, counts = synth.make(args.workload, seed=seed, workers=8)
    n = int(counts.sum())
    in_bytes = 2 * n
    x = torch.from_numpy(w.view(np.int16)).to(dev)
    cap = zc.zc_bound(counts)
    buf = torch.empty(cap, dtype=torch.uint8, device=dev)
    sizes = torch.empty(len(counts), dtype=torch.int64, device=dev)
    ws = torch.empty(zc.zc_workspace_bytes(counts), dtype=torch.uint8, device=dev)
    y = torch.empty(n, dtype=torch.int16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(times=None, i=0):
        flush.fill_(i & 0xFF)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e2 = torch.cuda.Event(enable_timing=True)
        e3 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        r = zc.zc_compress(x, counts, buf, sizes, ws, stream=stream)
        e1.record(stream)
        if r != zc.ZC_OK:
            raise zc.ZcError(r, "zc_compress")
        flush.fill_((i + 1) & 0xFF)
        e2.record(stream)
        r = zc.zc_decompress(buf, counts, y, status, stream=stream)
        e3.record(stream)
        if r != zc.ZC_OK:
            raise zc.ZcError(r, "zc_decompress")
        if times is not None:
            times.append((e0, e1, e2, e3))

    log("warmup %d" % args.warmup)
    for i in range(args.warmup):
        step(None, i)
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    times = []
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        step(times, i)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0

    tc = np.array([a.elapsed_time(b) for a, b, _, _ in times]) * 1e-3
    td = np.array([c.elapsed_time(d) for _, _, c, d in times]) * 1e-3
    st = int(status.item())
    ok = st == 0 and torch.equal(x, y)
    comp = int(sizes.sum().item())
    if not ok:
        log("ROUND TRIP FAILED (status %#x)" % st)
        sys.exit(1)

    ratio = in_bytes / comp
    c_mean, d_mean = float(tc.mean()), float(td.mean())
    comp_gbps = in_bytes / c_mean / 1e9
    dec_gbps = in_bytes / d_mean / 1e9
    step_s = c_mean + d_mean
    value = in_bytes / step_s / 1e9
    alg_c = (in_bytes + comp) / c_mean / 1e9      # algorithmic bytes / time
    alg_d = (comp + in_bytes) / d_mean / 1e9
    dom = "decompress" if d_mean >= c_mean else "compress"
    achieved = alg_d if dom == "decompress" else alg_c

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {
            "workload": synth.NAMES[args.workload],
            "values": n,
            "chunks": int(len(counts)),
            "bytes_in": in_bytes,
            "seed": seed,
            "step": "zc_compress + zc_decompress, MALL flushed before each",
        },
        "compress_GBps": round(comp_gbps, 2),
        "decompress_GBps": round(dec_gbps, 2),
        "compress_ms": round(c_mean * 1e3, 4),
        "decompress_ms": round(d_mean * 1e3, 4),
        "compress_ms_min": round(float(tc.min()) * 1e3, 4),
        "decompress_ms_min": round(float(td.min()) * 1e3, 4),
        "ratio": round(ratio, 5),
        "saving": round(1.0 - comp / in_bytes, 5),
        "comp_bytes": comp,
        "pct_hbm_peak_algorithmic": {
            "compress": round(100 * alg_c / HBM_PEAK_GBPS, 2),
            "decompress": round(100 * alg_d / HBM_PEAK_GBPS, 2),
        },
        "roofline": {
            "kernel": dom,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
        },
        "wall_s_timed_region": round(t_wall, 4),
    }

    if not args.no_cpu_baseline:
        threads = max(1, min(args.cpu_threads, os.cpu_count() or 1))
        log("cpu baseline: oracle, %d threads" % threads)
        t_c, t_d, cb, cok = cpu_baseline(w, counts, threads)
        line["cpu_baseline"] = {
            "value": round(in_bytes / (t_c + t_d) / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": "whole workload (%d chunks), compress then decompress, "
                      "chunks spread over %d threads" % (len(counts), threads),
            "compress_GBps": round(in_bytes / t_c / 1e9, 4),
            "decompress_GBps": round(in_bytes / t_d / 1e9, 4),
            "comp_bytes_equal_gpu": cb == comp,
            "roundtrip_ok": bool(cok),
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
