"""Benchmark: compress / decompress throughput of the bf16 exponent codec.

One step = one pass of the whole path over one buffer resident in HBM:
zc_compress of every chunk, then zc_decompress of every stream.  The default
workload is the FSDP parameter all-gather shard (64 chunks x 4 Mi bf16,
sigma log-uniform in [0.005, 0.05]); --workload picks another (1..5).

Throughput is GB/s of uncompressed input (2 bytes per value).  Each call is
timed with HIP events recorded on the stream the library launches on; a 1 GiB
write evicts the 256 MB Infinity Cache before each call, outside the timed
intervals.  After the timed steps a plain device copy of the input (2n bytes
read, 2n written) is timed the same way: it is the achievable streaming rate
on this device, and the reference kernel that calibrates the HBM byte
counters.

roofline.traffic is read from the committed counter summary of this workload
(profiles/zc_kernels_<workload>_traffic.txt) when the kernel sources hash to
the value recorded there; otherwise it is null.

With the default workload, workloads 1, 3, 4 and 5 are then timed the same
way (compress and decompress only, same warm-up and step counts) and
reported under per_config.

The oracle (plain C, test infrastructure) is timed on the host cores over the
same workload for the cpu_baseline field.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
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
KERNEL_NAMES = {"compress": "zc_compress_kernel",
                "decompress": "zc_decompress_kernel"}
# Every file the kernels are compiled from (and the flags they are built with).
KERNEL_SOURCES = [
    "lossless_bf16_tensor_sign_amd/csrc/zc_kernels.hip",
    "lossless_bf16_tensor_sign_amd/csrc/zc_table.cpp",
    "lossless_bf16_tensor_sign_amd/csrc/zc_table.h",
    "lossless_bf16_tensor_sign_amd/csrc/zc_table_emit.cpp",
    "lossless_bf16_tensor_sign_amd/build.py",
    "include/zc.h",
]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_sources_sha256():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            data = f.read()
        h.update(rel.encode() + b"\0" + str(len(data)).encode() + b"\0" + data)
    return h.hexdigest()


def traffic_path(workload_name):
    return os.path.join(ROOT, "profiles", "zc_kernels_%s_traffic.txt" % workload_name)


def read_traffic(workload_name):
    """Per-dispatch HBM bytes by kernel from the committed counter summary,
    or None when it is absent or was taken from other kernel sources."""
    path = traffic_path(workload_name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            ln = ln.strip()
            if not ln or ln.startswith("#") or "=" not in ln:
                continue
            k, v = ln.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    out = {}
    for name in KERNEL_NAMES.values():
        key = name + ".traffic_bytes"
        if key in kv:
            out[name] = int(float(kv[key]))
    return out


def device_info():
    """The GPU and the software of the run; the peak engine and memory clocks
    come from the HIP runtime (hipDeviceAttributeClockRate = 5 and
    hipDeviceAttributeMemoryClockRate = 60 in hip_runtime_api.h, kHz)."""
    import ctypes
    import torch
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "gcn_arch": p.gcnArchName, "compute_units": p.multi_processor_count,
            "hbm_GiB": round(p.total_memory / 2**30, 1), "l2_MiB": round(p.L2_cache_size / 2**20, 1),
            "hip_runtime": torch.version.hip, "torch": torch.__version__}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int()
        for key, attr in (("peak_engine_clock_MHz", 5), ("peak_memory_clock_MHz", 60)):
            if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) == 0:
                info[key] = v.value // 1000
    except OSError:
        pass
    return info


def host_cpu():
    """CPU model name and core counts of this host (from /proc/cpuinfo and the
    scheduler's affinity mask)."""
    model, sockets, cores_per = None, set(), {}
    try:
        with open("/proc/cpuinfo") as f:
            phys = None
            for ln in f:
                k, _, v = ln.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                    sockets.add(v)
                elif k == "cpu cores" and phys is not None:
                    cores_per[phys] = int(v)
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {
        "cpu_model": model,
        "logical_cpus": os.cpu_count(),
        "physical_cores": sum(cores_per.values()) if cores_per else None,
        "sockets": len(sockets) if sockets else None,
        "usable_cpus": usable,
    }


def cpu_baseline(w, counts, threads, budget_s):
    """The oracle on the host: one thread over the first chunk (per-core
    rate), then the first k chunks spread over `threads` threads, k chosen so
    that about budget_s seconds of CPU time are spent (the whole workload if
    it fits).  Each chunk is compressed, decompressed and checked."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle
    oracle.build(force=False)
    vo = np.concatenate([[0], np.cumsum(counts)])
    order = [c for c in range(len(counts)) if counts[c] > 0]

    def run(c):
        x = w[vo[c]:vo[c + 1]]
        t0 = time.perf_counter()
        s = oracle.compress_chunk(x)
        t1 = time.perf_counter()
        r, back = oracle.decompress_chunk(s, x.size)
        t2 = time.perf_counter()
        return t1 - t0, t2 - t1, s.size, r == 0 and np.array_equal(back, x)

    tc1, td1, _, ok1 = run(order[0])
    one = 2.0 * counts[order[0]]
    per_chunk = (tc1 + td1) * float(np.mean(counts[order])) / counts[order[0]]
    k = int(budget_s / max(per_chunk, 1e-9))
    k = min(len(order), max(threads, (k // threads) * threads))
    sample = order[:k]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(run, sample))
    wall = time.perf_counter() - t0
    nbytes = 2.0 * float(sum(counts[c] for c in sample))
    tc = sum(r[0] for r in res)
    td = sum(r[1] for r in res)
    ok = ok1 and all(r[3] for r in res)
    return {
        "value": round(nbytes / wall / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d of %d chunks (%.1f MB of input), each compressed then "
                  "decompressed and checked, spread over %d threads; value = "
                  "input bytes / wall time of both directions"
                  % (len(sample), len(order), nbytes / 1e6, threads),
        "compress_GBps_per_core": round(one / tc1 / 1e9, 4),
        "decompress_GBps_per_core": round(one / td1 / 1e9, 4),
        "thread_seconds_compress": round(tc, 3),
        "thread_seconds_decompress": round(td, 3),
        "wall_s": round(wall, 3),
        "comp_bytes_sample": int(sum(r[2] for r in res)),
        "roundtrip_ok": bool(ok),
        "host": host_cpu(),
    }


def time_pipeline(args, x, counts, dev, evict, ev):
    """zc_pipeline round trip (compress, device-copy link, decompress) in
    args.pipeline groups on three streams, against the same call with all
    stages on one stream; both after the cache flush, 5 runs each."""
    import numpy as np
    import torch
    from lossless_bf16_tensor_sign_amd import zc
    cap = zc.zc_bound(counts)
    send = torch.empty(cap, dtype=torch.uint8, device=dev)
    recv = torch.empty(cap, dtype=torch.uint8, device=dev)
    sizes = torch.empty(len(counts), dtype=torch.int64, device=dev)
    ws = torch.zeros(zc.zc_workspace_bytes(counts), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    cur = torch.cuda.current_stream()
    three = tuple(torch.cuda.Stream(device=dev) for _ in range(3))
    out = {"groups": args.pipeline}
    for label, streams in (("three_streams", three), ("one_stream", (cur, cur, cur))):
        times = []
        for i in range(6):
            evict(i + 21)
            for s_ in streams:
                s_.wait_stream(cur)
            e0, e1 = ev(), ev()
            e0.record(streams[0])
            r = zc.zc_pipeline(x, counts, args.pipeline, send, recv, sizes, y, status, ws,
                               s_comp=streams[0], s_link=streams[1], s_dec=streams[2])
            if r != zc.ZC_OK:
                raise zc.ZcError(r, "zc_pipeline")
            e1.record(streams[2])
            cur.wait_stream(streams[2])
            if i:
                times.append((e0, e1))
        torch.cuda.synchronize()
        if int(status.item()) != 0 or not torch.equal(x, y):
            log("PIPELINE ROUND TRIP FAILED")
            sys.exit(1)
        out[label + "_ms"] = round(float(np.mean([a.elapsed_time(b) for a, b in times])), 4)
    log("pipeline: %s" % out)
    return out


def measure_workload(wl, steps, warmup, dev, stream, evict, ev):
    """Compress and decompress timings of workload wl with host chunk counts,
    measured the way the headline workload is (cache flush before each call,
    HIP events on the library's stream), and its round trip checked.  For a
    workload of equal chunks (the gradient reduce-scatter buffer) the decode
    and chunk-order fp32 sum of its streams (zc_decompress_reduce, the
    receive side of a compressed reduce-scatter) is timed the same way and
    checked against chunk-order PyTorch fp32 additions."""
    import numpy as np
    import torch
    from lossless_bf16_tensor_sign_amd import synth, zc
    w, counts = synth.make(wl, seed=synth.default_seed(wl), workers=8)
    n = int(counts.sum())
    x = torch.from_numpy(w.view(np.int16)).to(dev)
    del w
    buf = torch.empty(zc.zc_bound(counts), dtype=torch.uint8, device=dev)
    sizes = torch.empty(len(counts), dtype=torch.int64, device=dev)
    ws = torch.zeros(zc.zc_workspace_bytes(counts), dtype=torch.uint8, device=dev)
    y = torch.empty(n, dtype=torch.int16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    tc, td = [], []
    for i in range(warmup + steps):
        evict(i + 31)
        e0, e1 = ev(), ev()
        e0.record(stream)
        r = zc.zc_compress(x, counts, buf, sizes, ws, stream=stream)
        e1.record(stream)
        if r != zc.ZC_OK:
            raise zc.ZcError(r, "zc_compress")
        evict(i + 32)
        e2, e3 = ev(), ev()
        e2.record(stream)
        r = zc.zc_decompress(buf, counts, y, status, stream=stream)
        e3.record(stream)
        if r != zc.ZC_OK:
            raise zc.ZcError(r, "zc_decompress")
        if i >= warmup:
            tc.append((e0, e1))
            td.append((e2, e3))
    torch.cuda.synchronize()
    if int(status.item()) != 0 or not torch.equal(x, y):
        log("ROUND TRIP FAILED on workload %d" % wl)
        sys.exit(1)
    comp = int(sizes.sum().item())
    c_s = float(np.mean([a.elapsed_time(b) for a, b in tc])) * 1e-3
    d_s = float(np.mean([a.elapsed_time(b) for a, b in td])) * 1e-3
    alg = 2 * n + comp
    out = {
        "values": n,
        "chunks": int(len(counts)),
        "steps": steps,
        "compress_ms": round(c_s * 1e3, 4),
        "decompress_ms": round(d_s * 1e3, 4),
        "compress_GBps": round(2 * n / c_s / 1e9, 2),
        "decompress_GBps": round(2 * n / d_s / 1e9, 2),
        "ratio": round(2 * n / comp, 5),
        "pct_hbm_peak_algorithmic": {
            "compress": round(100 * alg / c_s / 1e9 / HBM_PEAK_GBPS, 2),
            "decompress": round(100 * alg / d_s / 1e9 / HBM_PEAK_GBPS, 2),
        },
    }
    if wl == 3 and np.all(counts == counts[0]):
        shard, c = int(counts[0]), int(len(counts))
        need = zc.zc_reduce_scratch_bytes(shard, c)
        scratch = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        red = torch.empty(shard, dtype=torch.float32, device=dev)
        tr = []
        for i in range(warmup + steps):
            evict(i + 33)
            e0, e1 = ev(), ev()
            e0.record(stream)
            r = zc.zc_decompress_reduce(buf, shard, c, red, status, scratch, stream=stream)
            e1.record(stream)
            if r != zc.ZC_OK:
                raise zc.ZcError(r, "zc_decompress_reduce")
            if i >= warmup:
                tr.append((e0, e1))
        torch.cuda.synchronize()
        acc = torch.zeros(shard, dtype=torch.float32, device=dev)
        for k in range(c):
            acc = acc + (x[k * shard:(k + 1) * shard].to(torch.int32) << 16).view(torch.float32)
        same = (acc.view(torch.int32) == red.view(torch.int32)) | (acc.isnan() & red.isnan())
        if int(status.item()) != 0 or not bool(same.all()):
            log("DECODE + SUM FAILED on workload %d" % wl)
            sys.exit(1)
        r_s = float(np.mean([a.elapsed_time(b) for a, b in tr])) * 1e-3
        out["decode_sum"] = {
            "streams": c,
            "values_per_stream": shard,
            "form": "one kernel" if need == 0 else "slabs",
            "scratch_bytes": need,
            "ms": round(r_s * 1e3, 4),
            "ms_median": round(float(np.median([a.elapsed_time(b) for a, b in tr])), 4),
            "GBps_received": round(2 * n / r_s / 1e9, 2),
        }
    log("workload %d: %s" % (wl, out))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=16)
    ap.add_argument("--cpu-budget-s", type=float, default=20.0,
                    help="CPU seconds (summed over threads) of the oracle run")
    ap.add_argument("--copies", type=int, default=3,
                    help="timed plain device copies of the input after the steps")
    ap.add_argument("--flush", choices=["clean", "write"], default="clean",
                    help="cache state before each timed call: 'write' = 1 GiB written "
                         "(the Infinity Cache is left full of the flush's dirty lines); "
                         "'clean' = the same 1 GiB then read back (cold and clean)")
    ap.add_argument("--device-counts", action="store_true",
                    help="time zc_compress_dev / zc_decompress_dev, with the chunk "
                         "counts in device memory (the MoE router's split)")
    ap.add_argument("--pipeline", type=int, default=0, metavar="G",
                    help="also time zc_pipeline (compress, device-copy link, decompress) "
                         "in G chunk groups on three streams and on one")
    ap.add_argument("--reduce", action="store_true",
                    help="decode with zc_decompress_reduce: the chunks are one rank's "
                         "shard as received from each peer, summed in fp32 in chunk "
                         "order (equal chunks only)")
    ap.add_argument("--per-config", default=None, metavar="LIST",
                    help="comma-separated other workloads to time after the headline "
                         "one (compress and decompress only), reported under per_config; "
                         "default 1,3,4,5 for workload 2 and none otherwise; '' for none")
    ap.add_argument("--per-config-steps", type=int, default=None,
                    help="timed steps per other workload (default: --steps, after --warmup)")
    args = ap.parse_args()
    if args.per_config is None:
        args.per_config = "1,3,4,5" if args.workload == 2 else ""
    others = [int(v) for v in args.per_config.split(",") if v.strip()]
    if any(v not in (1, 2, 3, 4, 5) or v == args.workload for v in others):
        print("--per-config takes workloads 1..5 other than --workload", file=sys.stderr)
        sys.exit(2)

    if args.gpus != 1:
        print("bench.py measures one GPU only: this codec runs per GPU and no "
              "multi-GPU path is built, so --gpus %d is not supported."
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from lossless_bf16_tensor_sign_amd import synth, zc

    dev = torch.device("cuda:0")
    seed = synth.default_seed(args.workload)
    log("generating workload %d (%s)" % (args.workload, synth.NAMES[args.workload]))
    w, counts = synth.make(args.workload, seed=seed, workers=8)
    n = int(counts.sum())
    in_bytes = 2 * n
    x = torch.from_numpy(w.view(np.int16)).to(dev)
    if args.reduce and (args.device_counts or np.any(counts != counts[0])):
        print("--reduce needs equal chunks and host counts", file=sys.stderr)
        sys.exit(2)
    shard = int(counts[0])
    if args.device_counts:
        cap = zc.zc_bound_max(n, len(counts))
        wsb = zc.zc_workspace_bytes_max(n, len(counts))
    else:
        cap = zc.zc_bound(counts)
        wsb = zc.zc_workspace_bytes(counts)
    buf = torch.empty(cap, dtype=torch.uint8, device=dev)
    sizes = torch.empty(len(counts), dtype=torch.int64, device=dev)
    slots = torch.empty(len(counts), dtype=torch.int64, device=dev)
    dcounts = torch.from_numpy(np.asarray(counts, np.int64)).to(dev)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    y = torch.empty(n, dtype=torch.int16, device=dev)
    if args.reduce:
        # the decode + sum scratch (none when it runs as one kernel)
        y = torch.empty(max(zc.zc_reduce_scratch_bytes(shard, len(counts)) // 2, 8),
                        dtype=torch.int16, device=dev)
    red = torch.empty(shard if args.reduce else 4, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def evict(v):
        # 1 GiB written, so that no input or output of the previous call is
        # left in L2 or the Infinity Cache; with --flush clean it is then read
        # back, which writes the flush's own dirty lines out before the timed
        # call instead of during it
        flush.fill_(v & 0xFF)
        if args.flush == "clean":
            flush.view(torch.int64).sum()     # a plain 1 GiB read

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def step(times=None, i=0):
        evict(i)
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        e0.record(stream)
        if args.device_counts:
            r = zc.zc_compress_dev(x, dcounts, n, buf, sizes, slots, ws, stream=stream)
        else:
            r = zc.zc_compress(x, counts, buf, sizes, ws, stream=stream)
        e1.record(stream)
        if r != zc.ZC_OK:
            raise zc.ZcError(r, "zc_compress")
        evict(i + 1)
        e2.record(stream)
        if args.reduce:
            r = zc.zc_decompress_reduce(buf, shard, len(counts), red, status, y, stream=stream)
        elif args.device_counts:
            r = zc.zc_decompress_dev(buf, dcounts, n, y, status, ws, stream=stream)
        else:
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
    # (with --reduce, y is the scratch and holds no whole decode)
    ok = st == 0 and (args.reduce or torch.equal(x, y))
    if args.reduce:
        acc = torch.zeros(shard, dtype=torch.float32, device=dev)
        for k in range(len(counts)):
            acc = acc + (x[k * shard:(k + 1) * shard].to(torch.int32) << 16).view(torch.float32)
        same = (acc.view(torch.int32) == red.view(torch.int32)) | (acc.isnan() & red.isnan())
        ok = ok and bool(same.all())
        del acc
    comp = int(sizes.sum().item())
    if not ok:
        log("ROUND TRIP FAILED (status %#x)" % st)
        sys.exit(1)
    log("steps done: round trip exact")

    # plain device copy of the same bytes: streaming ceiling and the
    # calibration kernel of the byte counters
    tcopy = []
    ycopy = y if y.numel() == x.numel() else torch.empty_like(x)
    for i in range(args.copies):
        evict(i + 7)
        e0, e1 = ev(), ev()
        e0.record(stream)
        ycopy.copy_(x)
        e1.record(stream)
        tcopy.append((e0, e1))
    torch.cuda.synchronize()
    copy_s = float(np.mean([a.elapsed_time(b) for a, b in tcopy])) * 1e-3 if tcopy else None

    ratio = in_bytes / comp
    c_mean, d_mean = float(tc.mean()), float(td.mean())
    comp_gbps = in_bytes / c_mean / 1e9
    dec_gbps = in_bytes / d_mean / 1e9
    step_s = c_mean + d_mean
    value = in_bytes / step_s / 1e9
    alg_bytes = in_bytes + comp              # read 2n + write C, or read C + write 2n
    alg_c = alg_bytes / c_mean / 1e9
    # decode and sum: read C + write 4 n/C (the staged bf16 values are
    # written and read once more between the two kernels)
    alg_bytes_d = comp + 4 * shard if args.reduce else alg_bytes
    alg_d = alg_bytes_d / d_mean / 1e9
    dom = "decompress" if d_mean >= c_mean and not args.reduce else "compress"
    achieved = alg_d if dom == "decompress" else alg_c
    # the counter summaries cover the host-count kernels only
    traffic = None if args.device_counts else read_traffic(synth.NAMES[args.workload])
    dom_traffic = traffic.get(KERNEL_NAMES[dom]) if traffic else None

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
            "step": ("zc_compress_dev + zc_decompress_dev (counts in device memory)"
                     if args.device_counts else
                     "zc_compress + zc_decompress_reduce (fp32 chunk-order sum of %d "
                     "shards of %d values)" % (len(counts), shard)
                     if args.reduce else "zc_compress + zc_decompress") +
                    " of every chunk, 1 GiB cache flush before each call (untimed)",
            "flush": ("1 GiB written then read back (caches cold and clean)"
                      if args.flush == "clean" else "1 GiB written (caches cold, dirty)"),
        },
        "compress_GBps": round(comp_gbps, 2),
        "decompress_GBps": round(dec_gbps, 2),
        "compress_ms": round(c_mean * 1e3, 4),
        "decompress_ms": round(d_mean * 1e3, 4),
        "compress_ms_median": round(float(np.median(tc)) * 1e3, 4),
        "decompress_ms_median": round(float(np.median(td)) * 1e3, 4),
        "compress_ms_min": round(float(np.min(tc)) * 1e3, 4),
        "decompress_ms_min": round(float(np.min(td)) * 1e3, 4),
        "ratio": round(ratio, 5),
        "saving": round(1.0 - comp / in_bytes, 5),
        "comp_bytes": comp,
        "pct_hbm_peak_algorithmic": {
            "compress": round(100 * alg_c / HBM_PEAK_GBPS, 2),
            "decompress": round(100 * alg_d / HBM_PEAK_GBPS, 2),
        },
        "device_copy": None if copy_s is None else {
            "bytes_moved": 2 * in_bytes,
            "ms": round(copy_s * 1e3, 4),
            "GBps_moved": round(2 * in_bytes / copy_s / 1e9, 2),
            "frac_of_peak": round(2 * in_bytes / copy_s / 1e9 / HBM_PEAK_GBPS, 4),
        },
        "roofline": {
            "kernel": KERNEL_NAMES[dom],
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": dom_traffic,
            "algorithmic_bytes": alg_bytes,
            "traffic_by_kernel": traffic,
        },
        "wall_s_timed_region": round(t_wall, 4),
        "kernel_sources_sha256": kernel_sources_sha256(),
        "device": device_info(),
    }

    # sampled size estimate (8 tiles per chunk) and the switch's break-even
    # link speeds from this run's codec rates and stream sizes
    est = torch.empty(len(counts), dtype=torch.int64, device=dev)
    te = []
    for i in range(3):
        evict(i + 11)
        e0, e1 = ev(), ev()
        e0.record(stream)
        r = zc.zc_estimate(x, dcounts, n, 8, est, stream=stream)
        e1.record(stream)
        if r != zc.ZC_OK:
            raise zc.ZcError(r, "zc_estimate")
        te.append((e0, e1))
    torch.cuda.synchronize()
    est_total = int(est.sum().item())
    line["estimate"] = {
        "samples_per_chunk": 8,
        "ms": round(float(np.mean([a.elapsed_time(b) for a, b in te])), 4),
        "comp_bytes_estimated": est_total,
        "rel_error": round(est_total / comp - 1.0, 5),
    }
    sw = {}
    # (with --reduce the decode rate is that of decode + sum)
    colls = ["reduce_scatter"] if args.reduce else ["allgather", "alltoall"]
    for ranks in (8, 64):
        for coll in colls:
            st_, res = zc.zc_switch_decide(coll, ranks, in_bytes, est_total, 100.0, 0.0,
                                           comp_gbps, dec_gbps, dec_gbps)
            if st_ == zc.ZC_OK:
                sw["%s_%d" % (coll, ranks)] = round(res["breakeven_GBps"], 1)
    line["switch_breakeven_link_GBps"] = sw

    if args.pipeline:
        line["pipeline"] = time_pipeline(args, x, counts, dev, evict, ev)

    if others:
        # free the headline workload's buffers before the next ones are made
        del x, buf, y, ycopy, sizes, slots, dcounts, ws, red, est
        torch.cuda.empty_cache()
        line["per_config"] = {}
        for wl in others:
            log("per-config workload %d (%s)" % (wl, synth.NAMES[wl]))
            line["per_config"][synth.NAMES[wl]] = measure_workload(
                wl, args.per_config_steps or args.steps, args.warmup, dev, stream, evict, ev)

    if not args.no_cpu_baseline:
        threads = max(1, min(args.cpu_threads, os.cpu_count() or 1, len(counts)))
        log("cpu baseline: oracle, %d threads" % threads)
        line["cpu_baseline"] = cpu_baseline(w, counts, threads, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
