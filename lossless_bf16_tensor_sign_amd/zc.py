"""Python binding of libzc (the C ABI in include/zc.h).

Same names as the C entry points; this module only marshals pointers, sizes
and the current HIP stream.  Every step of compression and decompression runs
in the library's gfx950 kernels.  PyTorch provides device memory and streams.
There is no fallback: if libzc.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes as ct
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzc.so")

ZC_OK, ZC_EINVAL, ZC_ENOSPC, ZC_ECORRUPT, ZC_EHIP = 0, -1, -2, -3, -4
REASONS = {
    1: "HEADER", 2: "SIZE", 3: "GAP", 4: "TILE", 5: "GROUP", 6: "SYMBOL",
    7: "ESCAPE", 8: "LENGTH", 9: "EMAX", 10: "RAWMODE", 11: "PADDING",
}

ZC_COLL_ALLGATHER, ZC_COLL_REDUCE_SCATTER, ZC_COLL_ALLTOALL = 0, 1, 2
COLLECTIVES = {"allgather": ZC_COLL_ALLGATHER, "reduce_scatter": ZC_COLL_REDUCE_SCATTER,
               "alltoall": ZC_COLL_ALLTOALL}


class SwitchParams(ct.Structure):
    _fields_ = [("link_GBps", ct.c_double), ("step_latency_us", ct.c_double),
                ("compress_GBps", ct.c_double), ("decompress_GBps", ct.c_double),
                ("reduce_GBps", ct.c_double)]


class SwitchResult(ct.Structure):
    _fields_ = [("use_compressed", ct.c_int32), ("plain_us", ct.c_double),
                ("compressed_us", ct.c_double), ("breakeven_GBps", ct.c_double)]


_lib = None


class ZcError(RuntimeError):
    def __init__(self, code, what=""):
        super().__init__("%s: %s (%d)" % (what, zc_strerror(code), code))
        self.code = code


def lib():
    """The loaded libzc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libzc.so is not built (run __graft_entry__.build() or "
                "python lossless_bf16_tensor_sign_amd/build.py)")
        L = ct.CDLL(LIB_PATH)
        i64p = ct.POINTER(ct.c_int64)
        L.zc_chunk_bound.argtypes = [ct.c_int64]
        L.zc_chunk_bound.restype = ct.c_size_t
        L.zc_bound.argtypes = [i64p, ct.c_int32]
        L.zc_bound.restype = ct.c_size_t
        L.zc_workspace_bytes.argtypes = [i64p, ct.c_int32]
        L.zc_workspace_bytes.restype = ct.c_size_t
        L.zc_compress.argtypes = [ct.c_void_p, i64p, ct.c_int32, ct.c_void_p,
                                  ct.c_size_t, ct.c_void_p, ct.c_void_p,
                                  ct.c_size_t, ct.c_void_p]
        L.zc_compress.restype = ct.c_int
        L.zc_compress_noalloc.argtypes = [ct.c_void_p, i64p, ct.c_int32, ct.c_void_p,
                                          ct.c_size_t, ct.c_void_p, ct.c_void_p]
        L.zc_compress_noalloc.restype = ct.c_int
        L.zc_decompress.argtypes = [ct.c_void_p, ct.c_size_t, i64p, i64p,
                                    ct.c_int32, ct.c_void_p, ct.c_void_p,
                                    ct.c_void_p]
        L.zc_decompress.restype = ct.c_int
        L.zc_bound_max.argtypes = [ct.c_int64, ct.c_int32]
        L.zc_bound_max.restype = ct.c_size_t
        L.zc_workspace_bytes_max.argtypes = [ct.c_int64, ct.c_int32]
        L.zc_workspace_bytes_max.restype = ct.c_size_t
        L.zc_compress_dev.argtypes = [ct.c_void_p, ct.c_void_p, ct.c_int32, ct.c_int64,
                                      ct.c_void_p, ct.c_size_t, ct.c_void_p, ct.c_void_p,
                                      ct.c_void_p, ct.c_size_t, ct.c_void_p]
        L.zc_compress_dev.restype = ct.c_int
        L.zc_decompress_dev.argtypes = [ct.c_void_p, ct.c_size_t, ct.c_void_p, ct.c_void_p,
                                        ct.c_int32, ct.c_int64, ct.c_void_p, ct.c_void_p,
                                        ct.c_void_p, ct.c_size_t, ct.c_void_p]
        L.zc_decompress_dev.restype = ct.c_int
        L.zc_decompress_reduce.argtypes = [ct.c_void_p, ct.c_size_t, i64p, ct.c_int64,
                                           ct.c_int32, ct.c_void_p, ct.c_void_p, ct.c_void_p,
                                           ct.c_size_t, ct.c_void_p]
        L.zc_decompress_reduce.restype = ct.c_int
        L.zc_reduce_scratch_bytes.argtypes = [ct.c_int64, ct.c_int32]
        L.zc_reduce_scratch_bytes.restype = ct.c_size_t
        L.zc_decompress_reduce_bf16.argtypes = L.zc_decompress_reduce.argtypes
        L.zc_decompress_reduce_bf16.restype = ct.c_int
        L.zc_pipeline.argtypes = [ct.c_void_p, i64p, ct.c_int32, ct.c_int32, ct.c_void_p,
                                  ct.c_void_p, ct.c_size_t, ct.c_void_p, ct.c_void_p,
                                  ct.c_void_p, ct.c_void_p, ct.c_size_t, ct.c_void_p,
                                  ct.c_void_p, ct.c_void_p]
        L.zc_pipeline.restype = ct.c_int
        L.zc_estimate.argtypes = [ct.c_void_p, ct.c_void_p, ct.c_int32, ct.c_int64,
                                  ct.c_int32, ct.c_void_p, ct.c_void_p]
        L.zc_estimate.restype = ct.c_int
        L.zc_switch_decide.argtypes = [ct.c_int32, ct.c_int32, ct.c_double, ct.c_double,
                                       ct.POINTER(SwitchParams), ct.POINTER(SwitchResult)]
        L.zc_switch_decide.restype = ct.c_int
        L.zc_strerror.argtypes = [ct.c_int]
        L.zc_strerror.restype = ct.c_char_p
        L.zc_code_table.argtypes = [ct.c_int32, ct.POINTER(ct.c_int32),
                                    ct.POINTER(ct.c_uint32),
                                    ct.POINTER(ct.c_double)]
        L.zc_code_table.restype = ct.c_int
        _lib = L
    return _lib


def _counts(counts):
    a = np.ascontiguousarray(np.asarray(counts, dtype=np.int64).reshape(-1))
    return a, a.ctypes.data_as(ct.POINTER(ct.c_int64))


def _ptr(t):
    return None if t is None else ct.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ct.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context that makes `stream` current (None: the current stream).

    The allocating wrappers below allocate their buffers and read the status
    word inside it, so the caching allocator ties every buffer to the stream
    the kernels run on (a buffer freed on return is reused only by work
    ordered after them) and the status read is ordered after the decode."""
    import contextlib
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _offsets(in_offsets, num_chunks):
    if in_offsets is None:
        return None, None
    off, op = _counts(in_offsets)
    if len(off) < int(num_chunks):
        raise ValueError("in_offsets has %d entries for %d chunks" % (len(off), num_chunks))
    return off, op


# ----------------------------------------------------------- C entry points

def zc_chunk_bound(n: int) -> int:
    return int(lib().zc_chunk_bound(int(n)))


def zc_bound(counts) -> int:
    a, p = _counts(counts)
    return int(lib().zc_bound(p, len(a)))


def zc_workspace_bytes(counts) -> int:
    a, p = _counts(counts)
    return int(lib().zc_workspace_bytes(p, len(a)))


def zc_bound_max(total_values: int, num_chunks: int) -> int:
    return int(lib().zc_bound_max(int(total_values), int(num_chunks)))


def zc_workspace_bytes_max(total_values: int, num_chunks: int) -> int:
    return int(lib().zc_workspace_bytes_max(int(total_values), int(num_chunks)))


def zc_strerror(code: int) -> str:
    return lib().zc_strerror(int(code)).decode()


def zc_code_table(table_id: int = 1):
    """(lengths, codes, probabilities) of the library's table."""
    ln = (ct.c_int32 * 17)()
    cd = (ct.c_uint32 * 17)()
    pr = (ct.c_double * 17)()
    r = lib().zc_code_table(table_id, ln, cd, pr)
    if r != ZC_OK:
        raise ZcError(r, "zc_code_table")
    return (np.array(list(ln), np.int32), np.array(list(cd), np.uint32),
            np.array(list(pr), np.float64))


def zc_compress(d_in, counts, d_out, d_comp_sizes, d_ws, stream=None,
                out_capacity=None, ws_bytes=None) -> int:
    """Queue compression; tensors are device tensors (uint8 / int64)."""
    a, p = _counts(counts)
    cap = d_out.numel() * d_out.element_size() if out_capacity is None else out_capacity
    wsb = d_ws.numel() * d_ws.element_size() if ws_bytes is None else ws_bytes
    return int(lib().zc_compress(_ptr(d_in), p, len(a), _ptr(d_out), cap,
                                 _ptr(d_comp_sizes), _ptr(d_ws), wsb,
                                 _stream(stream)))


def zc_compress_noalloc(d_in, counts, d_out, d_comp_sizes, stream=None,
                        out_capacity=None) -> int:
    """Queue compression with the library's own per-GPU workspace (no
    workspace argument; nothing is allocated)."""
    a, p = _counts(counts)
    cap = d_out.numel() * d_out.element_size() if out_capacity is None else out_capacity
    return int(lib().zc_compress_noalloc(_ptr(d_in), p, len(a), _ptr(d_out), cap,
                                         _ptr(d_comp_sizes), _stream(stream)))


def zc_decompress(d_in, counts, d_out, d_status, in_offsets=None,
                  stream=None, in_bytes=None) -> int:
    """Queue decompression; d_status (int32 device) must hold 0."""
    a, p = _counts(counts)
    nb = d_in.numel() * d_in.element_size() if in_bytes is None else in_bytes
    off, op = _offsets(in_offsets, len(a))
    return int(lib().zc_decompress(_ptr(d_in), nb, op, p, len(a), _ptr(d_out),
                                   _ptr(d_status), _stream(stream)))


def zc_compress_dev(d_in, d_counts, total_values, d_out, d_comp_sizes, d_slot_off, d_ws,
                    stream=None, out_capacity=None, ws_bytes=None) -> int:
    """Queue compression with the counts in a device int64 tensor."""
    cap = d_out.numel() * d_out.element_size() if out_capacity is None else out_capacity
    wsb = d_ws.numel() * d_ws.element_size() if ws_bytes is None else ws_bytes
    return int(lib().zc_compress_dev(_ptr(d_in), _ptr(d_counts), d_counts.numel(),
                                     int(total_values), _ptr(d_out), cap, _ptr(d_comp_sizes),
                                     _ptr(d_slot_off), _ptr(d_ws), wsb, _stream(stream)))


def zc_decompress_dev(d_in, d_counts, total_values, d_out, d_status, d_ws, d_in_offsets=None,
                      stream=None, in_bytes=None, ws_bytes=None) -> int:
    """Queue decompression with the counts (and offsets) in device tensors."""
    if d_in_offsets is not None and d_in_offsets.numel() < d_counts.numel():
        raise ValueError("d_in_offsets has fewer entries than d_counts")
    nb = d_in.numel() * d_in.element_size() if in_bytes is None else in_bytes
    wsb = d_ws.numel() * d_ws.element_size() if ws_bytes is None else ws_bytes
    return int(lib().zc_decompress_dev(_ptr(d_in), nb, _ptr(d_in_offsets), _ptr(d_counts),
                                       d_counts.numel(), int(total_values), _ptr(d_out),
                                       _ptr(d_status), _ptr(d_ws), wsb, _stream(stream)))


def zc_reduce_scratch_bytes(n, num_chunks) -> int:
    """Scratch bytes zc_decompress_reduce needs (0 for n == 0 or a bad argument)."""
    return int(lib().zc_reduce_scratch_bytes(int(n), int(num_chunks)))


def zc_decompress_reduce(d_in, n, num_chunks, d_out, d_status, d_scratch, in_offsets=None,
                         stream=None, in_bytes=None, scratch_bytes=None, bf16=False) -> int:
    """Queue decode of num_chunks streams of n values and their fp32 sum
    (rounded once to bf16 into a 16-bit d_out when bf16=True)."""
    nb = d_in.numel() * d_in.element_size() if in_bytes is None else in_bytes
    if scratch_bytes is None:
        sb = 0 if d_scratch is None else d_scratch.numel() * d_scratch.element_size()
    else:
        sb = scratch_bytes
    off, op = _offsets(in_offsets, num_chunks)
    fn = lib().zc_decompress_reduce_bf16 if bf16 else lib().zc_decompress_reduce
    return int(fn(_ptr(d_in), nb, op, int(n), int(num_chunks), _ptr(d_out), _ptr(d_status),
                  _ptr(d_scratch), sb, _stream(stream)))


def zc_pipeline(d_in, counts, groups, d_send, d_recv, d_comp_sizes, d_out, d_status, d_ws,
                s_comp=None, s_link=None, s_dec=None, capacity=None, ws_bytes=None) -> int:
    """Queue the chunk-pipelined compress -> link -> decompress exchange."""
    a, p = _counts(counts)
    cap = min(d_send.numel() * d_send.element_size(),
              d_recv.numel() * d_recv.element_size()) if capacity is None else capacity
    wsb = d_ws.numel() * d_ws.element_size() if ws_bytes is None else ws_bytes
    return int(lib().zc_pipeline(_ptr(d_in), p, len(a), int(groups), _ptr(d_send),
                                 _ptr(d_recv), cap, _ptr(d_comp_sizes), _ptr(d_out),
                                 _ptr(d_status), _ptr(d_ws), wsb, _stream(s_comp),
                                 _stream(s_link), _stream(s_dec)))


def zc_estimate(d_in, d_counts, total_values, samples_per_chunk, d_est, stream=None) -> int:
    """Queue the sampled size estimate of each chunk (int64 device tensors)."""
    return int(lib().zc_estimate(_ptr(d_in), _ptr(d_counts), d_counts.numel(),
                                 int(total_values), int(samples_per_chunk), _ptr(d_est),
                                 _stream(stream)))


def zc_switch_decide(collective, ranks, nbytes, comp_bytes, link_GBps, step_latency_us,
                     compress_GBps, decompress_GBps=0.0, reduce_GBps=0.0):
    """Host cost model: returns (status, dict of the result fields)."""
    coll = COLLECTIVES.get(collective, collective)
    p = SwitchParams(float(link_GBps), float(step_latency_us), float(compress_GBps),
                     float(decompress_GBps), float(reduce_GBps))
    r = SwitchResult()
    st = int(lib().zc_switch_decide(int(coll), int(ranks), float(nbytes), float(comp_bytes),
                                    ct.byref(p), ct.byref(r)))
    return st, {"use_compressed": bool(r.use_compressed), "plain_us": r.plain_us,
                "compressed_us": r.compressed_us, "breakeven_GBps": r.breakeven_GBps}


# ------------------------------------------------ allocating conveniences

def _raise_on_status(what, status):
    st = int(status.item())
    if st != 0:
        raise ZcError(ZC_ECORRUPT, "%s: %s in chunk %d"
                      % (what, REASONS.get(st >> 24, st >> 24), st & 0xFFFFFF))


def compress(x, counts, stream=None):
    """Compress a device tensor of bf16 (or its uint16/int16 bits).

    Returns (slot-layout uint8 buffer, int64 device sizes)."""
    import torch
    a, _ = _counts(counts)
    dev = x.device
    with _on(stream):
        out = torch.empty(max(zc_bound(a), 16), dtype=torch.uint8, device=dev)
        sizes = torch.empty(max(len(a), 1), dtype=torch.int64, device=dev)
        ws = torch.zeros(max(zc_workspace_bytes(a), 8), dtype=torch.uint8, device=dev)
        r = zc_compress(x, a, out, sizes, ws, stream=stream)
    if r != ZC_OK:
        raise ZcError(r, "zc_compress")
    return out, sizes[:len(a)]


def decompress(buf, counts, in_offsets=None, stream=None, check=True):
    """Decode streams back to a uint16 device tensor of sum(counts) values."""
    import torch
    a, _ = _counts(counts)
    with _on(stream):
        out = torch.empty(max(int(a.sum()), 1), dtype=torch.int16, device=buf.device)
        status = torch.zeros(1, dtype=torch.int32, device=buf.device)
        r = zc_decompress(buf, a, out, status, in_offsets=in_offsets, stream=stream)
        if r != ZC_OK:
            raise ZcError(r, "zc_decompress")
        out = out[:int(a.sum())]
        if check:
            _raise_on_status("zc_decompress", status)
    return out, status


def compress_dev(x, d_counts, stream=None):
    """Compress with the split in a device int64 tensor (no host copy of it).

    Returns (buffer, int64 device sizes, int64 device slot offsets)."""
    import torch
    dev = x.device
    total, nc = x.numel(), d_counts.numel()
    with _on(stream):
        out = torch.empty(max(zc_bound_max(total, nc), 16), dtype=torch.uint8, device=dev)
        sizes = torch.empty(max(nc, 1), dtype=torch.int64, device=dev)
        slots = torch.empty(max(nc, 1), dtype=torch.int64, device=dev)
        ws = torch.zeros(max(zc_workspace_bytes_max(total, nc), 256), dtype=torch.uint8,
                         device=dev)
        r = zc_compress_dev(x, d_counts, total, out, sizes, slots, ws, stream=stream)
    if r != ZC_OK:
        raise ZcError(r, "zc_compress_dev")
    return out, sizes[:nc], slots[:nc]


def decompress_dev(buf, d_counts, total_values, d_in_offsets=None, stream=None, check=True):
    """Decode with the split (and offsets) in device tensors."""
    import torch
    dev = buf.device
    nc = d_counts.numel()
    with _on(stream):
        out = torch.empty(max(int(total_values), 1), dtype=torch.int16, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        ws = torch.empty(max(zc_workspace_bytes_max(total_values, nc), 256), dtype=torch.uint8,
                         device=dev)
        r = zc_decompress_dev(buf, d_counts, total_values, out, status, ws,
                              d_in_offsets=d_in_offsets, stream=stream)
        if r != ZC_OK:
            raise ZcError(r, "zc_decompress_dev")
        out = out[:int(total_values)]
        if check:
            _raise_on_status("zc_decompress_dev", status)
    return out, status


def decompress_reduce(buf, n, num_chunks, in_offsets=None, stream=None, check=True, bf16=False):
    """Decode num_chunks streams of n values each and sum them in fp32.

    Returns (device tensor of n sums: float32, or int16 bf16 bit patterns
    when bf16=True; int32 device status)."""
    import torch
    dev = buf.device
    with _on(stream):
        out = torch.empty(max(int(n), 8), dtype=torch.int16 if bf16 else torch.float32,
                          device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        need = zc_reduce_scratch_bytes(n, num_chunks)
        scratch = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        r = zc_decompress_reduce(buf, n, num_chunks, out, status, scratch,
                                 in_offsets=in_offsets, stream=stream, bf16=bf16)
        if r != ZC_OK:
            raise ZcError(r, "zc_decompress_reduce")
        out = out[:int(n)]
        if check:
            _raise_on_status("zc_decompress_reduce", status)
    return out, status


def estimate(x, d_counts, samples_per_chunk=8, stream=None):
    """Estimated stream bytes per chunk (int64 device tensor)."""
    import torch
    with _on(stream):
        est = torch.empty(max(d_counts.numel(), 1), dtype=torch.int64, device=x.device)
        r = zc_estimate(x, d_counts, x.numel(), samples_per_chunk, est, stream=stream)
    if r != ZC_OK:
        raise ZcError(r, "zc_estimate")
    return est[:d_counts.numel()]


def pipeline(x, counts, groups, streams=None, check=True):
    """Chunk-pipelined exchange of int16/uint16 device tensor x: returns
    (y, status, send, recv, sizes) with y the decoded values.  streams =
    (compress, link, decompress) torch streams, default all current."""
    import torch
    a = np.asarray(counts, np.int64)
    cap = zc_bound(a)
    send = torch.empty(max(cap, 16), dtype=torch.uint8, device=x.device)
    recv = torch.zeros(max(cap, 16), dtype=torch.uint8, device=x.device)
    sizes = torch.empty(max(len(a), 1), dtype=torch.int64, device=x.device)
    ws = torch.zeros(max(zc_workspace_bytes(a), 16), dtype=torch.uint8, device=x.device)
    y = torch.empty(int(a.sum()), dtype=x.dtype, device=x.device)
    status = torch.zeros(1, dtype=torch.int32, device=x.device)
    sc, sl, sd = (None, None, None) if streams is None else streams
    cur = torch.cuda.current_stream()
    for s_ in (sc, sl, sd):      # the buffers above were written on cur
        if s_ is not None:
            s_.wait_stream(cur)
    r = zc_pipeline(x, a, groups, send, recv, sizes, y, status, ws, s_comp=sc, s_link=sl,
                    s_dec=sd)
    # the buffers were allocated on cur but are used on the three streams:
    # keep the allocator from reusing them (ws in particular, which is freed
    # on return) before the work queued there has run
    for s_, bufs in ((sc, (x, send, sizes, ws)), (sl, (send, recv, sizes)),
                     (sd, (recv, y, status))):
        if s_ is not None:
            for b in bufs:
                b.record_stream(s_)
    if r != ZC_OK:
        raise ZcError(r, "zc_pipeline")
    if check:
        cur.wait_stream(cur if sd is None else sd)
        st = int(status.item())
        if st != 0:
            raise ZcError(ZC_ECORRUPT, "zc_pipeline: status %#x" % st)
    return y, status, send, recv, sizes
