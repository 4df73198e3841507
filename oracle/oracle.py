"""ctypes wrapper around the C oracle (``zc_oracle.c``).

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and bench.py's CPU-baseline
leg import this module.  The product library never does.

The oracle is plain single-threaded C; this module only marshals numpy
buffers.  ``build()`` compiles ``libzc_oracle.so`` next to this file with gcc.
"""
from __future__ import annotations

import ctypes as ct
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zc_oracle.c")
LIB = os.path.join(HERE, "libzc_oracle.so")

ERRORS = {
    -1: "EINVAL", -2: "ENOSPC", -10: "E_HEADER", -11: "E_SIZE", -12: "E_GAP",
    -13: "E_TILE", -14: "E_GROUP", -15: "E_SYMBOL", -16: "E_ESCAPE",
    -17: "E_LENGTH", -18: "E_EMAX", -19: "E_RAWMODE", -20: "E_PADDING",
}

NSYM = 17
ESC = 16


def build(force: bool = True) -> str:
    """Compile the oracle (plain C, -O2, no vector intrinsics)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
             "-o", tmp, SRC, "-lm"],
            check=True)
        os.replace(tmp, LIB)
    return LIB


class _Stats(ct.Structure):
    _fields_ = [("raw_groups", ct.c_int64), ("escapes", ct.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ct.CDLL(LIB)
        i64p = ct.POINTER(ct.c_int64)
        dp = ct.POINTER(ct.c_double)
        ip = ct.POINTER(ct.c_int)
        u32p = ct.POINTER(ct.c_uint32)
        L.zco_law_fixed_sigma.argtypes = [ct.c_int, ct.c_int, ct.c_double, dp]
        L.zco_law_phase_avg.argtypes = [ct.c_int, ct.c_int, ct.c_int, dp]
        L.zco_huffman_lengths.argtypes = [dp, ct.c_int, ip]
        L.zco_canonical_codes.argtypes = [ip, ct.c_int, u32p]
        L.zco_build_table.argtypes = [ct.c_int, dp, ip, u32p]
        L.zco_geometry.argtypes = [ct.c_int64, i64p, i64p, i64p, i64p]
        L.zco_chunk_bound.argtypes = [ct.c_int64]
        L.zco_chunk_bound.restype = ct.c_int64
        L.zco_slot_offsets.argtypes = [i64p, ct.c_int, i64p]
        L.zco_slot_offsets.restype = ct.c_int64
        L.zco_compress_chunk.argtypes = [ct.c_void_p, ct.c_int64, ct.c_void_p,
                                         ct.c_int64, ct.POINTER(_Stats)]
        L.zco_compress_chunk.restype = ct.c_int64
        L.zco_decompress_chunk.argtypes = [ct.c_void_p, ct.c_int64,
                                           ct.c_int64, ct.c_void_p]
        L.zco_compress.argtypes = [ct.c_void_p, i64p, ct.c_int, ct.c_void_p,
                                   ct.c_int64, i64p, ct.POINTER(_Stats)]
        L.zco_reduce_bf16_f32.argtypes = [ct.c_void_p, ct.c_int64, ct.c_int, ct.c_void_p]
        L.zco_reduce_bf16_f32.restype = None
        L.zco_reduce_bf16_bf16.argtypes = [ct.c_void_p, ct.c_int64, ct.c_int, ct.c_void_p]
        L.zco_reduce_bf16_bf16.restype = None
        L.zco_f32_to_bf16.argtypes = [ct.c_float]
        L.zco_f32_to_bf16.restype = ct.c_uint16
        L.zco_decompress.argtypes = [ct.c_void_p, ct.c_int64, i64p, i64p,
                                     ct.c_int, ct.c_void_p, ip]
        _lib = L
    return _lib


def _i64(a):
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a, a.ctypes.data_as(ct.POINTER(ct.c_int64))


# ---------------------------------------------------------------- table ---

def law_fixed_sigma(sigma: float, G: int = 128, K: int = 16) -> np.ndarray:
    out = np.zeros(K + 1, np.float64)
    lib().zco_law_fixed_sigma(G, K, sigma,
                              out.ctypes.data_as(ct.POINTER(ct.c_double)))
    return out


def law_phase_avg(G: int = 128, K: int = 16, Q: int = 64) -> np.ndarray:
    out = np.zeros(K + 1, np.float64)
    lib().zco_law_phase_avg(G, K, Q, out.ctypes.data_as(ct.POINTER(ct.c_double)))
    return out


def huffman_lengths(w) -> np.ndarray:
    w = np.ascontiguousarray(w, np.float64)
    out = np.zeros(len(w), np.int32)
    r = lib().zco_huffman_lengths(w.ctypes.data_as(ct.POINTER(ct.c_double)),
                                  len(w), out.ctypes.data_as(ct.POINTER(ct.c_int)))
    assert r == 0
    return out


def canonical_codes(lengths) -> np.ndarray:
    lengths = np.ascontiguousarray(lengths, np.int32)
    out = np.zeros(len(lengths), np.uint32)
    lib().zco_canonical_codes(lengths.ctypes.data_as(ct.POINTER(ct.c_int)),
                              len(lengths),
                              out.ctypes.data_as(ct.POINTER(ct.c_uint32)))
    return out


def table(table_id: int = 1):
    """(probabilities, lengths, codes) of the oracle's own table."""
    p = np.zeros(NSYM, np.float64)
    L = np.zeros(NSYM, np.int32)
    c = np.zeros(NSYM, np.uint32)
    r = lib().zco_build_table(table_id, p.ctypes.data_as(ct.POINTER(ct.c_double)),
                              L.ctypes.data_as(ct.POINTER(ct.c_int)),
                              c.ctypes.data_as(ct.POINTER(ct.c_uint32)))
    if r != 0:
        raise ValueError("unknown table_id %d" % table_id)
    return p, L, c


# ------------------------------------------------------------- geometry ---

def geometry(n: int):
    vals = [ct.c_int64() for _ in range(4)]
    lib().zco_geometry(n, *[ct.byref(v) for v in vals])
    return tuple(v.value for v in vals)   # T, NG, R, X


def chunk_bound(n: int) -> int:
    return lib().zco_chunk_bound(n)


def slot_offsets(counts):
    counts, cp = _i64(counts)
    off = np.zeros(len(counts), np.int64)
    total = lib().zco_slot_offsets(cp, len(counts),
                                   off.ctypes.data_as(ct.POINTER(ct.c_int64)))
    return off, total


# ---------------------------------------------------------------- codec ---

def compress_chunk(w: np.ndarray, stats: bool = False):
    """Compress one chunk of bf16 bit patterns (uint16).  Returns bytes."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    n = w.size
    cap = chunk_bound(n)
    out = np.zeros(cap, np.uint8)
    st = _Stats()
    r = lib().zco_compress_chunk(w.ctypes.data, n, out.ctypes.data, cap,
                                 ct.byref(st))
    if r < 0:
        raise RuntimeError("oracle compress failed: %s" % ERRORS.get(r, r))
    if stats:
        return out[:r].copy(), {"raw_groups": st.raw_groups,
                                "escapes": st.escapes}
    return out[:r].copy()


def decompress_chunk(stream, n: int, strict_errors: bool = True):
    """Decode one chunk stream.  Returns (status, uint16 array)."""
    stream = np.ascontiguousarray(np.frombuffer(bytes(stream), np.uint8)
                                  if not isinstance(stream, np.ndarray)
                                  else stream, dtype=np.uint8)
    out = np.zeros(max(n, 1), np.uint16)
    r = lib().zco_decompress_chunk(stream.ctypes.data, stream.size, n,
                                   out.ctypes.data)
    return r, out[:n]


def compress(w: np.ndarray, counts):
    """Slot-layout compression of a whole buffer.  Returns (buf, sizes, stats)."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    counts, cp = _i64(counts)
    assert int(counts.sum()) == w.size
    _, total = slot_offsets(counts)
    out = np.zeros(max(total, 1), np.uint8)
    sizes = np.zeros(len(counts), np.int64)
    st = _Stats()
    r = lib().zco_compress(w.ctypes.data if w.size else None, cp, len(counts),
                           out.ctypes.data, total,
                           sizes.ctypes.data_as(ct.POINTER(ct.c_int64)),
                           ct.byref(st))
    if r != 0:
        raise RuntimeError("oracle compress failed: %s" % ERRORS.get(r, r))
    return out[:total], sizes, {"raw_groups": st.raw_groups,
                                "escapes": st.escapes}


def decompress(buf: np.ndarray, counts, offsets=None):
    """Decode a whole buffer.  Returns (status, bad_chunk, uint16 array)."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    counts, cp = _i64(counts)
    out = np.zeros(max(int(counts.sum()), 1), np.uint16)
    bad = ct.c_int(-1)
    if offsets is not None:
        offsets, op = _i64(offsets)
    else:
        op = None
    r = lib().zco_decompress(buf.ctypes.data, buf.size, op, cp, len(counts),
                             out.ctypes.data, ct.byref(bad))
    return r, bad.value, out[:int(counts.sum())]


def reduce_bf16_f32(x: np.ndarray, n: int, num_chunks: int) -> np.ndarray:
    """Chunk-order fp32 sums of num_chunks contributions of n bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert x.size == n * num_chunks
    out = np.empty(n, np.float32)
    lib().zco_reduce_bf16_f32(x.ctypes.data, n, num_chunks, out.ctypes.data)
    return out


def f32_to_bf16(x) -> np.ndarray:
    """fp32 values to bf16 bit patterns, to nearest with ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    f = lib().zco_f32_to_bf16
    return np.array([f(float(v)) for v in x], np.uint16)


def reduce_bf16_bf16(x: np.ndarray, n: int, num_chunks: int) -> np.ndarray:
    """Chunk-order fp32 sums rounded once to bf16 (uint16 bit patterns)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert x.size == n * num_chunks
    out = np.empty(n, np.uint16)
    lib().zco_reduce_bf16_bf16(x.ctypes.data, n, num_chunks, out.ctypes.data)
    return out
