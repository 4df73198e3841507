"""The oracle over many chunks at once, in a thread pool.

Chunks are independent, and the oracle's C calls release the GIL (ctypes),
so a pool of threads runs them in parallel.  Used by the GPU tests to compare
every chunk of the full-size workloads with the oracle.  The pool size is the
host share of one GPU (16 threads), or fewer where the host has fewer cores.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

WORKERS = max(1, min(16, os.cpu_count() or 1))


def value_offsets(counts):
    return np.concatenate([[0], np.cumsum(np.asarray(counts, np.int64))])


def map_chunks(fn, num_chunks, workers=WORKERS):
    """[fn(c) for c in range(num_chunks)], evaluated in a thread pool."""
    if num_chunks <= 1 or workers <= 1:
        return [fn(c) for c in range(num_chunks)]
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, range(num_chunks)))


def compress_chunks(oracle, w, counts, workers=WORKERS):
    """The oracle's stream of every chunk (a list of uint8 arrays)."""
    vo = value_offsets(counts)
    return map_chunks(lambda c: oracle.compress_chunk(w[vo[c]:vo[c + 1]]), len(counts),
                      workers)


def compare_chunks(oracle, w, counts, gbuf, gsizes, offsets, label="", workers=WORKERS):
    """Every chunk c: the GPU stream at offsets[c] (gsizes[c] bytes of gbuf)
    equals the oracle's stream byte for byte, and the oracle decodes it back
    to the input.  Raises AssertionError naming the first bad chunk."""
    vo = value_offsets(counts)

    def one(c):
        x = w[vo[c]:vo[c + 1]]
        ref = oracle.compress_chunk(x)
        if int(gsizes[c]) != ref.size:
            return "%s chunk %d: size %d, oracle %d" % (label, c, int(gsizes[c]), ref.size)
        got = gbuf[offsets[c]:offsets[c] + ref.size]
        bad = np.nonzero(got != ref)[0]
        if bad.size:
            return "%s chunk %d: first differing byte %d of %d" % (label, c, bad[0], ref.size)
        r, back = oracle.decompress_chunk(got, x.size)
        if r != 0 or not np.array_equal(back, x):
            return "%s chunk %d: oracle does not decode the GPU stream (%d)" % (label, c, r)
        return None

    errors = [e for e in map_chunks(one, len(counts), workers) if e]
    assert not errors, errors[:3]
