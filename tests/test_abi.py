"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/zc.h declares, and its host-only functions (sizes, code table,
argument validation) agree with the oracle."""
import os
import re
import subprocess

import numpy as np
import pytest

from lossless_bf16_tensor_sign_amd import zc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "zc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(zc_\w+)\s*\(",
                                 src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"zc_compress", "zc_decompress", "zc_bound", "zc_chunk_bound",
            "zc_workspace_bytes", "zc_strerror", "zc_code_table"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", zc.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = zc.lib()
    for n in names:
        assert hasattr(lib, n)


def test_bounds_match_oracle(oracle):
    for n in [0, 1, 7, 8, 511, 8191, 8192, 8193, 1 << 20, 1 << 22, 29_417_472,
              (1 << 31) - 1]:
        assert zc.zc_chunk_bound(n) == oracle.chunk_bound(n), n
    assert zc.zc_chunk_bound(-1) == 0
    rng = np.random.default_rng(0)
    for _ in range(20):
        cnt = rng.integers(0, 50000, size=int(rng.integers(1, 200)))
        cnt[rng.random(cnt.size) < 0.2] = 0
        assert zc.zc_bound(cnt) == oracle.slot_offsets(cnt)[1]
    assert zc.zc_bound([5, -1]) == 0


def test_workspace_bytes():
    # a fixed header (launch tag and completion counters), then one status slot per
    # tile of the largest launch (at most 64 chunks per launch)
    one = zc.zc_workspace_bytes([0])          # header + 1 slot
    three = zc.zc_workspace_bytes([8193, 1])  # header + 3 slots
    slot = (three - one) // 2
    assert three - one == 2 * slot and slot >= 8 and slot % 8 == 0
    head = one - slot
    assert head >= 64 * 4
    cnt = [8192] * 64 + [3 * 8192]
    assert zc.zc_workspace_bytes(cnt) == head + slot * 64
    assert zc.zc_workspace_bytes([8192 * 5] * 2) == head + slot * 10


def test_reduce_scratch_bytes():
    # one slab holds the whole shard: every contribution at its length
    # rounded up to 8 values, one buffer
    assert zc.zc_reduce_scratch_bytes(4096, 4) == 2 * 4096 * 4
    assert zc.zc_reduce_scratch_bytes(20003, 8) == 2 * 20008 * 8
    assert zc.zc_reduce_scratch_bytes(1, 5) == 2 * 8 * 5
    # 8 to 64 streams of at least 512 tiles, in generations of 512 tile
    # positions at least 27/32 full, are decoded and summed in one kernel
    # with nothing staged
    tiles512 = 512 * 8192
    for n, c in [(tiles512, 8), (tiles512 - 8191, 64), (1 << 22, 64), (1 << 26, 13),
                 ((1 << 31) - 1, 64), (864 * 8192, 64), (1408 * 8192 - 5, 8)]:
        assert zc.zc_reduce_scratch_bytes(n, c) == 0, (n, c)
    # otherwise slabs of whole 8192-value tiles per stream, about 128 MiB
    # over all streams: two slab buffers for at most 64 streams, one for more
    slab = 128 << 20
    for n, c in [(tiles512 - 8192, 64), ((1 << 21) + 77, 64), (1 << 25, 3), (1 << 27, 1),
                 (1 << 22, 7), (1 << 22, 65), (1 << 22, 4096), (600 * 8192, 64),
                 (863 * 8192, 64), (1152 * 8192, 16)]:
        b = zc.zc_reduce_scratch_bytes(n, c)
        bufs = 2 if c <= 64 else 1
        per = b // (2 * c * bufs)
        assert b == 2 * c * per * bufs and per % 8192 == 0 and 8192 <= per < n, (n, c)
        assert per * 2 * c <= max(slab, 2 * c * 8192), (n, c)
    assert zc.zc_reduce_scratch_bytes(1 << 21, 64) == 2 * slab
    assert zc.zc_reduce_scratch_bytes(0, 4) == 0
    assert zc.zc_reduce_scratch_bytes(-1, 4) == 0
    assert zc.zc_reduce_scratch_bytes(10, -1) == 0


def test_code_table_matches_oracle(oracle):
    L, C, P = zc.zc_code_table(1)
    p, l, c = oracle.table(1)
    assert np.array_equal(L, l) and np.array_equal(C, c)
    assert np.allclose(P, p, rtol=1e-12, atol=0)
    with pytest.raises(zc.ZcError):
        zc.zc_code_table(2)


def test_argument_errors_before_any_gpu_work():
    lib = zc.lib()
    import ctypes as ct
    cnt = np.array([10, -1], np.int64)
    p = cnt.ctypes.data_as(ct.POINTER(ct.c_int64))
    assert lib.zc_compress(None, p, 2, None, 0, None, None, 0, None) == zc.ZC_EINVAL
    assert lib.zc_decompress(None, 0, None, p, 2, None, None, None) == zc.ZC_EINVAL
    assert lib.zc_compress(None, p, 0, None, 0, None, None, 0, None) == zc.ZC_OK
    cnt = np.array([10], np.int64)
    p = cnt.ctypes.data_as(ct.POINTER(ct.c_int64))
    # misaligned output pointer
    assert lib.zc_compress(ct.c_void_p(0x1000), p, 1, ct.c_void_p(0x2001), 1 << 20,
                           ct.c_void_p(0x3000), ct.c_void_p(0x4000), 1 << 20,
                           None) == zc.ZC_EINVAL
    # capacity too small
    assert lib.zc_compress(ct.c_void_p(0x1000), p, 1, ct.c_void_p(0x2000), 10,
                           ct.c_void_p(0x3000), ct.c_void_p(0x4000), 1 << 20,
                           None) == zc.ZC_ENOSPC
    # workspace too small
    assert lib.zc_compress(ct.c_void_p(0x1000), p, 1, ct.c_void_p(0x2000), 1 << 20,
                           ct.c_void_p(0x3000), ct.c_void_p(0x4000), 8,
                           None) == zc.ZC_ENOSPC
    # decompress: offset not a multiple of 16, header beyond in_bytes
    off = np.array([8], np.int64)
    op = off.ctypes.data_as(ct.POINTER(ct.c_int64))
    assert lib.zc_decompress(ct.c_void_p(0x1000), 4096, op, p, 1, ct.c_void_p(0x2000),
                             ct.c_void_p(0x3000), None) == zc.ZC_EINVAL
    assert lib.zc_decompress(ct.c_void_p(0x1000), 16, None, p, 1, ct.c_void_p(0x2000),
                             ct.c_void_p(0x3000), None) == zc.ZC_EINVAL
    for code in (0, -1, -2, -3, -4):
        assert zc.zc_strerror(code) != "unknown status"


def _splits(rng):
    """Splits of one total into C chunks, including the extreme ones."""
    for _ in range(30):
        c = int(rng.integers(1, 200))
        cnt = rng.integers(0, 60000, size=c)
        cnt[rng.random(c) < 0.3] = 0
        yield cnt
    yield np.array([0] * 64)
    yield np.array([1] * 200)
    yield np.array([8193] * 70)
    yield np.array([(1 << 22) * 3 + 5] + [0] * 63)
    yield np.array([8192] * 64)


def test_bound_max_covers_every_split(oracle):
    rng = np.random.default_rng(5)
    for cnt in _splits(rng):
        total, c = int(cnt.sum()), len(cnt)
        assert zc.zc_bound_max(total, c) >= oracle.slot_offsets(cnt)[1], cnt
        # the tiles of any launch (64 chunks) stay within floor(total / 8192) + 64
        for c0 in range(0, c, 64):
            part = cnt[c0:c0 + 64]
            items = int(np.maximum(1, (part + 8191) // 8192).sum())
            assert items <= total // 8192 + len(part)
        assert zc.zc_workspace_bytes_max(total, c) >= zc.zc_workspace_bytes(cnt)
    assert zc.zc_bound_max(0, 0) == 0
    assert zc.zc_bound_max(5, 0) == 0
    assert zc.zc_bound_max(-1, 3) == 0
    assert zc.zc_workspace_bytes_max(10, -1) == 0


def test_device_split_argument_errors_before_any_gpu_work():
    lib = zc.lib()
    import ctypes as ct
    V = ct.c_void_p
    big = 1 << 30
    # values without chunks, negative totals, null pointers
    assert lib.zc_compress_dev(V(0x1000), V(0x2000), 0, 10, V(0x3000), big, V(0x4000),
                               V(0x5000), V(0x6000), big, None) == zc.ZC_EINVAL
    assert lib.zc_compress_dev(V(0x1000), V(0x2000), 2, -1, V(0x3000), big, V(0x4000),
                               V(0x5000), V(0x6000), big, None) == zc.ZC_EINVAL
    assert lib.zc_compress_dev(V(0x1000), None, 2, 10, V(0x3000), big, V(0x4000),
                               V(0x5000), V(0x6000), big, None) == zc.ZC_EINVAL
    # misaligned workspace (256 bytes) and counts (8 bytes)
    assert lib.zc_compress_dev(V(0x1000), V(0x2000), 2, 10, V(0x3000), big, V(0x4000),
                               V(0x5000), V(0x6010), big, None) == zc.ZC_EINVAL
    assert lib.zc_compress_dev(V(0x1000), V(0x2004), 2, 10, V(0x3000), big, V(0x4000),
                               V(0x5000), V(0x6000), big, None) == zc.ZC_EINVAL
    # capacity and workspace below the bounds for that total
    assert lib.zc_compress_dev(V(0x1000), V(0x2000), 2, 10, V(0x3000),
                               zc.zc_bound_max(10, 2) - 1, V(0x4000), V(0x5000), V(0x6000),
                               big, None) == zc.ZC_ENOSPC
    assert lib.zc_compress_dev(V(0x1000), V(0x2000), 2, 10, V(0x3000), big, V(0x4000),
                               V(0x5000), V(0x6000), zc.zc_workspace_bytes_max(10, 2) - 1,
                               None) == zc.ZC_ENOSPC
    assert lib.zc_decompress_dev(V(0x1000), 4096, None, V(0x2000), 2, 10, V(0x3000),
                                 V(0x4000), V(0x5000), 8, None) == zc.ZC_ENOSPC
    assert lib.zc_decompress_dev(V(0x1008), 4096, None, V(0x2000), 2, 10, V(0x3000),
                                 V(0x4000), V(0x5000), big, None) == zc.ZC_EINVAL
    assert lib.zc_compress_dev(None, None, 0, 0, None, 0, None, None, None, 0,
                               None) == zc.ZC_OK


def test_estimate_argument_errors_before_any_gpu_work():
    lib = zc.lib()
    import ctypes as ct
    V = ct.c_void_p
    assert lib.zc_estimate(V(0x1000), V(0x2000), 2, 10, 0, V(0x3000), None) == zc.ZC_EINVAL
    assert lib.zc_estimate(V(0x1000), V(0x2000), -1, 10, 4, V(0x3000), None) == zc.ZC_EINVAL
    assert lib.zc_estimate(V(0x1000), V(0x2000), 2, -1, 4, V(0x3000), None) == zc.ZC_EINVAL
    assert lib.zc_estimate(V(0x1000), None, 2, 10, 4, V(0x3000), None) == zc.ZC_EINVAL
    assert lib.zc_estimate(V(0x1000), V(0x2000), 2, 10, 4, None, None) == zc.ZC_EINVAL
    assert lib.zc_estimate(None, V(0x2000), 2, 10, 4, V(0x3000), None) == zc.ZC_EINVAL
    assert lib.zc_estimate(None, None, 0, 5, 4, None, None) == zc.ZC_EINVAL
    assert lib.zc_estimate(None, None, 0, 0, 4, None, None) == zc.ZC_OK


def test_pipeline_argument_errors_before_any_gpu_work():
    lib = zc.lib()
    import ctypes as ct
    import numpy as np
    V = ct.c_void_p
    big = 1 << 30
    counts = np.array([100, 9000, 0], np.int64)
    cp = counts.ctypes.data_as(ct.POINTER(ct.c_int64))
    ws = zc.zc_workspace_bytes(counts)
    cap = zc.zc_bound(counts)

    def call(d_in=V(0x1000), groups=2, send=V(0x2000), recv=V(0x3000), capacity=big,
             sizes=V(0x4000), out=V(0x5000), status=V(0x6000), d_ws=V(0x7000), ws_bytes=big,
             num_chunks=3):
        return lib.zc_pipeline(d_in, cp, num_chunks, groups, send, recv, capacity, sizes, out,
                               status, d_ws, ws_bytes, None, None, None)
    # groups outside 1..num_chunks
    assert call(groups=0) == zc.ZC_EINVAL
    assert call(groups=4) == zc.ZC_EINVAL
    assert call(groups=-1) == zc.ZC_EINVAL
    # null buffers
    for kw in ("send", "recv", "sizes", "status", "d_ws", "d_in", "out"):
        assert call(**{kw: None}) == zc.ZC_EINVAL, kw
    # misaligned send / receive slots (16 bytes), values (2 bytes), sizes (8 bytes)
    assert call(send=V(0x2008)) == zc.ZC_EINVAL
    assert call(recv=V(0x3004)) == zc.ZC_EINVAL
    assert call(d_in=V(0x1001)) == zc.ZC_EINVAL
    assert call(out=V(0x5001)) == zc.ZC_EINVAL
    assert call(sizes=V(0x4004)) == zc.ZC_EINVAL
    # capacity and workspace one byte short
    assert call(capacity=cap - 1) == zc.ZC_ENOSPC
    assert call(ws_bytes=ws - 1) == zc.ZC_ENOSPC
    # no chunks: nothing to do
    assert call(num_chunks=0, groups=1) == zc.ZC_OK


def test_chunk_count_limit():
    # a decoder failure names its chunk in 24 bits: more chunks are refused
    lib = zc.lib()
    import ctypes as ct
    cnt = np.zeros(4, np.int64)
    p = cnt.ctypes.data_as(ct.POINTER(ct.c_int64))
    assert lib.zc_bound(p, (1 << 24) + 1) == 0          # rejected before counts are read
    assert lib.zc_workspace_bytes(p, (1 << 24) + 1) == 0
    assert lib.zc_compress(None, p, (1 << 24) + 1, None, 0, None, None, 0, None) == zc.ZC_EINVAL
    assert lib.zc_decompress(None, 0, None, p, (1 << 24) + 1, None, None, None) == zc.ZC_EINVAL
    assert zc.zc_bound_max(10, (1 << 24) + 1) == 0
    assert zc.zc_bound(cnt) > 0


def test_binding_checks_offsets_length():
    # the binding refuses an offsets array shorter than the counts before
    # calling the library (which would read past it)
    import torch
    d = torch.zeros(64, dtype=torch.uint8)
    out = torch.zeros(8, dtype=torch.int16)
    st = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError):
        zc.zc_decompress(d, [1, 1, 1], out, st, in_offsets=[0, 16])
