"""GPU parity of the reduce-scatter receive step (decode, then ordered sum).

zc_decompress_reduce decodes num_chunks compressed contributions of n bf16
values and sums them element by element in fp32, in chunk order, from +0.
The bar is bit-exactness against the oracle's chunk-order sum (NaN results
compared as NaN, since their sign and payload are unspecified).  At full size
every position is compared with the oracle, and also with a chunk-order sum
written as plain PyTorch fp32 additions.
"""
import sys

import numpy as np
import pytest
import torch

from lossless_bf16_tensor_sign_amd import synth, zc

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def to_dev(w):
    return torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(DEV)


def same_f32(got, want):
    """Bit-equal, except that NaN only has to meet NaN."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), "NaN positions differ, first %d" % np.nonzero(gn != wn)[0][0]
    gb, wb = got.view(np.uint32), want.view(np.uint32)
    bad = np.nonzero((gb != wb) & ~wn)[0]
    assert bad.size == 0, "first differing sum at %d: %#x vs %#x" % (
        bad[0], gb[bad[0]], wb[bad[0]])


def gpu_reduce(w, n, c):
    buf, sizes = zc.compress(to_dev(w), [n] * c)
    out, status = zc.decompress_reduce(buf, n, c, check=False)
    torch.cuda.synchronize()
    return int(status.item()), out.cpu().numpy()


def special_mix(size, seed):
    """Random bf16 patterns with zeros of both signs, subnormals, Inf and NaN."""
    rng = np.random.default_rng(seed)
    w = synth.gaussian_bits(size, 0.02, seed)
    pick = rng.random(size)
    w[pick < 0.02] = rng.integers(0, 1 << 16, int((pick < 0.02).sum()), dtype=np.uint16)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC0, 0x7F7F,
                         0xFF7F, 0x0080], np.uint16)
    m = (pick >= 0.02) & (pick < 0.03)
    w[m] = specials[rng.integers(0, specials.size, int(m.sum()))]
    return w


@pytest.mark.parametrize("n,c", [(20000, 8), (20003, 8), (24576, 11), (8192, 1),
                                 (1, 5), (7, 3), (65536 + 40, 17)])
def test_reduce_matches_oracle(oracle, n, c):
    w = special_mix(n * c, 1000 + n + c)
    say("reduce n=%d chunks=%d" % (n, c))
    st, got = gpu_reduce(w, n, c)
    assert st == 0, "status %#x" % st
    same_f32(got, oracle.reduce_bf16_f32(w, n, c))


def test_reduce_addition_order_is_chunk_order(oracle):
    # 2^24 + 1 rounds back to 2^24 in fp32, so the sum in chunk order is 0
    # while any order that adds the 1 last gives 1.
    n = 1024
    w = np.concatenate([np.full(n, 0x4B80, np.uint16), np.full(n, 0x3F80, np.uint16),
                        np.full(n, 0xCB80, np.uint16)])
    say("reduce order pin")
    st, got = gpu_reduce(w, n, 3)
    assert st == 0
    want = oracle.reduce_bf16_f32(w, n, 3)
    assert np.all(want == 0.0) and not np.signbit(want).any()
    same_f32(got, want)


def test_reduce_of_negative_zeros_is_positive_zero(oracle):
    n = 4096
    w = np.full(n * 4, 0x8000, np.uint16)
    st, got = gpu_reduce(w, n, 4)
    assert st == 0
    assert np.all(got.view(np.uint32) == 0)


def test_reduce_zero_chunks_writes_zeros():
    n = 1000
    out = torch.full((n,), 7.0, dtype=torch.float32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    scratch = torch.empty(16, dtype=torch.uint8, device=DEV)
    dummy = torch.empty(16, dtype=torch.uint8, device=DEV)
    r = zc.zc_decompress_reduce(dummy, n, 0, out, status, scratch)
    assert r == zc.ZC_OK
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.all(out.view(torch.int32) == 0)


def test_reduce_argument_errors():
    n, c = 4096, 4
    w = synth.gaussian_bits(n * c, 0.02, 5)
    buf, _ = zc.compress(to_dev(w), [n] * c)
    out = torch.empty(n + 4, dtype=torch.float32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    need = zc.zc_reduce_scratch_bytes(n, c)
    assert need == 2 * n * c                 # one slab holds this shard
    scratch = torch.empty(need, dtype=torch.uint8, device=DEV)
    assert zc.zc_decompress_reduce(buf, n, c, out, status, scratch,
                                   scratch_bytes=need - 1) == zc.ZC_ENOSPC
    assert zc.zc_decompress_reduce(buf, n, c, out[1:], status, scratch) == zc.ZC_EINVAL
    assert zc.zc_decompress_reduce(buf, -1, c, out, status, scratch) == zc.ZC_EINVAL
    assert zc.zc_decompress_reduce(buf, n, -1, out, status, scratch) == zc.ZC_EINVAL
    torch.cuda.synchronize()
    assert int(status.item()) == 0


def test_reduce_reports_corrupt_stream(oracle):
    n, c = 20000, 4
    w = synth.gaussian_bits(n * c, 0.02, 6)
    buf, sizes = zc.compress(to_dev(w), [n] * c)
    torch.cuda.synchronize()
    hb = buf.cpu().numpy().copy()
    off, _ = oracle.slot_offsets([n] * c)
    hb[off[2]] ^= 0xFF                      # magic of stream 2
    out, status = zc.decompress_reduce(torch.from_numpy(hb).to(DEV), n, c, check=False)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st >> 24 == 1 and (st & 0xFFFFFF) == 2, hex(st)


def test_reduce_ragged_slabs(oracle):
    # 64 streams of a shard longer than one slab (1 Mi values per stream at
    # 64 streams), ending in a partial tile: two slabs, the second ragged,
    # decoded and summed in alternating slab buffers
    c = 64
    n = (1 << 20) + 3 * 8192 + 77
    assert zc.zc_reduce_scratch_bytes(n, c) == 2 * 2 * c * (1 << 20)
    w = special_mix(n * c, 77)
    say("reduce ragged slabs n=%d chunks=%d" % (n, c))
    st, got = gpu_reduce(w, n, c)
    assert st == 0, "status %#x" % st
    same_f32(got, oracle.reduce_bf16_f32(w, n, c))


def test_reduce_more_than_64_streams_in_slabs(oracle):
    # 65 streams: each slab is decoded in two launches (64 + 1 streams),
    # then summed; two slabs, the second ragged
    c = 65
    n = 126 * 8192 + 3 * 8192 + 5
    assert zc.zc_reduce_scratch_bytes(n, c) == 2 * c * 126 * 8192
    w = special_mix(n * c, 78)
    say("reduce 65 streams in slabs n=%d" % n)
    st, got = gpu_reduce(w, n, c)
    assert st == 0, "status %#x" % st
    same_f32(got, oracle.reduce_bf16_f32(w, n, c))


def test_reduce_reports_corrupt_stream_in_a_later_slab(oracle):
    # a broken tile index entry in the second slab of stream 5
    c = 64
    n = (1 << 20) + 4 * 8192
    w = synth.gaussian_bits(n * c, 0.02, 9)
    buf, sizes = zc.compress(to_dev(w), [n] * c)
    torch.cuda.synchronize()
    hb = buf.cpu().numpy().copy()
    off, _ = oracle.slot_offsets([n] * c)
    T = (n + 8191) // 8192
    t = T - 1                                # the last tile (second slab)
    p = off[5] + 32 + 4 * t                  # its offset in the tile index
    hb[p:p + 4] = np.frombuffer(np.uint32(0xFFFFFF00).tobytes(), np.uint8)
    say("reduce corrupt tile %d of stream 5" % t)
    out, status = zc.decompress_reduce(torch.from_numpy(hb).to(DEV), n, c, check=False)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st != 0 and (st & 0xFFFFFF) == 5, hex(st)


def test_reduce_full_size_gradient_buffer(oracle):
    # The gradient reduce-scatter workload at its real shape: one rank
    # receives a compressed copy of its 4M-value shard from each of 64 peers.
    w, cnt = synth.make(3, workers=8)
    c, n = len(cnt), int(cnt[0])
    assert np.all(cnt == n)
    say("reduce full size: %d x %d" % (c, n))
    x = to_dev(w)
    buf, sizes = zc.compress(x, cnt)
    out, status = zc.decompress_reduce(buf, n, c, check=False)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    # every position: chunk-order fp32 additions, one elementwise add per chunk
    xs = x.view(c, n)
    acc = torch.zeros(n, dtype=torch.float32, device=DEV)
    for k in range(c):
        acc = acc + (xs[k].to(torch.int32) << 16).view(torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    same_f32(got, acc.cpu().numpy())
    # every position against the oracle
    same_f32(got, oracle.reduce_bf16_f32(w, n, c))


# ---- the same sums delivered in bf16 (rounded once, to nearest even) ----

def gpu_reduce_bf16(w, n, c):
    buf, sizes = zc.compress(to_dev(w), [n] * c)
    out, status = zc.decompress_reduce(buf, n, c, check=False, bf16=True)
    torch.cuda.synchronize()
    return int(status.item()), out.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n,c", [(20000, 8), (20003, 8), (24576, 11), (1, 5), (7, 3),
                                 (65536 + 40, 17)])
def test_reduce_bf16_matches_oracle(oracle, n, c):
    w = special_mix(n * c, 2000 + n + c)
    say("reduce bf16 n=%d chunks=%d" % (n, c))
    st, got = gpu_reduce_bf16(w, n, c)
    assert st == 0, "status %#x" % st
    want = oracle.reduce_bf16_bf16(w, n, c)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "first differing sum at %d: %#x vs %#x" % (bad[0], got[bad[0]],
                                                                  want[bad[0]])


def test_reduce_bf16_rounds_once_at_the_end(oracle):
    # 1 + 2^-8 + 2^-8 = 1 + 2^-7 in fp32 (one bf16 step above 1.0); two
    # chunks give the tie 1 + 2^-8, which goes to the even 1.0; the largest
    # bf16 twice overflows to infinity
    n = 1024
    rows = [np.full(n, v, np.uint16) for v in (0x3F80, 0x3B80, 0x3B80)]
    st, got = gpu_reduce_bf16(np.concatenate(rows), n, 3)
    assert st == 0 and np.all(got == 0x3F81)
    st, got = gpu_reduce_bf16(np.concatenate(rows[:2]), n, 2)
    assert st == 0 and np.all(got == 0x3F80)
    st, got = gpu_reduce_bf16(np.full(2 * n, 0x7F7F, np.uint16), n, 2)
    assert st == 0 and np.all(got == 0x7F80)


def test_reduce_bf16_full_size_gradient_buffer(oracle):
    w, cnt = synth.make(3, workers=8)
    c, n = len(cnt), int(cnt[0])
    say("reduce bf16 full size: %d x %d" % (c, n))
    x = to_dev(w)
    buf, sizes = zc.compress(x, cnt)
    out, status = zc.decompress_reduce(buf, n, c, check=False, bf16=True)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    # every position: chunk-order PyTorch fp32 additions, then PyTorch's
    # conversion to bfloat16 (round to nearest even)
    xs = x.view(c, n)
    acc = torch.zeros(n, dtype=torch.float32, device=DEV)
    for k in range(c):
        acc = acc + (xs[k].to(torch.int32) << 16).view(torch.float32)
    want = acc.to(torch.bfloat16).view(torch.int16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want)
    # every position against the oracle
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.reduce_bf16_bf16(w, n, c))


# ---- decode and sum in one kernel (8 to 64 streams of at least 512 tiles) ----

FUSED_N = 512 * 8192 - 77                 # 512 tile positions, the last one partial


def test_reduce_fused_two_rounds_ragged(oracle):
    # 13 streams: a round of 8 and a round of 5 with three waves idle, a
    # partial last tile, special values and random patterns (raw groups,
    # escapes); fp32 and bf16 sums at every position
    c, n = 13, FUSED_N
    assert zc.zc_reduce_scratch_bytes(n, c) == 0
    w = special_mix(n * c, 79)
    say("reduce fused n=%d chunks=%d" % (n, c))
    buf, _ = zc.compress(to_dev(w), [n] * c)
    out, st = zc.decompress_reduce(buf, n, c, check=False)
    out16, st16 = zc.decompress_reduce(buf, n, c, check=False, bf16=True)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st16.item()) == 0
    same_f32(out.cpu().numpy(), oracle.reduce_bf16_f32(w, n, c))
    assert np.array_equal(out16.cpu().numpy().view(np.uint16), oracle.reduce_bf16_bf16(w, n, c))


def test_reduce_fused_all_raw_tiles(oracle):
    # uniform random bits: every group raw, every tile stream 8 KiB, decoded
    # from global memory
    c, n = 8, 512 * 8192
    w = np.random.default_rng(80).integers(0, 1 << 16, n * c, dtype=np.uint16)
    say("reduce fused, random bits, n=%d chunks=%d" % (n, c))
    st, got = gpu_reduce(w, n, c)
    assert st == 0, "status %#x" % st
    same_f32(got, oracle.reduce_bf16_f32(w, n, c))


def test_reduce_fused_streams_at_given_offsets(oracle):
    # the streams taken in another order through in_offsets: the sums follow
    # the call's order
    c, n = 9, FUSED_N
    w = synth.gaussian_bits(n * c, 0.02, 81)
    buf, _ = zc.compress(to_dev(w), [n] * c)
    off, _ = oracle.slot_offsets([n] * c)
    perm = np.array([4, 0, 8, 2, 7, 1, 5, 3, 6])
    say("reduce fused, permuted offsets")
    out, st = zc.decompress_reduce(buf, n, c, in_offsets=np.asarray(off)[perm], check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    wp = w.reshape(c, n)[perm].reshape(-1)
    same_f32(out.cpu().numpy(), oracle.reduce_bf16_f32(wp, n, c))


@pytest.mark.parametrize("stream,what", [(3, "header"), (10, "tile")])
def test_reduce_fused_reports_corrupt_stream(oracle, stream, what):
    # a broken header in the first round, a broken tile index entry of the
    # last tile in the second round
    c, n = 13, FUSED_N
    w = synth.gaussian_bits(n * c, 0.02, 82)
    buf, _ = zc.compress(to_dev(w), [n] * c)
    torch.cuda.synchronize()
    hb = buf.cpu().numpy().copy()
    off, _ = oracle.slot_offsets([n] * c)
    T = (n + 8191) // 8192
    if what == "header":
        hb[off[stream]] ^= 0xFF
    else:
        p = off[stream] + 32 + 4 * (T - 1)
        hb[p:p + 4] = np.frombuffer(np.uint32(0xFFFFFF00).tobytes(), np.uint8)
    say("reduce fused, corrupt %s of stream %d" % (what, stream))
    out, status = zc.decompress_reduce(torch.from_numpy(hb).to(DEV), n, c, check=False)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st != 0 and (st & 0xFFFFFF) == stream, hex(st)
    if what == "header":
        assert st >> 24 == 1, hex(st)
