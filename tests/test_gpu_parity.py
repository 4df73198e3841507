"""GPU parity: the HIP path through the C ABI against the CPU oracle.

The bar is bit-exactness: the compressed stream byte for byte (up to each
chunk's comp_bytes), the sizes, and the round trip, on the same seeded inputs.
Cross-decoding (GPU decodes oracle streams, oracle decodes GPU streams) checks
both directions of the format.  Every chunk is compared, the full-size
workloads included (the oracle runs over their chunks in a thread pool).
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from lossless_bf16_tensor_sign_amd import synth, zc
from tests import golden_io, oracle_pool

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TILE = 8192


def say(msg):
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def to_dev(w):
    return torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(DEV)


def gpu_compress(w, counts):
    counts = np.asarray(counts, np.int64)
    buf, sizes = zc.compress(to_dev(w), counts)
    torch.cuda.synchronize()
    return buf.cpu().numpy(), sizes.cpu().numpy()


def gpu_decompress(buf_np, counts, offsets=None):
    d = torch.from_numpy(buf_np).to(DEV)
    out, status = zc.decompress(d, counts, in_offsets=offsets, check=False)
    torch.cuda.synchronize()
    return int(status.item()), out.cpu().numpy().view(np.uint16)


def check_against_oracle(oracle, w, counts, label=""):
    """GPU stream == oracle stream, byte for byte, for every chunk; the oracle
    decodes every GPU stream; the GPU decodes its own buffer."""
    counts = np.asarray(counts, np.int64)
    say("compress %s: %d chunks, %d values" % (label, len(counts), counts.sum()))
    gbuf, gsizes = gpu_compress(w, counts)
    off, total = oracle.slot_offsets(counts)
    assert gbuf.size >= total
    say("oracle comparison %s" % label)
    oracle_pool.compare_chunks(oracle, w, counts, gbuf, gsizes, off, label=label)
    for c in range(len(counts)):
        assert 32 <= gsizes[c] <= oracle.chunk_bound(int(counts[c]))
    say("decompress %s" % label)
    st, back = gpu_decompress(gbuf, counts)
    assert st == 0, "status %#x" % st
    assert np.array_equal(back, w)
    return gbuf, gsizes


# ------------------------------------------------------------ golden ---

@pytest.mark.parametrize("name", golden_io.names())
def test_golden_streams_gpu(name):
    w, want = golden_io.load(name)
    say("golden " + name)
    gbuf, gsizes = gpu_compress(w, [w.size])
    assert gsizes[0] == want.size
    assert np.array_equal(gbuf[:want.size], want)
    slot = np.zeros(zc.zc_bound([w.size]), np.uint8)
    slot[:want.size] = want
    st, back = gpu_decompress(slot, [w.size])
    assert st == 0 and np.array_equal(back, w)


# ------------------------------------------------------------ edges ---

@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 511, 512, 513, 8191, 8192, 8193,
                               20000, 3 * 8192 + 17, 5 * 8192])
def test_edge_sizes_single_chunk(oracle, n):
    w = synth.gaussian_bits(n, 0.03, seed=1000 + n)
    check_against_oracle(oracle, w, [n], label="n=%d" % n)


def test_ragged_multi_chunk_with_empties(oracle):
    cnt = np.array([0, 1, 7, 8192, 0, 8193, 13, 20000, 0, 3], np.int64)
    w = synth.gaussian_bits(int(cnt.sum()), 0.01, seed=7)
    w[::501] = 0x7FC0
    check_against_oracle(oracle, w, cnt, label="ragged")


def test_more_chunks_than_one_launch(oracle):
    rng = np.random.default_rng(8)
    cnt = rng.integers(0, 30000, size=200).astype(np.int64)
    cnt[rng.random(200) < 0.15] = 0
    w = synth.gaussian_bits(int(cnt.sum()), 0.02, seed=9)
    check_against_oracle(oracle, w, cnt, label="200 chunks")


@pytest.mark.parametrize("v", [0x7FC0, 0x8000, 0x0000, 0x7F7F, 0xFF80, 0x0001])
def test_constant_special_values(oracle, v):
    cnt = [1, 128, 8192, 8193 + 64]
    w = np.full(sum(cnt), v, np.uint16)
    check_against_oracle(oracle, w, cnt, label="const %#06x" % v)


def test_all_patterns_three_layouts(oracle):
    w = np.arange(65536, dtype=np.uint16)
    check_against_oracle(oracle, w, [65536], label="patterns in order")
    for seed in range(3):
        w = np.random.default_rng(seed).permutation(65536).astype(np.uint16)
        check_against_oracle(oracle, w, [65536], label="shuffle %d" % seed)
    w = synth.gaussian_bits(65536 * 128, 0.02, seed=99)
    q = np.arange(65536)
    t, lane = np.divmod(q, 64)
    k, j = np.divmod(q % 128, 8)
    w[t * TILE + k * 512 + lane * 8 + j] = q.astype(np.uint16)
    check_against_oracle(oracle, w, [w.size], label="patterns in gaussian groups")


def test_cross_decode_oracle_streams(oracle):
    cnt = np.array([5, 0, 8192, 9000, 1, 70000], np.int64)
    w = synth.gaussian_bits(int(cnt.sum()), 0.005, seed=21)
    w[::333] = 0
    buf, sizes, _ = oracle.compress(w, cnt)
    say("gpu decodes oracle slot buffer")
    st, back = gpu_decompress(buf, cnt)
    assert st == 0 and np.array_equal(back, w)
    # packed at 16-byte boundaries, explicit offsets
    off, _ = oracle.slot_offsets(cnt)
    offs = np.concatenate([[0], np.cumsum((sizes + 15) // 16 * 16)])[:-1]
    packed = np.zeros(int(offs[-1] + sizes[-1]) + 64, np.uint8)
    for c in range(len(cnt)):
        packed[offs[c]:offs[c] + sizes[c]] = buf[off[c]:off[c] + sizes[c]]
    st, back = gpu_decompress(packed, cnt, offsets=offs)
    assert st == 0 and np.array_equal(back, w)


def test_unaligned_chunk_starts(oracle):
    # chunk starts at odd value offsets: the scalar load/store path
    cnt = np.array([3, 8195, 1, 16390, 5], np.int64)
    w = synth.gaussian_bits(int(cnt.sum()), 0.02, seed=5)
    check_against_oracle(oracle, w, cnt, label="unaligned")


def test_deterministic_repeat(oracle):
    # Repeated calls give the same streams (slot bytes after a stream's end
    # are never written, so only [slot_off, slot_off + comp_bytes) counts).
    cnt = np.full(16, 1 << 18, np.int64)
    w = synth.gaussian_bits(int(cnt.sum()), 0.02, seed=3)
    x = to_dev(w)
    off, _ = oracle.slot_offsets(cnt)
    say("determinism x5")
    first = None
    for _ in range(5):
        buf, sizes = zc.compress(x, cnt)
        b, sz = buf.cpu().numpy(), sizes.cpu().numpy()
        streams = [b[off[c]:off[c] + sz[c]].copy() for c in range(len(cnt))]
        if first is None:
            first = streams
        else:
            for c in range(len(cnt)):
                assert np.array_equal(streams[c], first[c]), c


@pytest.mark.parametrize("cfg", [3, 4])
def test_deterministic_repeat_full_size(cfg):
    # The gradient workload (escape steps and raw groups in most tiles) and
    # the MoE layout (chunk-end tiles), compressed four times into zeroed
    # buffers: every byte of every call equals the first call's.
    w, cnt = synth.make(cfg, workers=8)
    x = to_dev(w)
    bound = zc.zc_bound(cnt)
    ws = torch.zeros(zc.zc_workspace_bytes(cnt), dtype=torch.uint8, device=x.device)
    say("determinism workload %d x4" % cfg)
    first = None
    for _ in range(4):
        out = torch.zeros(bound, dtype=torch.uint8, device=x.device)
        sizes = torch.zeros(len(cnt), dtype=torch.int64, device=x.device)
        assert zc.zc_compress(x, cnt, out, sizes, ws) == zc.ZC_OK
        torch.cuda.synchronize()
        if first is None:
            first = (out, sizes)
        else:
            assert torch.equal(sizes, first[1])
            assert torch.equal(out, first[0])


# ------------------------------------------------------- workloads ---

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_full_size(oracle, cfg):
    # every chunk of the workload, byte for byte against the oracle
    w, cnt = synth.make(cfg, workers=8)
    gbuf, gsizes = check_against_oracle(oracle, w, cnt, label="workload %d" % cfg)
    ratio = 2.0 * w.size / float(gsizes.sum())
    say("workload %d ratio %.4f" % (cfg, ratio))
    if cfg == 5:
        assert 0.98 < ratio < 1.0
    else:
        assert ratio > 1.3


def test_largest_chunk(oracle):
    # one chunk of ZC_MAX_CHUNK_VALUES (2^31 - 1) values: 262 144 tiles, the
    # last one ragged, streams past 4 GiB.  A tile's stream, group maxima,
    # group lengths and raw bytes depend only on its own values, so sampled
    # tiles are compared byte for byte with the oracle's stream of a chunk
    # made of those values alone; the whole chunk round-trips through the
    # strict decoder, which accepts only the unique encoding.
    n = (1 << 31) - 1
    T = (n + 8191) // 8192
    say("largest chunk: %d values, %d tiles" % (n, T))
    g = torch.Generator(device=DEV)
    g.manual_seed(20260131)
    x = (torch.randn(n, device=DEV, generator=g) * 0.02).to(torch.bfloat16).view(torch.int16)
    x[::997] = 0                                   # exact zeros: escapes
    mid = T // 2
    x[mid * 8192:(mid + 1) * 8192] = torch.randint(-32768, 32768, (8192,), device=DEV,
                                                   generator=g, dtype=torch.int32).to(torch.int16)
    buf, sizes = zc.compress(x, [n])
    torch.cuda.synchronize()
    comp = int(sizes[0].item())
    Tg, _, R, X = oracle.geometry(n)
    assert Tg == T and X < comp <= oracle.chunk_bound(n)
    hdr = buf[:32].cpu().numpy().view(np.uint32)
    assert hdr[4] == n and (int(hdr[6]) | (int(hdr[7]) << 32)) == comp
    toff = buf[32:32 + 4 * T].cpu().numpy().view(np.uint32).astype(np.int64)
    assert toff[0] == 0 and np.all(np.diff(toff) >= 0)
    for t in (0, 1, mid, T - 2, T - 1):
        m = min(8192, n - 8192 * t)
        w = x[8192 * t:8192 * t + m].cpu().numpy().view(np.uint16)
        ref = oracle.compress_chunk(w)
        _, _, R1, X1 = oracle.geometry(m)
        end = toff[t + 1] if t + 1 < T else comp - X
        got_stream = buf[X + toff[t]:X + end].cpu().numpy()
        assert np.array_equal(got_stream, ref[X1:]), "tile %d stream" % t
        emax = buf[32 + 4 * T + 64 * t:32 + 4 * T + 64 * (t + 1)].cpu().numpy()
        assert np.array_equal(emax, ref[36:100]), "tile %d emax" % t
        glen = buf[32 + 68 * T + 128 * t:32 + 68 * T + 128 * (t + 1)].cpu().numpy()
        assert np.array_equal(glen, ref[100:228]), "tile %d glen" % t
        raw = buf[R + 8192 * t:R + 8192 * t + m].cpu().numpy()
        assert np.array_equal(raw, ref[R1:R1 + m]), "tile %d raw bytes" % t
    say("largest chunk: decompress")
    y, status = zc.decompress(buf, [n], check=False)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(x, y)


# ------------------------------------------------ look-back fallback ---

@pytest.mark.parametrize("layout", ["equal", "ragged"])
def test_lookback_recompute_path(layout):
    # A spin limit of 0: every tile that finds a predecessor unpublished
    # recomputes that predecessor's size from its input at once.  The limit
    # is read once per process, so the case runs in a child process with
    # ZC_LOOKBACK_SPIN_LIMIT=0; it compares every chunk with the oracle, for
    # equal chunks and for uneven ones (tiles taken chunk by chunk in grid
    # order).
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, ZC_LOOKBACK_SPIN_LIMIT="0")
    say("look-back recompute path (child process), %s chunks" % layout)
    r = subprocess.run([sys.executable, "-m", "tests.lookback_child", layout], cwd=root,
                       env=env, capture_output=True, text=True, timeout=300)
    sys.stdout.write(r.stdout[-2000:])
    assert r.returncode == 0, r.stderr[-3000:]
    assert "lookback child ok" in r.stdout


# -------------------------------------------- device-resident split ---

def _zipf_split(total, chunks, seed):
    p = 1.0 / np.arange(1, chunks + 1) ** 1.1
    return np.random.default_rng(seed).multinomial(total, p / p.sum()).astype(np.int64)


DEV_SPLITS = {
    "ragged": np.array([0, 1, 7, 8192, 0, 8193, 13, 20000, 0, 3], np.int64),
    "equal": np.full(8, 3 * TILE, np.int64),
    "zipf64": _zipf_split(400_000, 64, 3),
    "150 chunks": np.random.default_rng(4).integers(0, 9000, 150).astype(np.int64),
}


@pytest.mark.parametrize("name", list(DEV_SPLITS))
def test_device_split_matches_host_path(oracle, name):
    # Counts that live on the device give the host path's streams, byte for
    # byte, at the same slot offsets; both decoders restore the input.
    cnt = DEV_SPLITS[name]
    total = int(cnt.sum())
    w = synth.gaussian_bits(total, 0.02, seed=40 + len(cnt))
    w[::611] = 0
    say("device split %s: %d chunks, %d values" % (name, len(cnt), total))
    hbuf, hsizes = gpu_compress(w, cnt)
    dc = torch.from_numpy(cnt).to(DEV)
    out, sizes, slots = zc.compress_dev(to_dev(w), dc)
    torch.cuda.synchronize()
    off, _ = oracle.slot_offsets(cnt)
    sizes, slots, ob = sizes.cpu().numpy(), slots.cpu().numpy(), out.cpu().numpy()
    assert np.array_equal(slots, off[:len(cnt)])
    assert np.array_equal(sizes, hsizes)
    vo = np.concatenate([[0], np.cumsum(cnt)])
    for c in range(len(cnt)):
        got = ob[off[c]:off[c] + sizes[c]]
        assert np.array_equal(got, hbuf[off[c]:off[c] + sizes[c]]), (name, c)
        if c % 7 == 0:
            assert np.array_equal(got, oracle.compress_chunk(w[vo[c]:vo[c + 1]])), (name, c)
    back, st = zc.decompress_dev(out, dc, total)
    assert int(st.item()) == 0
    assert np.array_equal(back.cpu().numpy().view(np.uint16), w)
    # explicit device offsets: the streams packed back to back
    packed = np.zeros(int(sum(((s + 15) // 16) * 16 for s in sizes)) + 16, np.uint8)
    poff, pos = [], 0
    for c in range(len(cnt)):
        packed[pos:pos + sizes[c]] = ob[off[c]:off[c] + sizes[c]]
        poff.append(pos)
        pos += ((int(sizes[c]) + 15) // 16) * 16
    doff = torch.tensor(poff, dtype=torch.int64, device=DEV)
    back, st = zc.decompress_dev(torch.from_numpy(packed).to(DEV), dc, total, d_in_offsets=doff)
    assert int(st.item()) == 0
    assert np.array_equal(back.cpu().numpy().view(np.uint16), w)


def test_device_split_full_moe_layout(oracle):
    # The MoE all-to-all workload at full size (64 Zipf-sized chunks): the
    # device-split call writes the host path's streams; compared on the GPU.
    w, cnt = synth.make(4, workers=8)
    total = int(cnt.sum())
    say("device split, MoE layout: %d values" % total)
    x = to_dev(w)
    hbuf, hsizes = zc.compress(x, cnt)
    dc = torch.from_numpy(cnt).to(DEV)
    dbuf, dsizes, dslots = zc.compress_dev(x, dc)
    torch.cuda.synchronize()
    off, _ = oracle.slot_offsets(cnt)
    assert np.array_equal(dslots.cpu().numpy(), off[:len(cnt)])
    assert torch.equal(hsizes, dsizes)
    for c, s in enumerate(dsizes.cpu().tolist()):
        assert torch.equal(hbuf[off[c]:off[c] + s], dbuf[off[c]:off[c] + s]), c
    back, st = zc.decompress_dev(dbuf, dc, total)
    assert int(st.item()) == 0 and torch.equal(back, x)


def test_device_split_rejects_bad_counts():
    cnt = np.array([100, 200, 300], np.int64)
    w = synth.gaussian_bits(600, 0.02, seed=3)
    x = to_dev(w)
    for bad in ([100, 200, 299], [100, -5, 505]):
        dc = torch.tensor(bad, dtype=torch.int64, device=DEV)
        total = 600
        out = torch.zeros(zc.zc_bound_max(total, 3), dtype=torch.uint8, device=DEV)
        sizes = torch.zeros(3, dtype=torch.int64, device=DEV)
        slots = torch.zeros(3, dtype=torch.int64, device=DEV)
        ws = torch.zeros(zc.zc_workspace_bytes_max(total, 3), dtype=torch.uint8, device=DEV)
        assert zc.zc_compress_dev(x, dc, total, out, sizes, slots, ws) == zc.ZC_OK
        torch.cuda.synchronize()
        assert sizes.cpu().tolist() == [-1, -1, -1]
        assert slots.cpu().tolist() == [-1, -1, -1]
        assert int(out.sum().item()) == 0
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        y = torch.empty(600, dtype=torch.int16, device=DEV)
        assert zc.zc_decompress_dev(out, dc, total, y, status, ws) == zc.ZC_OK
        torch.cuda.synchronize()
        assert int(status.item()) >> 24 == 2     # SIZE
    assert cnt.sum() == 600


# ---------------------------------------------------------- errors ---

def test_capacity_and_argument_errors():
    cnt = np.array([10000], np.int64)
    x = to_dev(synth.gaussian_bits(10000, 0.02, seed=1))
    out = torch.empty(zc.zc_bound(cnt) - 1, dtype=torch.uint8, device=DEV)
    sizes = torch.empty(1, dtype=torch.int64, device=DEV)
    ws = torch.zeros(zc.zc_workspace_bytes(cnt), dtype=torch.uint8, device=DEV)
    assert zc.zc_compress(x, cnt, out, sizes, ws) == zc.ZC_ENOSPC
    out = torch.empty(zc.zc_bound(cnt), dtype=torch.uint8, device=DEV)
    assert zc.zc_compress(x, cnt, out, sizes, ws[:16]) == zc.ZC_ENOSPC
    assert zc.zc_compress(x, [-5], out, sizes, ws) == zc.ZC_EINVAL


def _mutations(stream, rng, count):
    for i in range(count):
        m = stream.copy()
        pos = int(rng.integers(0, m.size))
        if i % 2:
            m[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
        else:
            m[pos] = np.uint8(rng.integers(0, 256))
        yield m


def test_corrupt_streams_match_oracle_verdict(oracle):
    # Both strict decoders must accept exactly the same mutated streams, and
    # agree on the decoded values when they accept.
    rng = np.random.default_rng(77)
    n = 2 * TILE + 300
    w = synth.gaussian_bits(n, 0.02, seed=12)
    w[rng.integers(0, n, 30)] = rng.integers(0, 65536, 30).astype(np.uint16)
    ref = oracle.compress_chunk(w)
    cap = zc.zc_bound([n])
    muts = list(_mutations(ref, rng, 300))
    # truncations: in_bytes smaller than comp_bytes
    say("corrupt streams: %d mutations" % len(muts))
    agree = 0
    for m in muts:
        r_o, back_o = oracle.decompress_chunk(m, n)
        slot = np.zeros(cap, np.uint8)
        slot[:m.size] = m
        st, back_g = gpu_decompress(slot, [n])
        assert (r_o == 0) == (st == 0), (r_o, hex(st))
        if st == 0:
            assert np.array_equal(back_g, back_o)
        agree += 1
    assert agree == len(muts)
    for cut in (40, ref.size // 2, ref.size - 4):
        d = torch.from_numpy(ref[:cut].copy()).to(DEV)
        out = torch.empty(n, dtype=torch.int16, device=DEV)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        assert zc.zc_decompress(d, [n], out, status) == zc.ZC_OK
        torch.cuda.synchronize()
        assert int(status.item()) >> 24 == 2     # SIZE


# ----------------------------------------------------- stress layouts ---

def _stress_tiles(kind, tiles, seed):
    """Crafted tiles that drive the kernels' less common paths."""
    rng = np.random.default_rng(seed)
    w = synth.gaussian_bits(tiles * TILE, 0.02, seed=seed)
    grid = w.reshape(tiles, 16, 64, 8)           # tile, step, lane, value
    if kind == "raw_heavy":
        # lanes below `cut` get one huge value, which forces raw mode; the
        # tile stream then exceeds 4 KiB without every group being raw
        for t in range(tiles):
            cut = int(rng.integers(34, 60))
            grid[t, 0, :cut, 3] = 0x7F00          # e = 254
    elif kind == "escape_runs":
        # runs of three zeros inside one half-step (members 4h..4h+2): three
        # escapes (66 bits) overflow the 64-bit decode window; the group stays
        # coded (a few escapes are far below 8 bits per value)
        for t in range(tiles):
            for lane in range(64):
                for h in rng.choice(32, size=3, replace=False):
                    k, j0 = divmod(4 * int(h), 8)
                    grid[t, k, lane, j0:j0 + 3] = 0
    elif kind == "long_codes":
        # values 12-15 binades below the group maximum: long code words
        for t in range(tiles):
            for lane in range(64):
                pos = rng.integers(0, 128, size=6)
                e = 110 + rng.integers(0, 4, size=6)
                grid[t, pos // 8, lane, pos % 8] = (e << 7).astype(np.uint16)
            grid[t, 0, :, 0] = 125 << 7
    elif kind == "escape_single":
        # one zero per lane and step, its pair partner a short code: every
        # escape pair fits in 32 bits (escape words are 22 bits)
        for t in range(tiles):
            for k in range(16):
                j = 2 * rng.integers(0, 4, size=64) + rng.integers(0, 2, size=64)
                grid[t, k, np.arange(64), j] = 0
    elif kind == "escape_long":
        # zeros whose pair partner is 11-14 binades below the group maximum
        # (long code words): such a pair exceeds 32 bits, the others fit
        for t in range(tiles):
            grid[t, 0, :, 0] = 125 << 7
            for lane in range(64):
                for q in rng.choice(63, size=4, replace=False):
                    m = 2 * (int(q) + 1)
                    k, j = divmod(m, 8)
                    grid[t, k, lane, j] = 0
                    grid[t, k, lane, j + 1] = (111 + int(rng.integers(0, 4))) << 7
    return grid.reshape(-1)


@pytest.mark.parametrize("kind", ["raw_heavy", "escape_runs", "long_codes", "escape_single",
                                  "escape_long"])
def test_stress_layouts(oracle, kind):
    seed = {"raw_heavy": 11, "escape_runs": 12, "long_codes": 13, "escape_single": 14,
            "escape_long": 15}[kind]
    w = _stress_tiles(kind, 5, seed=seed)
    n = w.size
    # full tiles, then the same data with a ragged tail and an unaligned start
    check_against_oracle(oracle, w, [n], label=kind)
    cnt = np.array([3, n - 3 - 1000, 1000], np.int64)
    check_against_oracle(oracle, w, cnt, label=kind + " ragged")


def test_stress_paths_are_taken(oracle):
    # the crafted layouts really produce the intended stream shapes
    s = oracle.compress_chunk(_stress_tiles("raw_heavy", 2, seed=1))
    T, NG, R, X = oracle.geometry(2 * TILE)
    toffs = s[32:32 + 4 * T].view(np.uint32)
    assert toffs[1] - toffs[0] > 4096            # tile stream beyond the LDS buffer
    glen = s[32 + 68 * T:32 + 68 * T + 2 * NG].view(np.uint16)
    assert 0 < int((glen == 1024).sum()) < NG     # raw and coded groups mixed
    for kind in ("escape_single", "escape_long"):
        s = oracle.compress_chunk(_stress_tiles(kind, 2, seed=1))
        glen = s[32 + 68 * T:32 + 68 * T + 2 * NG].view(np.uint16)
        assert int(glen.max()) < 1024, kind       # every group coded


# ------------------------------------------- corrupt-stream reports ---

def _corrupt_chunk70_buffer(oracle):
    # 100 small chunks in the slot layout, chunk 70's stream damaged
    cnt = np.array([3000 + 37 * (c % 11) for c in range(100)], np.int64)
    w = synth.gaussian_bits(int(cnt.sum()), 0.02, seed=70)
    buf, sizes, _ = oracle.compress(w, cnt)
    off, _ = oracle.slot_offsets(cnt)
    bad = buf.copy()
    bad[off[70] + 12] ^= 1                    # reserved header word
    return cnt, w, bad


def test_corrupt_chunk_index_past_first_launch(oracle):
    # chunk 70 lies in the second 64-chunk launch: the status word names it
    # by its index in the call, with the header reason
    cnt, w, bad = _corrupt_chunk70_buffer(oracle)
    say("corrupt chunk 70 of 100 (host counts)")
    st, back = gpu_decompress(bad, cnt)
    assert st >> 24 == 1 and st & 0xFFFFFF == 70, hex(st)
    vo = np.concatenate([[0], np.cumsum(cnt)])
    assert np.array_equal(back[:vo[70]], w[:vo[70]])
    assert np.array_equal(back[vo[71]:], w[vo[71]:])
    say("corrupt chunk 70 of 100 (device counts)")
    dc = torch.from_numpy(cnt).to(DEV)
    y, status = zc.decompress_dev(torch.from_numpy(bad).to(DEV), dc, int(cnt.sum()),
                                  check=False)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st >> 24 == 1 and st & 0xFFFFFF == 70, hex(st)


def test_decoder_writes_stay_in_the_chunk(oracle):
    # Canary: three chunks decoded into a window of a larger buffer filled
    # with a sentinel; the middle chunk's stream is damaged in many ways.
    # The outer chunks must decode exactly, the sentinel before and after the
    # window must stay, and the middle chunk's region may change only inside
    # itself (nothing spills into its neighbours).
    rng = np.random.default_rng(123)
    cnt = np.array([TILE + 77, 2 * TILE + 300, 5000], np.int64)
    w = synth.gaussian_bits(int(cnt.sum()), 0.02, seed=124)
    w[rng.integers(0, w.size, 40)] = rng.integers(0, 65536, 40).astype(np.uint16)
    buf, sizes, _ = oracle.compress(w, cnt)
    off, _ = oracle.slot_offsets(cnt)
    vo = np.concatenate([[0], np.cumsum(cnt)])
    n = int(cnt.sum())
    guard = 4096                                 # values on each side of the window
    sentinel = np.int16(0x5A5A)
    mid = buf[off[1]:off[1] + sizes[1]]
    T, _, R, X = oracle.geometry(int(cnt[1]))
    # damage in each section: header and index [0, R), sign+mantissa bytes
    # [R, X) (these decode validly to other values), exponent streams [X, end)
    muts = []
    for lo, hi in ((0, R), (R, X), (X, mid.size)):
        for i in range(50):
            m = mid.copy()
            pos = int(rng.integers(lo, hi))
            if i % 2:
                m[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
            else:
                m[pos] = np.uint8(rng.integers(0, 256))
            muts.append(m)
    # targeted: n, comp_bytes, a tile offset, a group length, a group maximum
    for pos, val in ((16, 0xFF), (24, 0xFF), (31, 0x7F), (32 + 4, 0xFF),
                     (32 + 68 * T + 2 * 5 + 1, 0xFF), (32 + 4 * T + 9, 0xFF)):
        m = mid.copy()
        m[pos] = val
        muts.append(m)
    say("canary: %d damaged middle streams" % len(muts))
    big = torch.empty(n + 2 * guard, dtype=torch.int16, device=DEV)
    window = big[guard:guard + n]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rejected = 0
    for i, m in enumerate(muts):
        b = buf.copy()
        b[off[1]:off[1] + sizes[1]] = m
        big.fill_(sentinel)
        status.zero_()
        d = torch.from_numpy(b).to(DEV)
        assert zc.zc_decompress(d, cnt, window, status) == zc.ZC_OK
        torch.cuda.synchronize()
        got = big.cpu().numpy()
        st = int(status.item())
        assert np.all(got[:guard] == sentinel), i
        assert np.all(got[guard + n:] == sentinel), i
        out = got[guard:guard + n].view(np.uint16)
        assert np.array_equal(out[:vo[1]], w[:vo[1]]), i
        assert np.array_equal(out[vo[2]:], w[vo[2]:]), i
        r_o, back_o = oracle.decompress_chunk(m, int(cnt[1]))
        assert (st == 0) == (r_o == 0), (i, hex(st), r_o)
        if st:
            assert st & 0xFFFFFF == 1, hex(st)
            rejected += 1
        else:
            assert np.array_equal(out[vo[1]:vo[2]], back_o), i
    # the oracle rejects about 30 of each 50 in the index and exponent
    # sections, none in the sign+mantissa bytes
    assert 40 <= rejected <= 110, rejected


# ------------------------------------------- workspace launch tags ---

WS_HEADER = 8448         # header bytes: u32 tag of the last launch at 0, then 64 u32
WS_COUNTERS = 64         # counters of finished workgroups, one per 128-byte line from 128
WS_SLOT = 64             # one 8-byte status word per 64-byte line after the header


def _compress_into(x, cnt, ws):
    cnt = np.asarray(cnt, np.int64)
    out = torch.zeros(zc.zc_bound(cnt), dtype=torch.uint8, device=DEV)
    sizes = torch.zeros(len(cnt), dtype=torch.int64, device=DEV)
    assert zc.zc_compress(x, cnt, out, sizes, ws) == zc.ZC_OK
    torch.cuda.synchronize()
    return out.cpu().numpy(), sizes.cpu().numpy()


def test_workspace_reused_across_calls(oracle):
    # One workspace for a run of calls with different data and layouts: the
    # status words of earlier calls carry older tags and are never taken for
    # this call's; every call's streams equal the oracle's, and the header
    # holds the number of calls made, its counter back at zero.
    layouts = [np.full(6, 5 * TILE, np.int64), np.array([3, 9 * TILE + 1, 0, TILE], np.int64),
               np.full(3, 11 * TILE, np.int64), np.array([70 * TILE + 9], np.int64)]
    ws = torch.zeros(max(zc.zc_workspace_bytes(c) for c in layouts), dtype=torch.uint8,
                     device=DEV)
    for i, cnt in enumerate(layouts * 2):
        w = synth.gaussian_bits(int(cnt.sum()), 0.001 * (i + 1), seed=300 + i)
        w[::(101 + i)] = 0
        say("reused workspace, call %d: %s" % (i, cnt.tolist()))
        b, sz = _compress_into(to_dev(w), cnt, ws)
        off, _ = oracle.slot_offsets(cnt)
        oracle_pool.compare_chunks(oracle, w, cnt, b, sz, off, label="call %d" % i)
        hdr = ws[:WS_HEADER].cpu().numpy().view(np.uint32)
        counters = hdr[32:32 + 32 * WS_COUNTERS:32]
        assert hdr[0] == i + 1 and not counters.any(), (i, hdr[0], counters)


def test_workspace_tag_wraps(oracle):
    # The launch tag wraps after 2^32 - 1 launches: the launch that takes the
    # last tag clears every status slot of the workspace before it stores the
    # tag, and the next launch starts again at 1.  Forced here by writing the
    # header; both calls must still equal the oracle.
    cnt = np.full(4, 7 * TILE, np.int64)
    ws = torch.zeros(zc.zc_workspace_bytes(cnt), dtype=torch.uint8, device=DEV)
    ws[:4].view(torch.int32)[0] = -2           # stored tag 0xFFFFFFFE
    for i, tag in enumerate((0xFFFFFFFF, 1)):
        w = synth.gaussian_bits(int(cnt.sum()), 0.02, seed=400 + i)
        b, sz = _compress_into(to_dev(w), cnt, ws)
        off, _ = oracle.slot_offsets(cnt)
        oracle_pool.compare_chunks(oracle, w, cnt, b, sz, off, label="wrap call %d" % i)
        h = ws.cpu().numpy()
        assert int(h[:4].view(np.uint32)[0]) == tag
        slots = h[WS_HEADER:].reshape(-1, WS_SLOT)[:, :8].copy().view(np.uint64).ravel()
        if tag == 0xFFFFFFFF:
            assert not slots.any()                 # cleared after the last use of the tag
        else:
            assert np.all((slots >> np.uint64(32)) == 1)    # every tile published with tag 1
