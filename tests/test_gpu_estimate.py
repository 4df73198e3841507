"""GPU parity of the sampled size estimate (zc_estimate) against the oracle.

The expected values come from the oracle's own streams: each tile's stream
bytes are read off the stream's tile index (consecutive tile_off entries, and
the exponent section's end for the last tile), then sampled and scaled with
the rule the header states.  With every tile sampled the estimate must equal
the exact size, which zc_compress must also write.
"""
import sys

import numpy as np
import pytest
import torch

from lossless_bf16_tensor_sign_amd import synth, zc
from tests import oracle_pool

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TILE = 8192


def say(msg):
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def oracle_tile_bytes(oracle, w):
    """(X, per-tile exponent-stream bytes) of the oracle's stream for w."""
    s = oracle.compress_chunk(w)
    T, _, _, X = oracle.geometry(w.size)
    comp = int(s[24:32].view(np.uint64)[0])
    assert comp == s.size
    if T == 0:
        return X, np.zeros(0, np.int64)
    off = s[32:32 + 4 * T].view(np.uint32).astype(np.int64)
    ends = np.append(off[1:], comp - X)
    return X, ends - off


def expected(oracle, w, counts, samples):
    vo = np.concatenate([[0], np.cumsum(counts)])
    out = []
    for c, n in enumerate(counts):
        X, tb = oracle_tile_bytes(oracle, w[vo[c]:vo[c + 1]])
        T = tb.size
        k = min(samples, T)
        if k == 0:
            out.append(X)
            continue
        s = int(sum(int(tb[(i * T) // k]) for i in range(k)))
        out.append(X + (s * T + k // 2) // k)
    return np.array(out, np.int64)


def gpu_estimate(w, counts, samples):
    x = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(DEV)
    d = torch.from_numpy(np.asarray(counts, np.int64)).to(DEV)
    est = zc.estimate(x, d, samples)
    torch.cuda.synchronize()
    return est.cpu().numpy()


def ragged_case(seed):
    rng = np.random.default_rng(seed)
    counts = np.array([0, 1, 7, 8192, 8193, 20003, 0, 3 * 8192 + 5, 65536 + 17, 517],
                      np.int64)
    parts = []
    for c, n in enumerate(counts):
        g = synth.gaussian_bits(int(n), float(10.0 ** rng.uniform(-3, 0)), seed + c)
        if c % 3 == 0 and n:
            m = rng.random(int(n)) < 0.01          # escapes and raw groups
            g[m] = rng.integers(0, 1 << 16, int(m.sum()), dtype=np.uint16)
        parts.append(g)
    return np.concatenate(parts), counts


@pytest.mark.parametrize("samples", [1, 2, 3, 1 << 20])
def test_estimate_matches_oracle_ragged(oracle, samples):
    w, counts = ragged_case(41)
    say("estimate ragged, samples=%d" % samples)
    got = gpu_estimate(w, counts, samples)
    assert np.array_equal(got, expected(oracle, w, counts, samples))


def test_exact_estimate_equals_compressed_sizes(oracle):
    w, counts = ragged_case(43)
    got = gpu_estimate(w, counts, 1 << 20)
    buf, sizes = zc.compress(torch.from_numpy(w.view(np.int16)).to(DEV), counts)
    torch.cuda.synchronize()
    assert np.array_equal(got, sizes.cpu().numpy())
    vo = np.concatenate([[0], np.cumsum(counts)])
    for c in range(len(counts)):
        assert got[c] == oracle.compress_chunk(w[vo[c]:vo[c + 1]]).size


def test_estimate_incompressible_chunk(oracle):
    rng = np.random.default_rng(5)
    w = rng.integers(0, 1 << 16, 5 * TILE + 77, dtype=np.uint16)
    counts = [w.size]
    for s in (1, 4, 100):
        assert np.array_equal(gpu_estimate(w, counts, s), expected(oracle, w, counts, s))


def test_invalid_split_gives_minus_one():
    w = synth.gaussian_bits(3 * TILE, 0.02, 9)
    x = torch.from_numpy(w.view(np.int16)).to(DEV)
    for bad in ([TILE, TILE, TILE + 1], [-1, TILE, 2 * TILE + 1], [2 ** 31, 0, 0]):
        d = torch.tensor(bad, dtype=torch.int64, device=DEV)
        est = torch.zeros(3, dtype=torch.int64, device=DEV)
        assert zc.zc_estimate(x, d, w.size, 4, est) == zc.ZC_OK
        torch.cuda.synchronize()
        assert est.cpu().tolist() == [-1, -1, -1]


def test_estimate_full_moe_workload(oracle):
    # The MoE all-to-all workload at full size (64 Zipf-sized chunks): with 8
    # samples per chunk every chunk's estimate equals the oracle-derived one,
    # and the total is within a few percent of the real compressed size; with
    # samples >= T every estimate is the exact size.
    w, cnt = synth.make(4, workers=8)
    say("estimate MoE layout: %d values" % w.size)
    vo = oracle_pool.value_offsets(cnt)
    per_chunk = oracle_pool.map_chunks(
        lambda c: oracle_tile_bytes(oracle, w[vo[c]:vo[c + 1]]), len(cnt))

    def expect(samples):
        out = []
        for X, tb in per_chunk:
            T = tb.size
            k = min(samples, T)
            s = int(sum(int(tb[(i * T) // k]) for i in range(k))) if k else 0
            out.append(X + ((s * T + k // 2) // k if k else 0))
        return np.array(out, np.int64)

    got = gpu_estimate(w, cnt, 8)
    assert np.array_equal(got, expect(8))
    exact = gpu_estimate(w, cnt, 1 << 20)
    assert np.array_equal(exact, expect(1 << 20))
    _, sizes = zc.compress(torch.from_numpy(w.view(np.int16)).to(DEV), cnt)
    real = sizes.cpu().numpy()
    assert np.array_equal(exact, real)
    assert abs(int(got.sum()) - int(real.sum())) / int(real.sum()) < 0.02
