"""zc_compress_noalloc (compress with the library's own per-GPU workspace)
against zc_compress, through the C ABI: two calls in a row, the second with
a smaller input, each byte-identical to zc_compress's streams and sizes and
decoding back to its input; then a request beyond the array's limit is
refused before any work is queued."""
import numpy as np
import pytest
import torch

from lossless_bf16_tensor_sign_amd import synth, zc

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TILE = 8192


def _one(w, counts):
    counts = np.asarray(counts, np.int64)
    x = torch.from_numpy(w.view(np.int16)).to(DEV)
    cap = zc.zc_bound(counts)
    ref, ref_sizes = zc.compress(x, counts)
    out = torch.zeros(cap, dtype=torch.uint8, device=DEV)
    sizes = torch.full((len(counts),), -7, dtype=torch.int64, device=DEV)
    assert zc.zc_compress_noalloc(x, counts, out, sizes) == zc.ZC_OK
    torch.cuda.synchronize()
    s, rs = sizes.cpu().numpy(), ref_sizes.cpu().numpy()
    assert np.array_equal(s, rs)
    off = np.concatenate([[0], np.cumsum([zc.zc_bound([c]) for c in counts])])[:-1]
    o, r = out.cpu().numpy(), ref.cpu().numpy()
    for c in range(len(counts)):
        assert np.array_equal(o[off[c]:off[c] + s[c]], r[off[c]:off[c] + s[c]]), c
    y, st = zc.decompress(out, counts)
    assert int(st.item()) == 0 and torch.equal(y, x)


def test_noalloc_matches_workspace_call_twice():
    # first call: many tiles in 70 chunks (two launches); second: fewer tiles,
    # so most status words it reads were written by the first call
    rng = np.random.default_rng(5)
    big = rng.integers(0, 40 * TILE, 70).astype(np.int64)
    big[::9] = 0
    w1 = synth.gaussian_bits(int(big.sum()), 0.02, seed=51)
    w1[::613] = 0
    _one(w1, big)
    small = np.array([3 * TILE + 5, 17, 0, TILE], np.int64)
    w2 = synth.gaussian_bits(int(small.sum()), 0.01, seed=52)
    _one(w2, small)


def test_noalloc_full_fsdp_shard():
    w, cnt = synth.make(2, workers=8)
    _one(w, cnt)


def test_noalloc_refuses_beyond_its_array():
    cnt = np.full(64, 1 << 24, np.int64)     # 131 072 tiles in one launch
    assert zc.zc_workspace_bytes(cnt) > 4 << 20
    x = torch.empty(8, dtype=torch.int16, device=DEV)
    out = torch.empty(16, dtype=torch.uint8, device=DEV)
    sizes = torch.empty(64, dtype=torch.int64, device=DEV)
    assert zc.zc_compress_noalloc(x, cnt, out, sizes) == zc.ZC_ENOSPC
