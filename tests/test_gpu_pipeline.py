"""GPU tests of zc_pipeline, the chunk-pipelined compress -> link ->
decompress exchange (ZipCCL abstract, technique (2); pith.science, Figure 5
and Figure 14 caption).  On one GPU a device copy carries each group's
streams from the sender's slots to the receiver's.

Checked on every case: the decoded values equal the input bit for bit;
each chunk's stream in the send buffer equals the oracle's stream for that
chunk byte for byte (and so the single-call zc_compress output); the receive
buffer holds exactly those bytes in the same slots and nothing beyond them
(it starts zeroed); the status word stays 0.  Streams: three distinct torch
streams at default priority, and all three equal.
"""
import numpy as np
import pytest
import torch

from lossless_bf16_tensor_sign_amd import synth, zc
from tests import oracle_pool

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print("[pipeline] " + msg, flush=True)


def check(oracle, w, counts, groups, streams):
    counts = np.asarray(counts, np.int64)
    say("%d chunks %s, %d groups, %s streams" % (len(counts), counts.tolist()[:8], groups,
                                                   "three" if streams else "one"))
    x = torch.from_numpy(w.view(np.int16)).to(DEV)
    y, status, send, recv, sizes = zc.pipeline(x, counts, groups, streams=streams)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(y.cpu().numpy().view(np.uint16), w)
    s = send.cpu().numpy()
    r = recv.cpu().numpy()
    g_sizes = sizes.cpu().numpy()[:len(counts)]
    off, total = oracle.slot_offsets(counts)
    vo = np.concatenate([[0], np.cumsum(counts)])
    for c in range(len(counts)):
        ref = oracle.compress_chunk(w[vo[c]:vo[c + 1]])
        assert g_sizes[c] == ref.size, (c, g_sizes[c], ref.size)
        assert np.array_equal(s[off[c]:off[c] + ref.size], ref), c
        assert np.array_equal(r[off[c]:off[c] + ref.size], ref), c
        end = off[c + 1] if c + 1 < len(counts) else total
        assert not r[off[c] + ref.size:end].any(), c    # nothing past the stream


def three_streams():
    return tuple(torch.cuda.Stream(device=DEV) for _ in range(3))


@pytest.mark.parametrize("groups", [1, 2, 3, 7])
def test_ragged_chunks(oracle, groups):
    counts = [20000, 0, 8192, 5, 16384 + 17, 1, 40000]
    w = synth.gaussian_bits(int(sum(counts)), 0.02, seed=11)
    w[::997] = 0x7FC0                     # NaNs: raw groups and escapes
    w[5::1013] = 0x0000
    check(oracle, w, counts, groups, three_streams())


def test_one_stream_and_all_raw(oracle):
    counts = [8192 * 3, 8192, 8192 * 2 + 100]
    rng = np.random.default_rng(12)
    w = rng.integers(0, 1 << 16, size=int(sum(counts)), dtype=np.uint16)
    check(oracle, w, counts, 3, None)


def test_many_chunks_one_group_each(oracle):
    counts = [8192 * 2] * 64 + [333]      # more than one launch of 64 chunks
    w = synth.gaussian_bits(int(sum(counts)), 0.01, seed=13)
    check(oracle, w, counts, 65, three_streams())


def test_full_fsdp_shape(oracle):
    # the FSDP all-gather shard (64 x 4 Mi) in 8 groups: every value is
    # checked by the round trip, and every chunk's stream in the send and in
    # the receive buffer against the oracle
    w, counts = synth.make(2, workers=8)
    counts = np.asarray(counts, np.int64)
    x = torch.from_numpy(w.view(np.int16)).to(DEV)
    say("fsdp 64 x 4 Mi, 8 groups")
    y, status, send, recv, sizes = zc.pipeline(x, counts, 8, streams=three_streams())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(y, x)
    off, _ = oracle.slot_offsets(counts)
    g_sizes = sizes.cpu().numpy()
    say("oracle comparison of both buffers")
    oracle_pool.compare_chunks(oracle, w, counts, send.cpu().numpy(), g_sizes, off, label="send")
    oracle_pool.compare_chunks(oracle, w, counts, recv.cpu().numpy(), g_sizes, off, label="recv")
