"""HIP graph capture of the codec calls.

A training step that compresses a gradient bucket and decodes what it
receives can be captured once and replayed.  The calls only launch kernels:
no allocation, no memset and no host synchronisation.  The look-back
workspace keeps its launch tag on the device, so every replay tags its own
status words, also when eager calls share the workspace between replays.

Each replay is checked against the eager result of the same call, with eager
work on the same buffers between replays: the outputs are cleared, and an
eager compress runs on the shared workspace.
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


def _gradient_bucket():
    # chunks of the gradient workload (escape steps and raw groups in most
    # tiles), cut to ragged lengths: whole tiles, a chunk-end tile and a
    # chunk of less than one tile
    cnt = np.array([1 << 20, (1 << 20) - 77, 3 * 8192 + 5, 1000, 1 << 20], np.int64)
    parts = [synth.chunk(3, c)[:int(n)] for c, n in enumerate(cnt)]
    w = np.concatenate(parts)
    return torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(DEV), cnt


def _capture(run):
    # warm up on a side stream, then capture (the usual torch pattern)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    return g


def test_graph_replays_compress_and_decompress():
    x, cnt = _gradient_bucket()
    bound = zc.zc_bound(cnt)
    total = int(cnt.sum())

    # eager reference
    ws_e = torch.zeros(zc.zc_workspace_bytes(cnt), dtype=torch.uint8, device=DEV)
    out_e = torch.zeros(bound, dtype=torch.uint8, device=DEV)
    sizes_e = torch.zeros(len(cnt), dtype=torch.int64, device=DEV)
    assert zc.zc_compress(x, cnt, out_e, sizes_e, ws_e) == zc.ZC_OK

    # static buffers of the captured step
    ws = torch.zeros(zc.zc_workspace_bytes(cnt), dtype=torch.uint8, device=DEV)
    out = torch.zeros(bound, dtype=torch.uint8, device=DEV)
    sizes = torch.zeros(len(cnt), dtype=torch.int64, device=DEV)
    y = torch.zeros(total, dtype=torch.int16, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def step():
        assert zc.zc_compress(x, cnt, out, sizes, ws) == zc.ZC_OK
        assert zc.zc_decompress(out, cnt, y, status) == zc.ZC_OK

    say("graph capture: compress + decompress, %d chunks" % len(cnt))
    g = _capture(step)
    other = torch.zeros(bound, dtype=torch.uint8, device=DEV)
    other_sizes = torch.zeros(len(cnt), dtype=torch.int64, device=DEV)
    for r in range(4):
        out.zero_()
        sizes.zero_()
        y.zero_()
        status.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, r
        assert torch.equal(sizes, sizes_e), r
        assert torch.equal(out, out_e), r
        assert torch.equal(y, x), r
        # eager work between replays, on the captured step's workspace
        assert zc.zc_compress(x, cnt, other, other_sizes, ws) == zc.ZC_OK
        torch.cuda.synchronize()
        assert torch.equal(other, out_e), r


@pytest.mark.parametrize("n", [(1 << 20) + 8192 + 33, 512 * 8192])
@pytest.mark.parametrize("bf16", [False, True])
def test_graph_replays_decode_sum(bf16, n):
    # the receive side of a compressed reduce-scatter: 8 contributions of one
    # shard, decoded and summed in chunk order (a ragged shard in slabs, and
    # one of 512 tiles decoded and summed in one kernel)
    c = 8
    w = np.concatenate([synth.chunk(3, i)[:n] for i in range(c)])
    x = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(DEV)
    cnt = np.full(c, n, np.int64)
    buf, _ = zc.compress(x, cnt)
    ref, st = zc.decompress_reduce(buf, n, c, bf16=bf16)
    assert int(st.item()) == 0

    scratch = torch.empty(max(zc.zc_reduce_scratch_bytes(n, c), 16), dtype=torch.uint8, device=DEV)
    out = torch.zeros(max(n, 8), dtype=torch.int16 if bf16 else torch.float32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def step():
        assert zc.zc_decompress_reduce(buf, n, c, out, status, scratch, bf16=bf16) == zc.ZC_OK

    say("graph capture: decode + sum, %d x %d, bf16=%s" % (c, n, bf16))
    g = _capture(step)
    bits = (lambda t: t) if bf16 else (lambda t: t.view(torch.int32))
    for r in range(3):
        out.zero_()
        scratch.fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, r
        assert torch.equal(bits(out[:n]), bits(ref)), r
