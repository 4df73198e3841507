"""Child process of test_lookback_recompute_path (run with
ZC_LOOKBACK_SPIN_LIMIT set in its environment, which the library reads once
per process): compresses one layout on cuda:0 and compares every chunk with
the oracle, then checks the round trip.  Prints "lookback child ok"."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from lossless_bf16_tensor_sign_amd import synth, zc  # noqa: E402
from oracle import oracle  # noqa: E402
from tests import oracle_pool  # noqa: E402

TILE = 8192


def main(layout):
    if layout == "equal":
        cnt = np.full(8, 6 * TILE, np.int64)
    else:
        cnt = np.array([3, 40 * TILE + 5, 7 * TILE, 0, 2 * TILE + 1], np.int64)
    print("[child] spin limit %s, %s chunks %s" % (os.environ.get("ZC_LOOKBACK_SPIN_LIMIT"),
                                                  layout, cnt.tolist()), flush=True)
    w = synth.gaussian_bits(int(cnt.sum()), 0.02, seed=31)
    w[::997] = 0
    x = torch.from_numpy(w.view(np.int16)).to("cuda:0")
    buf, sizes = zc.compress(x, cnt)
    torch.cuda.synchronize()
    off, _ = oracle.slot_offsets(cnt)
    oracle_pool.compare_chunks(oracle, w, cnt, buf.cpu().numpy(), sizes.cpu().numpy(), off,
                               label="spin limit 0, " + layout)
    y, status = zc.decompress(buf, cnt)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(y.cpu().numpy().view(np.uint16), w)
    print("lookback child ok", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
