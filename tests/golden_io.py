"""Reader for the hand-derived golden stream files in tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    """Returns (values uint16[n], expected stream bytes uint8[length])."""
    n = None
    length = None
    vals = {}
    fills = []
    spans = []
    bfills = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            if key == "n":
                n = int(rest[0])
            elif key == "length":
                length = int(rest[0])
            elif key == "values":
                for i, v in enumerate(rest):
                    vals[i] = int(v, 16)
            elif key == "values_at":
                base = int(rest[0])
                for i, v in enumerate(rest[1:]):
                    vals[base + i] = int(v, 16)
            elif key == "value_fill":
                fills.append((int(rest[0]), int(rest[1]), int(rest[2], 16)))
            elif key == "at":
                spans.append((int(rest[0]), bytes.fromhex("".join(rest[1:]))))
            elif key == "fill":
                bfills.append((int(rest[0]), int(rest[1]), int(rest[2], 16)))
            else:
                raise ValueError("bad directive %r in %s" % (key, name))
    w = np.zeros(n, np.uint16)
    for i0, cnt, v in fills:
        w[i0:i0 + cnt] = v
    for i, v in vals.items():
        w[i] = v
    exp = np.zeros(length, np.uint8)
    for off, cnt, b in bfills:
        exp[off:off + cnt] = b
    for off, data in spans:
        exp[off:off + len(data)] = np.frombuffer(data, np.uint8)
    return w, exp


def names():
    return sorted(f for f in os.listdir(GOLDEN) if f.startswith("zcb1_"))
