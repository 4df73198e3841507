"""The host cost model of the compressed/plain switch (zc_switch_decide).

The pages name the switch (abstract, technique (3); pith.science, Figure 15
caption) but give no model, so these tests pin the model's structure: a
worked example done by hand, the break-even link speed where the two times
meet, and the cases where the answer is fixed whatever the numbers.
"""
import math

import pytest

from lossless_bf16_tensor_sign_amd import zc

COLLS = ["allgather", "reduce_scatter", "alltoall"]


def decide(coll, ranks=8, nbytes=1e9, comp=0.7e9, link=100.0, lat=10.0, rc=2300.0,
           rd=2300.0, rr=1500.0):
    st, r = zc.zc_switch_decide(coll, ranks, nbytes, comp, link, lat, rc, rd, rr)
    assert st == zc.ZC_OK
    return r


def test_worked_example_allgather():
    # 8 ranks, 1 GB buffer compressed to 0.7 GB, 100 GB/s link, 10 us steps,
    # codec 2300 GB/s both ways.  By hand:
    #   wire        7/8 GB = 0.875 GB -> 8750 us plain, 0.6125 GB -> 6125 us
    #   steps       7 x 10 us = 70 us
    #   codec       own shard 0.125 GB / 2300 GB/s = 54.348 us
    #               7 shards 0.875 GB / 2300 GB/s = 380.435 us
    #   break-even  0.2625 GB / 434.783 us = 603.75 GB/s
    r = decide("allgather")
    assert r["plain_us"] == pytest.approx(8820.0, rel=1e-12)
    assert r["compressed_us"] == pytest.approx(70 + 6125 + 54.347826 + 380.434783, rel=1e-8)
    assert r["breakeven_GBps"] == pytest.approx(603.75, rel=1e-9)
    assert r["use_compressed"]


def test_worked_example_reduce_scatter():
    # 64 ranks, the same buffer, 50 GB/s link: all-to-all then decode + sum.
    #   wire        63/64 GB = 0.984375 GB -> 19687.5 us, compressed 13781.25 us
    #   steps       63 x 10 us = 630 us
    #   codec       1 GB / 2300 GB/s + 1 GB / 1500 GB/s = 434.783 + 666.667 us
    r = decide("reduce_scatter", ranks=64, link=50.0)
    assert r["plain_us"] == pytest.approx(20317.5, rel=1e-12)
    assert r["compressed_us"] == pytest.approx(630 + 13781.25 + 434.782609 + 666.666667,
                                               rel=1e-8)
    assert r["breakeven_GBps"] == pytest.approx(0.29531250e9 / 1101.449275e-6 / 1e9, rel=1e-8)


@pytest.mark.parametrize("coll", COLLS)
@pytest.mark.parametrize("ranks", [2, 8, 64])
def test_times_meet_at_the_breakeven_link(coll, ranks):
    b = decide(coll, ranks=ranks)["breakeven_GBps"]
    assert 0 < b < math.inf
    at = decide(coll, ranks=ranks, link=b)
    assert at["plain_us"] == pytest.approx(at["compressed_us"], rel=1e-9)
    assert decide(coll, ranks=ranks, link=b * (1 - 1e-6))["use_compressed"]
    assert not decide(coll, ranks=ranks, link=b * (1 + 1e-6))["use_compressed"]


@pytest.mark.parametrize("coll", COLLS)
def test_decision_is_monotone_in_link_speed(coll):
    flips = 0
    prev = True
    for link in [1, 3, 10, 30, 100, 300, 1000, 3000, 10000]:
        now = decide(coll, link=link)["use_compressed"]
        assert not (now and not prev), "compression may only stop paying as the link gets faster"
        flips += now != prev
        prev = now
    assert flips == 1


@pytest.mark.parametrize("coll", COLLS)
@pytest.mark.parametrize("comp", [1e9, 1.2e9])
def test_no_gain_without_a_smaller_stream(coll, comp):
    r = decide(coll, comp=comp, link=0.001)
    assert r["breakeven_GBps"] == 0.0
    assert not r["use_compressed"]


@pytest.mark.parametrize("coll", COLLS)
def test_step_latency_does_not_move_the_breakeven(coll):
    a = decide(coll, lat=0.0)
    b = decide(coll, lat=500.0)
    assert a["breakeven_GBps"] == pytest.approx(b["breakeven_GBps"], rel=1e-12)
    assert (b["plain_us"] - a["plain_us"]) == pytest.approx(7 * 500.0, rel=1e-12)


def test_faster_codec_raises_the_breakeven():
    slow = decide("alltoall", rc=500, rd=500)["breakeven_GBps"]
    fast = decide("alltoall", rc=5000, rd=5000)["breakeven_GBps"]
    assert fast == pytest.approx(10 * slow, rel=1e-12)


def test_single_rank_moves_nothing():
    r = decide("allgather", ranks=1)
    assert r["plain_us"] == 0.0 and not r["use_compressed"]


@pytest.mark.parametrize("args", [
    dict(coll=7), dict(ranks=0), dict(nbytes=-1.0), dict(nbytes=math.nan),
    dict(comp=0.0), dict(comp=math.inf), dict(link=0.0), dict(link=math.inf),
    dict(lat=-1.0), dict(rc=0.0), dict(coll="allgather", rd=0.0),
    dict(coll="reduce_scatter", rr=0.0),
])
def test_invalid_arguments(args):
    a = dict(coll="alltoall", ranks=8, nbytes=1e9, comp=0.7e9, link=100.0, lat=10.0,
             rc=2300.0, rd=2300.0, rr=1500.0)
    a.update(args)
    st, _ = zc.zc_switch_decide(a["coll"], a["ranks"], a["nbytes"], a["comp"], a["link"],
                                a["lat"], a["rc"], a["rd"], a["rr"])
    assert st == zc.ZC_EINVAL
