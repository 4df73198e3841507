"""Pins of the oracle's reduce-scatter receive step (ordered fp32 sum of
decoded bf16 contributions), against facts fixed by IEEE 754 arithmetic and
closed forms, not against a re-typing of the loop."""
import numpy as np
import pytest

BF16_ONE = 0x3F80


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def test_small_integers_sum_exactly(oracle):
    # contribution c is the value c + 1 at every position: the sum is the
    # triangular number C (C + 1) / 2, exact in fp32
    C, n = 64, 37
    vals = np.arange(1, C + 1, dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)   # exact in bf16 (<= 8 bits)
    x = np.repeat(bits, n)
    out = oracle.reduce_bf16_f32(x, n, C)
    assert np.all(out == C * (C + 1) / 2)


def test_chunk_order_is_fixed(oracle):
    # 2^24, 1, -2^24: in chunk order 2^24 + 1 rounds back to 2^24 (tie to
    # even), so the sum is 0; adding 1 - 2^24 first would give 1
    x = np.array([0x4B80, 0x3F80, 0xCB80], np.uint16)
    assert f32_bits(oracle.reduce_bf16_f32(x, 1, 3))[0] == 0
    # the reverse chunk order keeps the 1
    assert oracle.reduce_bf16_f32(x[::-1].copy(), 1, 3)[0] == 1.0


def test_signed_zeros_and_one_chunk(oracle):
    # the sum starts at +0: +0 + (-0) = +0 under round-to-nearest
    neg0 = np.full(4, 0x8000, np.uint16)
    out = oracle.reduce_bf16_f32(neg0, 1, 4)
    assert f32_bits(out)[0] == 0x00000000
    # one contribution: the fp32 value of the bf16 pattern (widened exactly),
    # except -0 which becomes +0
    pats = np.arange(65536, dtype=np.uint16)
    out = oracle.reduce_bf16_f32(pats, 65536, 1)
    want = pats.astype(np.uint32) << 16
    want[pats == 0x8000] = 0
    nan = np.isnan(out)
    assert np.array_equal(nan, ((pats & 0x7F80) == 0x7F80) & ((pats & 0x7F) != 0))
    assert np.array_equal(f32_bits(out)[~nan], want[~nan])


def test_infinities_and_subnormals(oracle):
    inf, ninf = 0x7F80, 0xFF80
    out = oracle.reduce_bf16_f32(np.array([inf, ninf], np.uint16), 1, 2)
    assert np.isnan(out[0])
    out = oracle.reduce_bf16_f32(np.array([inf, BF16_ONE, BF16_ONE], np.uint16), 1, 3)
    assert out[0] == np.inf
    # the smallest bf16 subnormal, 2^-133, summed 64 times: 2^-127, exact
    # (no flush of subnormals to zero)
    out = oracle.reduce_bf16_f32(np.full(64, 0x0001, np.uint16), 1, 64)
    assert out[0] == np.float32(2.0 ** -127)


# ---- fp32 -> bf16 rounding (round to nearest, ties to even) and the bf16 sum

def f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def test_rounding_hand_cases(oracle):
    cases = {
        0x3F800000: 0x3F80,   # 1.0 exact
        0x3F808000: 0x3F80,   # 1 + 2^-8: halfway, 1.0 has the even last bit
        0x3F818000: 0x3F82,   # 1 + 3 * 2^-8: halfway, rounds up to the even one
        0x3F808001: 0x3F81,   # just above halfway
        0x3F807FFF: 0x3F80,   # just below halfway
        0xBF808001: 0xBF81,   # sign is kept
        0x7F7F7FFF: 0x7F7F,   # below the overflow midpoint: largest finite
        0x7F7F8000: 0x7F80,   # the overflow midpoint ties to infinity (even)
        0xFF7F8000: 0xFF80,
        0x7F800000: 0x7F80,   # infinities and zeros stay
        0xFF800000: 0xFF80,
        0x80000000: 0x8000,
        0x00008000: 0x0000,   # halfway to the smallest bf16 subnormal: to even 0
        0x00018000: 0x0002,   # halfway between subnormals 1 and 2: to even 2
        0x7FC00001: 0x7FC0,   # NaNs become the quiet NaN
        0xFF800001: 0x7FC0,
    }
    got = oracle.f32_to_bf16(f32(list(cases)))
    assert [hex(v) for v in got] == [hex(v) for v in cases.values()]


def test_rounding_keeps_every_bf16_value(oracle):
    b = np.arange(1 << 16, dtype=np.uint32)
    got = oracle.f32_to_bf16(f32(b << 16)).astype(np.uint32)
    nan = ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    assert np.array_equal(got[~nan], b[~nan])
    assert np.all(got[nan] == 0x7FC0)


def test_rounding_matches_torch_cpu_conversion(oracle):
    # torch's CPU float32 -> bfloat16 conversion rounds to nearest even; on
    # random bit patterns and near-halfway values the two must agree (NaN
    # only as NaN)
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    u = rng.integers(0, 1 << 32, 60000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 1 << 16, 20000, dtype=np.uint32) << 16) | 0x8000
    near = ties + rng.integers(-2, 3, 20000).astype(np.int64).astype(np.uint32)
    bits = np.concatenate([u, ties, near])
    x = f32(bits)
    got = oracle.f32_to_bf16(x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    isnan = np.isnan(x)
    assert np.array_equal(got[~isnan], want[~isnan])
    assert np.all(got[isnan] == 0x7FC0)


def test_bf16_sum_rounds_once_at_the_end(oracle):
    # 1 + 2^-8 + 2^-8: the fp32 sum is 1 + 2^-7 exactly, one bf16 step above
    # 1.0; rounding after every addition would have kept 1.0 (each partial
    # sum 1 + 2^-8 is a tie that goes to the even 1.0)
    x = np.array([BF16_ONE, 0x3B80, 0x3B80], np.uint16)
    assert oracle.reduce_bf16_bf16(x, 1, 3)[0] == 0x3F81
    assert oracle.reduce_bf16_bf16(x[:2].copy(), 1, 2)[0] == 0x3F80   # a tie: to even 1.0
    # a sum past the largest bf16 rounds to infinity
    big = np.array([0x7F7F, 0x7F7F], np.uint16)
    assert oracle.reduce_bf16_bf16(big, 1, 2)[0] == 0x7F80
