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
