"""Pins for the oracle's exponent extraction and byte grouping.

The reorder is checked against the IEEE field definitions through math.frexp
and numpy's sign bit (textbook float decomposition, independent of the
oracle's bit formula), and shown to be a bijection exhaustively on 16-bit
patterns.
"""
import math

import numpy as np
import pytest
import torch

import oracle

BF16, FP16, FP32, U8 = 1, 2, 3, 0


@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_reorder_bijective_16bit(dtype):
    ys = [oracle.reorder(dtype, x) for x in range(1 << 16)]
    assert len(set(ys)) == 1 << 16 and max(ys) < (1 << 16)
    assert all(oracle.unreorder(dtype, y) == x for x, y in enumerate(ys))


def test_reorder_u8_identity():
    assert all(oracle.reorder(U8, x) == x for x in range(256))


def test_reorder_fp32_bijective_sample():
    rng = np.random.default_rng(11)
    xs = list(rng.integers(0, 1 << 32, 20000, dtype=np.uint64)) + [
        0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x00000001, 0x807FFFFF, 0xFFFFFFFF]
    for x in xs:
        y = oracle.reorder(FP32, int(x))
        assert oracle.unreorder(FP32, y) == int(x)
    ys = {oracle.reorder(FP32, int(x)) for x in xs}
    assert len(ys) == len(set(int(x) for x in xs))


def _fields_from_frexp(v, mant_bits):
    """(biased exponent, sign, mantissa integer) of a normal float by frexp."""
    m, e = math.frexp(abs(v))          # |v| = m * 2**e, m in [0.5, 1)
    bias = (1 << {7: 7, 10: 4, 23: 7}[mant_bits]) - 1  # 127, 15, 127
    biased = e - 1 + bias
    frac = int(round((2 * m - 1) * (1 << mant_bits)))
    return biased, int(math.copysign(1, v) < 0), frac


def test_bf16_streams_are_ieee_fields():
    vals = torch.tensor([1.0, -2.0, 0.02, -3.5e-3, 1e-30, 6.0e4, -1.7e38, 0.75],
                        dtype=torch.bfloat16)
    bits = vals.view(torch.int16).numpy().view(np.uint16)
    for v, x in zip(vals.float().tolist(), bits):
        y = oracle.reorder(BF16, int(x))
        e, s, m = _fields_from_frexp(v, 7)
        assert y >> 8 == e            # stream 1: the biased exponent byte
        assert (y >> 7) & 1 == s      # sign just below it
        assert y & 0x7F == m          # mantissa untouched


def test_fp16_streams_are_ieee_fields():
    vals = np.array([1.0, -2.0, 0.02, -3.5e-3, 6.0e4, 0.75, -1e-4], dtype=np.float16)
    for v, x in zip(vals.astype(np.float64), vals.view(np.uint16)):
        y = oracle.reorder(FP16, int(x))
        e, s, m = _fields_from_frexp(float(v), 10)
        assert y >> 11 == e and (y >> 10) & 1 == s and y & 0x3FF == m


def test_fp32_streams_are_ieee_fields():
    rng = np.random.default_rng(3)
    vals = (rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000)).astype(np.float32)
    for v, x in zip(vals.astype(np.float64), vals.view(np.uint32)):
        y = oracle.reorder(FP32, int(x))
        e, s, m = _fields_from_frexp(float(v), 23)
        assert y >> 24 == e and (y >> 23) & 1 == s and y & 0x7FFFFF == m


def test_chunk_streams_bf16_match_numpy_fields():
    """Stream 1 = biased exponent (np.frexp), stream 0 = sign<<7 | top mantissa bits."""
    x = torch.randn(5000, dtype=torch.float32).mul_(0.02).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    f = x.float().numpy().astype(np.float64)
    m, e = np.frexp(np.abs(f))
    normal = f != 0
    exp_field = np.where(normal, e + 126, 0)
    frac = np.where(normal, np.rint((2 * m - 1) * 128), 0).astype(np.int64)
    sign = np.signbit(f).astype(np.int64)
    C = 2048  # 1024 elements per chunk, last chunk shorter (5000 = 4*1024 + 904)
    for c in range(5):
        lo, hi = c * 1024, min(5000, (c + 1) * 1024)
        s0 = oracle.chunk_stream(bits, BF16, C, c, 0)
        s1 = oracle.chunk_stream(bits, BF16, C, c, 1)
        assert s0.size == s1.size == hi - lo
        assert np.array_equal(s1, exp_field[lo:hi].astype(np.uint8))
        assert np.array_equal(s0, (sign[lo:hi] << 7 | frac[lo:hi]).astype(np.uint8))


def test_histogram_is_bincount():
    rng = np.random.default_rng(5)
    s = rng.integers(0, 256, 100001).astype(np.uint8)
    assert np.array_equal(oracle.histogram(s), np.bincount(s, minlength=256))
    assert oracle.histogram(s).sum() == s.size
