"""Pin the oracle's fp32 -> q8_1 activation quantization.

The quantize pass ("13 . r7-r8 raw-byte MMQ kernel", section 3.2; the q8_1
format in "When Does a Kernel Win Surface?", section 6.2) maps each
32-value block to d = amax/127, codes = round(x * (1/d)) and a block sum.
The pins are closed forms on hand-built blocks (zero, one-hot, constant,
integer-valued, exact ties), a scaling law, and bounds on random data.
"""
import numpy as np
import pytest

import oracle
from tests import npdecode


def _q(block):
    return oracle.quantize_q8_1(np.asarray(block, np.float32).reshape(1, 32))[0, 0]


def _fields(y):
    d, s, q = npdecode.q8_1_fields(y[None, None])
    return d[0, 0], s[0, 0], q[0, 0]


def test_zero_block():
    y = _q(np.zeros(32))
    assert not y.any()                       # d = s = +0, all codes 0


@pytest.mark.parametrize("v", [1.0, -3.5, 1e-3, 6.0e4, -2.0 ** -20])
@pytest.mark.parametrize("i", [0, 13, 31])
def test_one_nonzero(v, i):
    x = np.zeros(32, np.float32)
    x[i] = v
    d, s, q = _fields(_q(x))
    expect = np.zeros(32, np.int64)
    expect[i] = 127 if v > 0 else -127
    assert np.array_equal(q, expect)
    d32 = np.float32(abs(np.float32(v))) / np.float32(127)
    assert d == np.float64(np.float16(d32))
    assert s == np.float64(np.float16(d32 * np.float32(expect[i])))


@pytest.mark.parametrize("c", [0.37, -12.0, 1e-6])
def test_constant_block(c):
    d, s, q = _fields(_q(np.full(32, c)))
    assert (q == (127 if c > 0 else -127)).all()


def test_integer_block_with_amax_127_is_identity():
    rng = np.random.default_rng(3)
    for _ in range(50):
        x = rng.integers(-127, 127, 32, endpoint=True).astype(np.float32)
        x[rng.integers(32)] = 127 * rng.choice([-1, 1])
        d, s, q = _fields(_q(x))
        assert d == 1.0                         # 127/127
        assert np.array_equal(q, x.astype(np.int64))
        assert s == np.float64(np.float16(np.float32(q.sum())))


@pytest.mark.parametrize("e", [-10, -3, 0, 4])
def test_exact_ties_round_half_away(e):
    """d = 2^e exactly when amax = 127 * 2^e; then x = (k + 1/2) d lands on a
    tie that half-away rounding sends to k+1 (ties-to-even would give k for
    even k)."""
    scale = np.float32(2.0 ** e)
    k = np.arange(31)                            # 0..30
    sign = np.where(k % 3 == 0, -1, 1)
    x = np.empty(32, np.float32)
    x[:31] = sign * (k + 0.5) * scale
    x[31] = 127 * scale
    d, s, q = _fields(_q(x))
    assert d == float(scale)
    assert np.array_equal(q[:31], sign * (k + 1))
    assert q[31] == 127
    rint = np.rint(x[:31] / scale)
    assert (rint != sign * (k + 1)).any()         # the case really separates the two rules


def test_scaling_by_power_of_two():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    y0 = oracle.quantize_q8_1(x)
    y1 = oracle.quantize_q8_1(x * np.float32(4.0))
    d0, s0, q0 = npdecode.q8_1_fields(y0)
    d1, s1, q1 = npdecode.q8_1_fields(y1)
    assert np.array_equal(q0, q1)
    assert np.array_equal(d1, 4 * d0) and np.array_equal(s1, 4 * s0)


def test_random_invariants_and_roundtrip_bound():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((256, 512)) * rng.uniform(0.01, 100, (256, 1))).astype(np.float32)
    y = oracle.quantize_q8_1(x)
    d, s, q = npdecode.q8_1_fields(y)
    xb = x.reshape(256, 16, 32).astype(np.float64)
    amax = np.abs(xb).max(-1)
    assert (np.abs(q) <= 127).all()
    assert ((np.abs(q).max(-1) == 127) == (amax > 0)).all()
    # the fp32 scale that quantized is amax/127; its fp16 copy is stored
    d32 = (amax.astype(np.float32) / np.float32(127))
    assert np.array_equal(d, d32.astype(np.float16).astype(np.float64))
    assert np.array_equal(s, (d32 * q.sum(-1).astype(np.float32)).astype(np.float16).astype(np.float64))
    # each code is within half a step of x/d (up to the fp32 reciprocal's error)
    r = xb / d32[..., None].astype(np.float64)
    assert (np.abs(r - q) <= 0.5 + 127 * 2.0 ** -22).all()
    # round trip through the stored fp16 scale
    err = np.abs(xb - d[..., None] * q)
    assert (err <= d32[..., None] * (0.5 + 127 * 2.0 ** -11) + 1e-30).all()


def test_clamp_never_binds():
    """|x * (1/d)| <= 127 (1 + 2^-22) for finite x, so codes stay in [-127, 127]."""
    rng = np.random.default_rng(9)
    x = rng.uniform(-1, 1, (4096, 32)).astype(np.float32)
    x[np.arange(4096), rng.integers(0, 32, 4096)] = np.float32(1.0)
    d32 = np.abs(x).max(-1) / np.float32(127)
    v = x * (np.float32(1) / d32)[:, None]
    assert (np.abs(v) <= 127 * (1 + 2.0 ** -22)).all()
    q = npdecode.q8_1_fields(oracle.quantize_q8_1(x.reshape(1, -1)))[2]
    assert np.abs(q).max() == 127


def test_non_finite_rejected():
    x = np.zeros((1, 32), np.float32)
    x[0, 5] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize_q8_1(x)
    x[0, 5] = np.nan
    with pytest.raises(ValueError):
        oracle.quantize_q8_1(x)


def test_block_independence_and_layout():
    """Each 36-byte block depends only on its own 32 inputs, in row-major order."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 96)).astype(np.float32)
    y = oracle.quantize_q8_1(x)
    for m in range(3):
        for b in range(3):
            assert np.array_equal(y[m, b], _q(x[m, 32 * b:32 * b + 32]))


@pytest.mark.parametrize("amax", [1e-39, 1e-38, 3.0e-37])
def test_reciprocal_overflow_block_is_zero(amax):
    """amax/127 below 1/FLT_MAX makes 1/d overflow; such a block quantizes
    like the zero block (codes 0, s = 0) and its fp16 d is 0."""
    x = (np.linspace(-1, 1, 32) * amax).astype(np.float32)
    assert np.isinf(np.float32(1) / (np.abs(x).max() / np.float32(127)))
    y = _q(x)
    assert not y.any()


def test_just_above_reciprocal_overflow_has_codes():
    x = (np.linspace(-1, 1, 32) * 1e-36).astype(np.float32)
    d, s, q = _fields(_q(x))
    assert d == 0.0 and q[0] == -127 and q[-1] == 127
