"""Pin the oracle's software binary16 conversions to library routines.

f16 -> f32 is checked on all 65,536 bit patterns against numpy; f32 -> f16
on all 2^32 bit patterns against torch's CPU conversion (IEEE
round-to-nearest-even with gradual underflow), plus a stratified sample
against numpy so that the two libraries are seen to agree.
"""
import numpy as np
import pytest
import torch

import oracle


def _is_nan16(h):
    return ((h & 0x7C00) == 0x7C00) & ((h & 0x03FF) != 0)


def test_f16_to_f32_all_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = _is_nan16(h)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.isnan(ours[nan]).all()
    assert np.array_equal(np.signbit(ours[nan]), np.signbit(ref[nan]))


def test_f32_to_f16_known_values():
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF),
        (65519.996, 0x7BFF), (65520.0, 0x7C00), (1e9, 0x7C00), (2.0 ** -14, 0x0400),
        (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (2.0 ** -25 * 1.0000001, 0x0001),
        (3 * 2.0 ** -25, 0x0002), (1.0 + 2.0 ** -11, 0x3C00), (1.0 + 3 * 2.0 ** -11, 0x3C02),
        (float("inf"), 0x7C00), (float("-inf"), 0xFC00),
    ]
    for v, bits in cases:
        assert oracle.lib().oracle_f32_to_f16(np.float32(v)) == bits, v


@pytest.mark.slow
def test_f32_to_f16_all_patterns_vs_torch():
    chunk = 1 << 24
    base = np.arange(chunk, dtype=np.uint32)
    for c in range(1 << 8):
        bits = base + np.uint32(c * chunk)
        f = bits.view(np.float32)
        ours = oracle.f32_to_f16_bits(f)
        ref = torch.from_numpy(f).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(f)
        if nan.any():
            assert _is_nan16(ours[nan]).all()
            assert np.array_equal(ours[nan] >> 15, ref[nan] >> 15)
        ok = np.array_equal(ours[~nan], ref[~nan])
        if not ok:
            bad = np.nonzero(ours[~nan] != ref[~nan])[0][:5]
            raise AssertionError(f"chunk {c}: {bits[~nan][bad]} -> {ours[~nan][bad]} vs {ref[~nan][bad]}")


def test_f32_to_f16_sample_vs_numpy():
    rng = np.random.default_rng(7)
    # every exponent, random mantissas and signs, plus the halfway patterns
    exps = np.repeat(np.arange(256, dtype=np.uint32), 512)
    mans = rng.integers(0, 1 << 23, exps.size, dtype=np.uint32)
    mans[::4] = (mans[::4] & ~np.uint32(0x1FFF)) | np.uint32(0x1000)   # exact ties at half precision
    signs = rng.integers(0, 2, exps.size, dtype=np.uint32) << np.uint32(31)
    bits = signs | (exps << np.uint32(23)) | mans
    f = bits.view(np.float32)
    keep = ~np.isnan(f)
    ours = oracle.f32_to_f16_bits(f[keep])
    ref = f[keep].astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
