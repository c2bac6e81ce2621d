"""Pin the oracle's reading of the Q4_K super-block layout.

The pages name the 6-bit scale/min helper of the K-quant format and the
144-byte super-block (d @0, dmin @2, scales @4, codes @16: "13 . r7-r8
raw-byte MMQ kernel", section 3.2) but do not print the bit packing; the
oracle takes the GGUF K-quant packing.  These tests pin that the packer and
unpacker are inverse bijections, that every 6-bit field is addressed, and
where each 4-bit code lives, against the independent numpy decoder.
"""
import numpy as np
import pytest

import oracle
from block_quantized_int8_q8_amd import inputs
from tests import npdecode


def test_block_sizes():
    assert inputs.q8_0_weights(1, 32, 0).shape == (1, 1, 34)
    assert inputs.q8_1_blocks(1, 32, 0).shape == (1, 1, 36)
    assert inputs.q4_K_weights(1, 256, 0).shape == (1, 1, 144)
    assert oracle.quantize_q8_1(np.ones((1, 32), np.float32)).shape == (1, 1, 36)


@pytest.mark.parametrize("j", range(8))
def test_scale_min_each_field_each_value(j):
    rng = np.random.default_rng(j)
    for v in range(64):
        sc = rng.integers(0, 64, 8).astype(np.uint8)
        mn = rng.integers(0, 64, 8).astype(np.uint8)
        sc[j] = v
        mn[(j + 3) % 8] = 63 - v
        s12 = oracle.q4k_pack_scale_min(sc, mn)
        for jj in range(8):
            assert oracle.q4k_scale_min(s12, jj) == (sc[jj], mn[jj])


def test_random_blobs_unpack_pack_identity():
    """All 96 bits are used, so unpack then pack restores any 12 bytes."""
    rng = np.random.default_rng(1)
    for _ in range(2000):
        s12 = rng.integers(0, 256, 12).astype(np.uint8)
        vals = [oracle.q4k_scale_min(s12, j) for j in range(8)]
        sc = np.array([a for a, _ in vals], np.uint8)
        mn = np.array([b for _, b in vals], np.uint8)
        assert np.array_equal(oracle.q4k_pack_scale_min(sc, mn), s12)


def test_scale_min_matches_numpy_decoder():
    w = inputs.q4_K_weights(64, 1024, 5)
    _, _, sc, mn, _ = npdecode.q4_K_fields(w)
    for n in range(64):
        for sb in range(4):
            for j in range(8):
                assert oracle.q4k_scale_min(w[n, sb, 4:16], j) == (sc[n, sb, j], mn[n, sb, j])


def test_out_of_range_scale_rejected():
    with pytest.raises(ValueError):
        oracle.q4k_pack_scale_min(np.full(8, 64, np.uint8), np.zeros(8, np.uint8))


def test_one_hot_code_placement():
    """A single non-zero nibble at byte p (low or high) is element
    64*(p//32) + p%32 (+32 for the high nibble) and no other."""
    for p in range(128):
        for high in (0, 1):
            blk = np.zeros(144, np.uint8)
            blk[16 + p] = (0x7 << 4) if high else 0x7
            codes = np.array([oracle.q4k_code(blk, e) for e in range(256)])
            e0 = 64 * (p // 32) + p % 32 + 32 * high
            expect = np.zeros(256, int)
            expect[e0] = 7
            assert np.array_equal(codes, expect), (p, high)
            assert np.array_equal(npdecode.q4_K_fields(blk[None])[4][0], expect)


def test_dequant_q4_K_block_closed_form():
    sc = np.arange(8, dtype=np.uint8) * 7 + 3
    mn = (60 - np.arange(8) * 5).astype(np.uint8)
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.array([0.5], "<f2").view(np.uint8)      # d
    blk[2:4] = np.array([0.25], "<f2").view(np.uint8)     # dmin
    blk[4:16] = oracle.q4k_pack_scale_min(sc, mn)
    blk[16:144] = (np.arange(128) * 37 % 256).astype(np.uint8)
    w = oracle.dequant_q4_K_block(blk)
    codes = npdecode.q4_K_fields(blk[None])[4][0]
    j = np.arange(256) // 32
    assert np.array_equal(w.astype(np.float64), 0.5 * sc[j] * codes - 0.25 * mn[j])
    assert np.array_equal(npdecode.dequant_q4_K(blk[None, None])[0], 0.5 * sc[j] * codes - 0.25 * mn[j])


def test_generator_fields_have_the_documented_distributions():
    w = inputs.q4_K_weights(256, 2048, 4)
    d, dmin, sc, mn, codes = npdecode.q4_K_fields(w)
    assert 9e-4 < d.min() and d.max() < 1.01e-2
    assert 0 <= dmin.min() and dmin.max() < 1.01e-2
    for a, top in ((sc, 63), (mn, 63), (codes, 15)):
        assert a.min() == 0 and a.max() == top
        counts = np.bincount(a.ravel(), minlength=top + 1)
        assert counts.min() > 0.8 * counts.mean()
    q = inputs.q8_0_weights(128, 1024, 4)
    qd, qq = npdecode.q8_0_fields(q)
    assert qq.min() == -127 and qq.max() == 127
    assert 9e-4 < qd.min() and qd.max() < 1.01e-2
