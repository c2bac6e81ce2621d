"""Pins of the oracle's Q6_K path (reading R22: the GGUF layout of a format
the pages name with 16-element scale groups and 6-bit codes centred at 32,
"When Does a Kernel Win Surface?", section 4.1; term per group R23).

Pins, none of which reuses the oracle's code:
  * the code and scale of every element position against an independent
    numpy decode;
  * one-hot low bytes and high bits that move exactly one code, by the
    amount the layout gives them;
  * each scale byte scales exactly its 16 elements;
  * group dots == int64 numpy sums of the decoded, centred codes;
  * fp32 outputs within the fp32 accumulation bound of the exact fp64 sum;
  * the hand-summed fixture in tests/golden/gemm_hand.json, exactly;
  * codes all 32 give exactly zero; a planted misreading of the high-bit
    order changes the fixture's value.
"""
import numpy as np
import pytest

import oracle
from block_quantized_int8_q8_amd import inputs
from tests import golden_cases, npdecode

U = 2.0 ** -24


def test_codes_and_scales_match_numpy_decode():
    w = inputs.q6_K_weights(2, 256, 1)
    d, sc, codes = npdecode.q6_K_fields(w)
    for n in range(2):
        for e in range(256):
            assert oracle.q6k_code(w[n, 0], e) == codes[n, 0, e]
        for g in range(16):
            assert oracle.q6k_scale(w[n, 0], g) == sc[n, 0, g]
    deq = np.stack([oracle.dequant_q6_K_block(w[n, 0]) for n in range(2)]).astype(np.float64)
    assert np.array_equal(deq, npdecode.dequant_q6_K(w))   # fp16 x int8 x 6-bit: exact in fp32


@pytest.mark.parametrize("h,r,l", [(0, 0, 0), (0, 1, 31), (1, 0, 7), (1, 1, 16)])
def test_one_hot_low_byte(h, r, l):
    """Low byte 64h + 32r + l: its low nibble is element 128h + 32r + l, its
    high nibble element 128h + 32(r + 2) + l."""
    w = inputs.q6_K_weights(1, 256, 2, low_byte=0, high_byte=0)
    assert all(oracle.q6k_code(w[0, 0], e) == 0 for e in range(256))
    for val, e in ((0x01, 128 * h + 32 * r + l), (0x10, 128 * h + 32 * (r + 2) + l)):
        v = w.copy()
        v[0, 0, 64 * h + 32 * r + l] = val
        got = np.array([oracle.q6k_code(v[0, 0], i) for i in range(256)])
        assert got[e] == 1 and np.count_nonzero(got) == 1


@pytest.mark.parametrize("h,q,l", [(0, 0, 0), (0, 3, 31), (1, 1, 5), (1, 2, 20)])
def test_one_hot_high_bits(h, q, l):
    """Bits 2q and 2q+1 of high byte 128 + 32h + l are bits 4 and 5 of
    element 128h + 32q + l."""
    w = inputs.q6_K_weights(1, 256, 3, low_byte=0, high_byte=0)
    for bit, add in ((2 * q, 16), (2 * q + 1, 32)):
        v = w.copy()
        v[0, 0, 128 + 32 * h + l] = 1 << bit
        got = np.array([oracle.q6k_code(v[0, 0], i) for i in range(256)])
        assert got[128 * h + 32 * q + l] == add and np.count_nonzero(got) == 1


@pytest.mark.parametrize("g", [0, 1, 7, 8, 15])
def test_scale_byte_covers_its_sixteen_elements(g):
    w = inputs.q6_K_weights(1, 256, 4, scale_value=0, d_value=1.0)
    w[0, 0, 192 + g] = 1
    deq = oracle.dequant_q6_K_block(w[0, 0])
    nz = np.flatnonzero(deq)
    codes = np.array([oracle.q6k_code(w[0, 0], e) for e in range(256)])
    expect = [e for e in range(16 * g, 16 * g + 16) if codes[e] != 32]
    assert list(nz) == expect


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (5, 3, 512), (16, 9, 1024)])
def test_group_dots_brute_force(M, N, K):
    x = inputs.q8_1_blocks(M, K, 1900 + K)
    w = inputs.q6_K_weights(N, K, 1910 + K)
    _, _, xq = npdecode.q8_1_fields(x)
    _, _, codes = npdecode.q6_K_fields(w)
    a = xq.reshape(M, K // 16, 16)
    b = (codes - 32).reshape(N, K // 16, 16)
    assert np.array_equal(oracle.group_dots_q6_K(x, w, M, N, K), np.einsum("mgi,ngi->mng", a, b))


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (3, 5, 512), (16, 8, 1024)])
def test_gemm_vs_fp64(M, N, K):
    x = oracle.quantize_q8_1(inputs.activations(M, K, 1920 + K))
    w = inputs.q6_K_weights(N, K, 1930 + K)
    out = oracle.gemm_q6_K(x, w, M, N, K)
    xd, _, xq = npdecode.q8_1_fields(x)
    d, sc, codes = npdecode.q6_K_fields(w)
    ng = K // 16
    I = np.einsum("mgi,ngi->mng", xq.reshape(M, ng, 16), (codes - 32).reshape(N, ng, 16))
    ws = (d[..., None] * sc).reshape(N, ng)
    terms = np.repeat(xd, 2, axis=1)[:, None, :] * ws[None] * I
    exact = terms.sum(-1)
    err = np.abs(out.astype(np.float64) - exact)
    assert (err <= (ng + 2) * U * np.abs(terms).sum(-1) + 1e-300).all()
    # the same value as the fully dequantized product, in exact arithmetic
    pure = npdecode.dequant_q8_1(x) @ npdecode.dequant_q6_K(w).T
    assert np.allclose(exact, pure, rtol=0, atol=1e-9 * np.abs(terms).sum(-1).max())


def test_gemm_hand_case():
    x, w, K, expect = golden_cases.gemm_q6_K_case()
    xq = oracle.quantize_q8_1(x)
    assert oracle.gemm_q6_K(xq, w, 1, 1, K)[0, 0] == expect


def test_centre_codes_give_zero():
    """Every code 32 (low bits 0, high bit pairs 2 = byte 0xAA): all centred
    codes are 0, so every output is exactly +0 whatever the scales."""
    M, N, K = 4, 3, 512
    x = oracle.quantize_q8_1(inputs.activations(M, K, 1940))
    w = inputs.q6_K_weights(N, K, 1941, low_byte=0, high_byte=0xAA)
    out = oracle.gemm_q6_K(x, w, M, N, K)
    assert np.array_equal(out.view(np.uint32), np.zeros_like(out.view(np.uint32)))


def test_planted_high_bit_misreading_changes_the_fixture():
    """Reading the high-bit pairs from the top down (bits 6-2q, 7-2q) gives
    the hand fixture another value, so the fixture pins the order."""
    x, w, K, expect = golden_cases.gemm_q6_K_case()
    _, sc, codes = npdecode.q6_K_fields(w)
    lo = codes & 15
    qh = w[0, 0, 128:192].astype(np.int64).reshape(2, 32)
    wrong_hi = np.stack([(qh >> (6 - 2 * q)) & 3 for q in range(4)], axis=-2).reshape(256)
    wrong = lo.reshape(256) + 16 * wrong_hi
    d = 0.5
    val = sum(127.0 * (d * sc[0, 0, g]) * (wrong[16 * g] - 32) for g in range(16))
    assert val != expect


def test_moe_accepts_q6_K():
    T, E, topk, N, K = 9, 3, 2, 5, 256
    x = oracle.quantize_q8_1(inputs.activations(T, K, 1970))
    w = inputs.q6_K_weights(E * N, K, 1971)
    ids = inputs.moe_ids(T, E, topk, 1972)
    out = oracle.moe_gemm(3, x, w, ids, topk, T, N, K, E)
    for r in range(T * topk):
        e = int(ids.reshape(-1)[r])
        ref = oracle.gemm_q6_K(x[r // topk: r // topk + 1], w.reshape(E, N, 1, 210)[e], 1, N, K)
        assert np.array_equal(out[r].view(np.uint32), ref[0].view(np.uint32))
