"""The oracle against the hand-derived fixtures in tests/golden/."""
import numpy as np

import oracle
from tests import golden_cases, npdecode


def test_q8_1_hand_blocks():
    x, d_bits, s_bits, codes = golden_cases.q8_1_blocks()
    y = oracle.quantize_q8_1(x.reshape(1, -1))[0]
    assert np.array_equal(y[:, 0:2].copy().view("<u2")[:, 0], d_bits)
    assert np.array_equal(y[:, 2:4].copy().view("<u2")[:, 0], s_bits)
    assert np.array_equal(y[:, 4:].view(np.int8).astype(np.int64), codes)


def test_gemm_hand_cases():
    x, w, K, expect = golden_cases.gemm_q8_0_case()
    assert oracle.gemm_q8_0(oracle.quantize_q8_1(x), w, 1, 1, K)[0, 0] == expect
    x, w, K, expect = golden_cases.gemm_q4_K_case()
    _, _, sc, mn, codes = npdecode.q4_K_fields(w)
    assert (sc == 2).all() and (mn == 3).all() and (codes == 5).all()
    assert oracle.gemm_q4_K(oracle.quantize_q8_1(x), w, 1, 1, K)[0, 0] == expect
    x, w, K, expect = golden_cases.gemm_q5_K_case()
    codes = npdecode.q5_K_fields(w)[4].reshape(8, 32)
    assert (codes[0::2, 0] == 5).all() and (codes[1::2, 0] == 21).all()
    assert oracle.gemm_q5_K(oracle.quantize_q8_1(x), w, 1, 1, K)[0, 0] == expect
