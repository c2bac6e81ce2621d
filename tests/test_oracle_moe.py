"""Pins of the oracle's indexed-MoE GEMM ("When Does a Kernel Win Surface?",
section 4.5, fused indexed-MoE prefill GEMM: each routed row is its token's activations
times the weights of the expert it was routed to).

The MoE-specific part of the oracle is indexing (token = r // topk, expert =
ids[r], expert-major weight storage); these tests pin it against an
independent numpy decoding with fp64 products, a reduction to the dense GEMM,
an invariance under relabelling the experts, and a planted mistake.
"""
import numpy as np
import pytest

import oracle
from block_quantized_int8_q8_amd import inputs
from tests import npdecode

U = 2.0 ** -24


def _experts(fmt, E, N, K, seed):
    gen = inputs.q8_0_weights if fmt == 0 else inputs.q4_K_weights
    return np.stack([gen(N, K, seed + e) for e in range(E)])          # [E, N, blocks, bytes]


@pytest.mark.parametrize("fmt,K", [(0, 64), (0, 256), (1, 256), (1, 512)])
def test_moe_vs_fp64_dequant_brute_force(fmt, K):
    T, E, topk, N = 5, 4, 3, 7
    x = oracle.quantize_q8_1(inputs.activations(T, K, 11 + K))
    w = _experts(fmt, E, N, K, 40)
    ids = inputs.moe_ids(T, E, topk, 12 + K)
    out = oracle.moe_gemm(fmt, x, w, ids, topk, T, N, K, E)
    deq = npdecode.dequant_q8_0 if fmt == 0 else npdecode.dequant_q4_K
    xdq = npdecode.dequant_q8_1(x)                                     # [T, K] fp64
    for r in range(T * topk):
        t, e = r // topk, ids.reshape(-1)[r]
        wdq = deq(w[e])                                                # [N, K] fp64
        exact = wdq @ xdq[t]
        absterm = np.abs(wdq) @ np.abs(xdq[t])
        bound = (K // 32 + 2) * U * absterm * (4 if fmt == 1 else 1) + 1e-300
        # Q4_K: the min term goes through the stored fp16 block sum
        if fmt == 1:
            xd, xs, xq = npdecode.q8_1_fields(x[t:t + 1])
            _, dmin, _, mn, _ = npdecode.q4_K_fields(w[e])
            dm = (dmin[..., None] * mn).reshape(N, -1)
            bound = bound + (np.abs(dm) * np.abs(xs - xd * xq.sum(-1))).sum(-1) * (1 + 1e-12)
        assert (np.abs(out[r].astype(np.float64) - exact) <= bound).all(), (r, t, e)


@pytest.mark.parametrize("fmt,K", [(0, 256), (1, 512)])
def test_one_expert_is_the_dense_gemm_of_repeated_rows(fmt, K):
    T, topk, N = 6, 2, 9
    x = oracle.quantize_q8_1(inputs.activations(T, K, 21))
    w = _experts(fmt, 1, N, K, 50)
    ids = np.zeros((T, topk), np.int32)
    out = oracle.moe_gemm(fmt, x, w, ids, topk, T, N, K, 1)
    dense = (oracle.gemm_q8_0 if fmt == 0 else oracle.gemm_q4_K)(np.repeat(x, topk, axis=0), w[0],
                                                                   T * topk, N, K)
    assert np.array_equal(out, dense)


def test_relabelling_experts_changes_nothing():
    fmt, T, E, topk, N, K = 1, 8, 6, 3, 5, 256
    x = oracle.quantize_q8_1(inputs.activations(T, K, 31))
    w = _experts(fmt, E, N, K, 60)
    ids = inputs.moe_ids(T, E, topk, 32)
    perm = np.random.default_rng(33).permutation(E)            # new label of old expert e = perm[e]
    w2 = np.empty_like(w)
    w2[perm] = w
    a = oracle.moe_gemm(fmt, x, w, ids, topk, T, N, K, E)
    b = oracle.moe_gemm(fmt, x, w2, perm[ids].astype(np.int32), topk, T, N, K, E)
    assert np.array_equal(a, b)


def test_planted_mistake_swapped_experts_is_caught():
    fmt, T, E, topk, N, K = 0, 4, 3, 2, 6, 256
    x = oracle.quantize_q8_1(inputs.activations(T, K, 41))
    w = _experts(fmt, E, N, K, 70)
    ids = np.array([[0, 1], [1, 2], [2, 0], [0, 2]], np.int32)
    good = oracle.moe_gemm(fmt, x, w, ids, topk, T, N, K, E)
    bad = oracle.moe_gemm(fmt, x, w[[1, 0, 2]], ids, topk, T, N, K, E)
    routed = np.isin(ids.reshape(-1), [0, 1])
    assert not np.array_equal(good[routed], bad[routed])
    assert np.array_equal(good[~routed], bad[~routed])


def test_row_subset_and_bad_ids():
    fmt, T, E, topk, N, K = 1, 7, 5, 2, 4, 256
    x = oracle.quantize_q8_1(inputs.activations(T, K, 51))
    w = _experts(fmt, E, N, K, 80)
    ids = inputs.moe_ids(T, E, topk, 52)
    full = oracle.moe_gemm(fmt, x, w, ids, topk, T, N, K, E)
    rows = [0, 3, 13]
    assert np.array_equal(oracle.moe_gemm(fmt, x, w, ids, topk, T, N, K, E, rows=rows), full[rows])
    bad = ids.copy()
    bad[2, 1] = E
    with pytest.raises(ValueError):
        oracle.moe_gemm(fmt, x, w, bad, topk, T, N, K, E)


def test_routing_generator():
    ids = inputs.moe_ids(300, 16, 4, 7)
    assert ids.shape == (300, 4) and ids.dtype == np.int32
    assert all(len(set(r)) == 4 for r in ids)                  # distinct experts per token
    assert ids.min() >= 0 and ids.max() < 16
    skew = np.bincount(inputs.moe_ids(4000, 16, 2, 8, skew=1.5).ravel(), minlength=16)
    assert skew[0] > 3 * skew[-1]                              # skewed toward low expert ids
