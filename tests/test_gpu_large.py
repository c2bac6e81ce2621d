"""GPU parity at the largest sizes the launch plan accepts.

- an output of more than 2^31 elements (every output offset is 64-bit), with
  M and N both ragged against the 128 x 128 tile;
- the largest row-tile grid the planner lets through (grid y = 65535, so
  M = 65535 * 128 rows); one more row tile is refused (host test).

The activations (several GB) are drawn on the device by a seeded generator;
the q8_1 bytes of the sampled rows are checked bit-exactly against the
oracle's quantize of the same fp32 rows, and the sampled output rows against
the oracle's GEMM within the 1e-5 tolerance (Q8_0 bit-identical).  Every
output starts as NaN and no NaN may remain anywhere.
"""
import sys

import numpy as np
import pytest
import torch

import block_quantized_int8_q8_amd as mmq
import oracle
from block_quantized_int8_q8_amd import inputs
from tests import metrics

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

WEIGHTS = {mmq.FMT_Q8_0: inputs.q8_0_weights, mmq.FMT_Q4_K: inputs.q4_K_weights}
GEMM = {mmq.FMT_Q8_0: mmq.gemm_q8_0, mmq.FMT_Q4_K: mmq.gemm_q4_K}
ORACLE = {mmq.FMT_Q8_0: oracle.gemm_q8_0, mmq.FMT_Q4_K: oracle.gemm_q4_K}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run_and_check(fmt, M, N, K, seed, rows):
    _say(f"large fmt={fmt} M={M} N={N} K={K}")
    x = inputs.activations_device(M, K, seed, DEV)
    xq = mmq.quantize_q8_1(x)
    w = WEIGHTS[fmt](N, K, seed + 1)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    GEMM[fmt](xq, torch.from_numpy(w).to(DEV), M, N, K, out)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out).any()), "an output element was never written"
    idx = torch.tensor(rows, dtype=torch.int64, device=DEV)
    xq_ref = oracle.quantize_q8_1(x.index_select(0, idx).cpu().numpy())
    assert np.array_equal(xq.index_select(0, idx).cpu().numpy(), xq_ref)
    ref = ORACLE[fmt](xq_ref, w, len(rows), N, K, nthreads=16)
    rep = metrics.report(out.index_select(0, idx).cpu().numpy(), ref)
    _say(rep)
    assert rep["normalized_max_error"] <= metrics.TOL
    if fmt == mmq.FMT_Q8_0:
        assert rep["bit_identical_fraction"] == 1.0
    del x, xq, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K])
def test_output_past_2_31_elements(fmt):
    M, N, K = 131073, 16400, 256          # 1025 row tiles (one row in the last), 129 column tiles (16 in the last)
    assert M * N > 2 ** 31
    cross = -(-(2 ** 31) // N)            # first row whose output offset passes 2^31
    rng = np.random.default_rng(11)
    rows = sorted({0, 1, cross - 1, cross, M // 2, M - 129, M - 128, M - 2, M - 1}
                  | set(int(r) for r in rng.integers(0, M, 6)))
    _run_and_check(fmt, M, N, K, 8100 + fmt, rows)


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K])
def test_largest_row_tile_grid(fmt):
    M, N, K = 65535 * 128, 130, 256
    ok, desc = mmq.plan_describe(fmt, M, N, K)
    assert ok and "grid=2x65535" in desc, desc
    rng = np.random.default_rng(12)
    rows = sorted({0, 127, 128, M // 2, M - 129, M - 128, M - 1} | set(int(r) for r in rng.integers(0, M, 6)))
    _run_and_check(fmt, M, N, K, 8200 + fmt, rows)
