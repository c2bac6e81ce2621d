"""Seeded random shapes through whichever kernel the planner picks for them:
the matvecs (M <= 8), the batch-decode kernel (9 <= M <= 32, and row blocks
of 32 up to M = 192 for narrow GEMMs), the tile kernel (with and without
split-K) and GEMM sets mixing member widths.  Every output element must be
written and lie within the fp32 accumulation bound of the exact value (the
bound the oracle itself is pinned to), and within the 1e-5 normalized error
of the oracle where the output is large enough for its rms to set the
scale ("When the Product Won't Collapse", section 2: the block-scaled
contraction; any summation order of the block terms is admissible)."""
import numpy as np
import pytest
import torch

import block_quantized_int8_q8_amd as mmq
import oracle
from block_quantized_int8_q8_amd import inputs
from tests.test_gpu_parity import (_check_reordered, _kernel, _nan_out, _oracle_gemm, _run_gemm, _say, _to_dev,
                                   _weights)

pytestmark = pytest.mark.gpu


def _shape(r, fmt):
    # M drawn from each kernel's range in turn
    lo, hi = [(1, 9), (9, 33), (33, 129), (129, 400)][int(r.integers(0, 4))]
    M = int(r.integers(lo, hi))
    kb = int(r.integers(1, 40)) if fmt == mmq.FMT_Q8_0 else 8 * int(r.integers(1, 6))
    return M, 32 * kb


def _cases(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = int(r.integers(0, 4))
        M, K = _shape(r, fmt)
        out.append((i, fmt, M, int(r.integers(1, 700)), K))
    return out


@pytest.mark.parametrize("i,fmt,M,N,K", _cases(48, 20261203))
def test_random_shape_matches_oracle(i, fmt, M, N, K):
    _say(f"random shape {i}: fmt={fmt} M={M} N={N} K={K} kernel={_kernel(fmt, M, N, K)}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 400 + i))
    w = _weights(fmt, N, K, 500 + i)
    got = _run_gemm(fmt, xq, w, M, N, K)
    _check_reordered(fmt, got, _oracle_gemm(fmt, xq, w, M, N, K), xq, w, M, N, K)


def _set_cases(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = int(r.integers(0, 4))
        M, K = _shape(r, fmt)
        Ns = tuple(int(v) for v in r.integers(1, 400, int(r.integers(1, 5))))
        out.append((i, fmt, M, Ns, K))
    return out


@pytest.mark.parametrize("i,fmt,M,Ns,K", _set_cases(16, 20261204))
def test_random_set_matches_oracle(i, fmt, M, Ns, K):
    """A GEMM set of 1-4 members of random widths: each member written in
    full and within the bounds against the oracle."""
    _say(f"random set {i}: fmt={fmt} M={M} Ns={Ns} K={K} kernel={_kernel(fmt, M, sum(Ns), K)}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 600 + i))
    ws = [_weights(fmt, n, K, 700 + 10 * i + g) for g, n in enumerate(Ns)]
    outs = [_nan_out(M, n) for n in Ns]
    mmq.gemm_multi(fmt, _to_dev(xq), [_to_dev(w) for w in ws], list(Ns), M, K, outs)
    torch.cuda.synchronize()
    for n, w, o in zip(Ns, ws, outs):
        got = o.cpu().numpy()
        assert not np.isnan(got).any(), "output element left unwritten"
        _check_reordered(fmt, got, _oracle_gemm(fmt, xq, w, M, n, K), xq, w, M, n, K)
