"""The allocation-free indexed-MoE entry point, mmq_moe_gemm_noalloc: the
routing tables live in the library's static device scratch instead of a
caller workspace.  Its output must equal mmq_moe_gemm's (the same kernels on
the same tables: bit for bit) on two calls in a row, the second with a
smaller input, so that the second call reads nothing the first one left;
and both must meet the oracle's bar.  Also run alone in a fresh process."""
import ctypes
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


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _weights(fmt, E, N, K, seed):
    f = {mmq.FMT_Q8_0: inputs.q8_0_weights, mmq.FMT_Q4_K: inputs.q4_K_weights,
         mmq.FMT_Q5_K: inputs.q5_K_weights}[fmt]
    return f(E * N, K, seed)


def _noalloc_c_abi(fmt, xq, w, E, ids, topk, T, N, K, out):
    """Straight through the C ABI (ctypes), no binding helper in between."""
    L = mmq.lib()
    p = ctypes.c_void_p
    rc = L.mmq_moe_gemm_noalloc(fmt, p(xq.data_ptr()), p(w.data_ptr()), E, p(ids.data_ptr()), topk,
                                p(out.data_ptr()), T, N, K, p(torch.cuda.current_stream().cuda_stream))
    return rc


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K, mmq.FMT_Q5_K])
def test_noalloc_equals_workspace_entry_point(fmt):
    # (T, E, topk, N, K): the second call is smaller in every dimension
    calls = [(300, 16, 4, 256, 512), (37, 5, 3, 130, 256)]
    for i, (T, E, topk, N, K) in enumerate(calls):
        _say(f"no-alloc MoE fmt={fmt} call {i}: T={T} E={E} topk={topk} N={N} K={K}")
        xq_h = oracle.quantize_q8_1(inputs.activations(T, K, 400 + 10 * i + fmt))
        w_h = _weights(fmt, E, N, K, 401 + 10 * i)
        ids_h = inputs.moe_ids(T, E, topk, 402 + 10 * i, skew=1.0).astype(np.int32)
        xq, w, ids = _dev(xq_h), _dev(w_h), _dev(ids_h)
        ref = torch.full((T * topk, N), float("nan"), dtype=torch.float32, device=DEV)
        mmq.moe_gemm(fmt, xq, w, E, ids, topk, T, N, K, ref)
        got = torch.full((T * topk, N), float("nan"), dtype=torch.float32, device=DEV)
        assert _noalloc_c_abi(fmt, xq, w, E, ids, topk, T, N, K, got) == 1, mmq.last_error()
        torch.cuda.synchronize()
        g, r = got.cpu().numpy(), ref.cpu().numpy()
        assert not np.isnan(g).any(), "routed row left unwritten"
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32))
        rep = metrics.report(g, oracle.moe_gemm(fmt, xq_h, w_h, ids_h, topk, T, N, K, E, nthreads=16))
        _say(rep)
        assert rep["normalized_max_error"] <= metrics.TOL
        if fmt == mmq.FMT_Q8_0:
            assert rep["bit_identical_fraction"] == 1.0


def test_noalloc_refuses_beyond_its_scratch():
    fmt, E, topk, N, K = mmq.FMT_Q8_0, 4, 8, 32, 32
    T = mmq.MOE_NOALLOC_MAX_ROUTED // topk + 1
    _say(f"no-alloc MoE refusal: T*topk={T * topk}")
    xq = torch.zeros((T, 1, 36), dtype=torch.uint8, device=DEV)
    w = torch.zeros((E * N * 34,), dtype=torch.uint8, device=DEV)
    ids = torch.zeros((T, topk), dtype=torch.int32, device=DEV)
    out = torch.full((T * topk, N), float("nan"), dtype=torch.float32, device=DEV)
    assert _noalloc_c_abi(fmt, xq, w, E, ids, topk, T, N, K, out) == 0
    assert "exceeds the static scratch" in mmq.last_error()
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    # the largest accepted size launches
    T = mmq.MOE_NOALLOC_MAX_ROUTED // topk
    xq, ids = xq[:T], ids[:T]
    out = torch.full((T * topk, N), float("nan"), dtype=torch.float32, device=DEV)
    assert mmq.moe_gemm_noalloc(fmt, xq, w, E, ids, topk, T, N, K, out) is out
    torch.cuda.synchronize()
    assert (out == 0).all()
