"""GPU checks of the tile-packed Q8_0 path (mmq_pack_q8_0, mmq_gemm_q8_0_packed).

The pack kernel's bytes must equal the numpy model of the header's layout
(tests/nppack.py) byte for byte.  The packed GEMM computes the row-major Q8_0
GEMM's arithmetic in the same order, so its output is held to the oracle by
the same bars as mmq_gemm_q8_0 ("When the Product Won't Collapse", section 2:
1e-5 by the normalized measure, bit-identical where K is not split) and is
bit-identical to mmq_gemm_q8_0 wherever that call also runs the tile kernel.
Outputs start as NaN, so an element never written fails.
"""
import re
import sys

import numpy as np
import pytest
import torch

import block_quantized_int8_q8_amd as mmq
import oracle
from block_quantized_int8_q8_amd import inputs
from tests import metrics, nppack

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
Q8 = mmq.FMT_Q8_0


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _nan(M, N):
    return torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)


def _plan(M, N, K):
    """(kernel, split_k) of the row-major call for this shape."""
    d = mmq.plan_describe(Q8, M, N, K)[1]
    return re.search(r"kernel=(\w+)", d).group(1), int(re.search(r"split_k=(\d+)", d).group(1))


@pytest.mark.parametrize("N,K", [(1, 32), (127, 96), (128, 128), (300, 544), (129, 3616), (3584, 3584)])
def test_pack_matches_layout(N, K):
    _say(f"pack N={N} K={K}")
    w = inputs.q8_0_weights(N, K, 40 + N)
    nb = mmq.packed_bytes_q8_0(N, K)
    packed = torch.full((nb,), 0x5A, dtype=torch.uint8, device=DEV)   # every byte must be written
    mmq.pack_q8_0(_dev(w), N, K, packed)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), nppack.pack(w, N, K))


@pytest.mark.parametrize("M,N,K", [(200, 300, 768), (300, 130, 2048), (2000, 300, 512),
                                   (250, 257, 96), (300, 200, 3616),          # K % 128 != 0: partial last k-step
                                   (96, 33000, 512),                          # idle wave rows, wide N
                                   (200, 64, 3584), (200, 100, 18944),        # split K
                                   (1, 1, 32), (5, 300, 512), (129, 257, 1024), (33, 517, 256)])
def test_packed_gemm_matches_oracle_and_row_major(M, N, K):
    _say(f"packed gemm M={M} N={N} K={K}")
    x = inputs.activations(M, K, 60 + M)
    xq = oracle.quantize_q8_1(x)
    w = inputs.q8_0_weights(N, K, 70 + N)
    xq_d, w_d = _dev(xq), _dev(w)
    packed = mmq.pack_q8_0(w_d, N, K)
    out = _nan(M, N)
    mmq.gemm_q8_0_packed(xq_d, packed, M, N, K, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert not np.isnan(got).any(), "output element left unwritten"
    ref = oracle.gemm_q8_0(xq, w, M, N, K, nthreads=16)
    rep = metrics.report(got, ref)
    assert rep["normalized_max_error"] <= metrics.TOL, rep
    kernel, split = _plan(M, N, K)
    if kernel == "mmq":
        # the row-major call plans the same tile kernel: same split, same bits
        if split == 1:
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
        row = _nan(M, N)
        mmq.gemm_q8_0(xq_d, w_d, M, N, K, row)
        torch.cuda.synchronize()
        assert np.array_equal(got.view(np.uint32), row.cpu().numpy().view(np.uint32))


def test_packed_headline_shape_full_output():
    """2048 x 3584 x 3584 (the benchmarked shape): quantize and packed GEMM on
    the device, every output element against the oracle (bit-identical) and
    against the row-major GEMM."""
    fmt_name, M, N, K = inputs.CONFIGS[2]
    assert fmt_name == "q8_0"
    _say(f"packed headline M={M} N={N} K={K}")
    x = inputs.activations(M, K, inputs.seed_for(2, 0))
    w = inputs.q8_0_weights(N, K, inputs.seed_for(2, 1))
    xq_d = mmq.quantize_q8_1(_dev(x))
    w_d = _dev(w)
    packed = mmq.pack_q8_0(w_d, N, K)
    out = _nan(M, N)
    mmq.gemm_q8_0_packed(xq_d, packed, M, N, K, out)
    row = _nan(M, N)
    mmq.gemm_q8_0(xq_d, w_d, M, N, K, row)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), row.cpu().numpy().view(np.uint32))
    xq = oracle.quantize_q8_1(x)
    assert np.array_equal(xq_d.cpu().numpy(), xq)
    ref = oracle.gemm_q8_0(xq, w, M, N, K, nthreads=16)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_packed_refusals_leave_output_untouched():
    _say("packed refusals")
    import ctypes
    M, N, K = 64, 130, 512
    xq = _dev(inputs.q8_1_blocks(M, K, 1))
    w = _dev(inputs.q8_0_weights(N, K, 2))
    nb = mmq.packed_bytes_q8_0(N, K)
    packed = torch.full((nb,), 0x5A, dtype=torch.uint8, device=DEV)
    L = mmq.lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    # the library's own checks (the binding would stop these first)
    assert L.mmq_pack_q8_0(p(w), N, K, p(packed), nb - 1, s) == 0
    assert "needs" in mmq.last_error()
    assert L.mmq_pack_q8_0(p(w), N, K - 16, p(packed), nb, s) == 0
    assert "multiple of 32" in mmq.last_error()
    assert L.mmq_pack_q8_0(None, N, K, p(packed), nb, s) == 0
    torch.cuda.synchronize()
    assert (packed == 0x5A).all()
    mmq.pack_q8_0(w, N, K, packed)
    out = _nan(M, N)
    with pytest.raises(mmq.MMQError, match="multiple of 32"):
        mmq.gemm_q8_0_packed(xq, packed, M, N, K - 16, out)
    with pytest.raises(mmq.MMQError, match=">= 1"):
        mmq.gemm_q8_0_packed(xq, packed, 0, N, K, out)
    try:
        mmq.set_extra_lds(200 * 1024)
        with pytest.raises(mmq.MMQError, match="LDS"):
            mmq.gemm_q8_0_packed(xq, packed, M, N, K, out)
    finally:
        mmq.set_extra_lds(0)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    mmq.gemm_q8_0_packed(xq, packed, M, N, K, out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()


def test_packed_graph_replays_match_eager():
    """Pack once, then the packed GEMM captured in a HIP graph: every replay
    (with eager work between them) equals the eager output."""
    _say("packed graph replay")
    M, N, K = 300, 640, 1024
    xq = _dev(oracle.quantize_q8_1(inputs.activations(M, K, 5)))
    packed = mmq.pack_q8_0(_dev(inputs.q8_0_weights(N, K, 6)), N, K)
    eager = _nan(M, N)
    mmq.gemm_q8_0_packed(xq, packed, M, N, K, eager)
    torch.cuda.synchronize()
    out = _nan(M, N)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            mmq.gemm_q8_0_packed(xq, packed, M, N, K, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32))
