"""GPU parity of the indexed-MoE GEMM ("When Does a Kernel Win Surface?",
section 4.5): mmq_moe_gemm against the oracle's oracle_moe_gemm on the same
seeded inputs.

Bars as for the dense GEMM: normalized error <= 1e-5, and Q8_0 and Q6_K
bit-identical (every routed row is computed by the dense kernel's arithmetic
in its order, wherever the routing places it: in a 128-row tile or in the
launch for small remainders, whose K-quant rows also follow the oracle's
order exactly).  Outputs start as a NaN sentinel, so a
routed row the kernel never wrote fails."""
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
         mmq.FMT_Q5_K: inputs.q5_K_weights, mmq.FMT_Q6_K: inputs.q6_K_weights}[fmt]
    return f(E * N, K, seed)   # E matrices of N rows, one after another


def _run(fmt, xq, w, E, ids, topk, T, N, K, out=None):
    if out is None:
        out = torch.full((T * topk, N), float("nan"), dtype=torch.float32, device=DEV)
    mmq.moe_gemm(fmt, _dev(xq), _dev(w), E, _dev(ids.astype(np.int32)), topk, T, N, K, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(fmt, got, ref):
    assert not np.isnan(got).any(), "routed row left unwritten"
    rep = metrics.report(got, ref)
    _say(rep)
    assert rep["normalized_max_error"] <= metrics.TOL
    if fmt in (mmq.FMT_Q8_0, mmq.FMT_Q6_K):
        assert rep["bit_identical_fraction"] == 1.0


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K, mmq.FMT_Q5_K, mmq.FMT_Q6_K])
@pytest.mark.parametrize("T,E,topk,N,K,skew", [
    (37, 8, 3, 200, 512, 0.0),      # ragged N, several experts per tile row
    (300, 16, 4, 130, 1024, 2.0),   # skewed: popular experts span several 128-row tiles
    (1, 8, 2, 256, 256, 0.0),       # one token (decode-sized)
    (129, 4, 4, 257, 768, 0.0),     # every token routed to every expert
    (700, 3, 1, 384, 256, 0.0),     # topk 1: plain row gather
])
def test_moe_matches_oracle(fmt, T, E, topk, N, K, skew):
    _moe_case(fmt, T, E, topk, N, K, skew)


@pytest.mark.parametrize("T,E,topk,N,K", [(37, 5, 3, 201, 288), (150, 4, 2, 131, 3616)])
def test_moe_q8_0_any_whole_blocks(T, E, topk, N, K):
    """Q8_0 with K/32 odd and N odd: every other expert's matrix starts 2
    bytes off the dword grid, and the last k-step holds fewer than 4 blocks."""
    _moe_case(mmq.FMT_Q8_0, T, E, topk, N, K, 0.0)


def _moe_case(fmt, T, E, topk, N, K, skew):
    _say(f"moe fmt={fmt} T={T} E={E} topk={topk} N={N} K={K} skew={skew}")
    xq = oracle.quantize_q8_1(inputs.activations(T, K, 50 + T))
    w = _weights(fmt, E, N, K, 60 + N)
    ids = inputs.moe_ids(T, E, topk, 70 + T, skew=skew)
    got = _run(fmt, xq, w, E, ids, topk, T, N, K)
    _check(fmt, got, oracle.moe_gemm(fmt, xq, w, ids, topk, T, N, K, E, nthreads=16))


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K])
def test_moe_one_expert_takes_all(fmt):
    """All 300 routed rows on expert 2 of 5 (three row tiles, one partial);
    the other experts empty."""
    T, E, topk, N, K = 300, 5, 1, 192, 512
    _say(f"moe one expert fmt={fmt}")
    xq = oracle.quantize_q8_1(inputs.activations(T, K, 81))
    w = _weights(fmt, E, N, K, 82)
    ids = np.full((T, topk), 2, np.int32)
    got = _run(fmt, xq, w, E, ids, topk, T, N, K)
    _check(fmt, got, oracle.moe_gemm(fmt, xq, w, ids, topk, T, N, K, E, nthreads=16))
    # equal to the dense GEMM with expert 2's matrix
    wrow = w.reshape(E, N, *w.shape[1:])[2]
    dense = mmq.gemm(fmt, _dev(xq), _dev(wrow), T, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint32), dense.cpu().numpy().view(np.uint32))


def test_moe_out_of_range_ids_leave_rows_untouched():
    fmt, T, E, topk, N, K = mmq.FMT_Q8_0, 90, 6, 2, 160, 256
    _say("moe out-of-range ids")
    xq = oracle.quantize_q8_1(inputs.activations(T, K, 91))
    w = _weights(fmt, E, N, K, 92)
    ids = inputs.moe_ids(T, E, topk, 93)
    bad = np.zeros(T * topk, bool)
    bad[[0, 5, 17, 179]] = True
    ids_bad = ids.reshape(-1).copy()
    ids_bad[[0, 5]] = -1
    ids_bad[[17, 179]] = E
    got = _run(fmt, xq, w, E, ids_bad.reshape(T, topk), topk, T, N, K)
    assert np.isnan(got[bad]).all()
    ref = oracle.moe_gemm(fmt, xq, w, ids, topk, T, N, K, E, nthreads=16)
    _check(fmt, got[~bad], ref[~bad])


def test_moe_workspace_reuse_and_refusals():
    fmt, E, N, K = mmq.FMT_Q8_0, 8, 128, 256
    _say("moe workspace reuse / refusals")
    big_T, small_T, topk = 400, 33, 2
    ws = torch.empty((mmq.moe_workspace_bytes(big_T, topk, E),), dtype=torch.uint8, device=DEV)
    w = _weights(fmt, E, N, K, 101)
    for T in (big_T, small_T):   # the second call reuses the first call's routing tables
        xq = oracle.quantize_q8_1(inputs.activations(T, K, 102 + T))
        ids = inputs.moe_ids(T, E, topk, 103 + T)
        out = torch.full((T * topk, N), float("nan"), dtype=torch.float32, device=DEV)
        mmq.moe_gemm(fmt, _dev(xq), _dev(w), E, _dev(ids), topk, T, N, K, out, workspace=ws)
        torch.cuda.synchronize()
        _check(fmt, out.cpu().numpy(), oracle.moe_gemm(fmt, xq, w, ids, topk, T, N, K, E, nthreads=16))
    # refusals launch nothing
    T = small_T
    xq = _dev(oracle.quantize_q8_1(inputs.activations(T, K, 104)))
    ids = _dev(inputs.moe_ids(T, E, topk, 105))
    out = torch.full((T * topk, N), float("nan"), dtype=torch.float32, device=DEV)
    short = torch.empty((mmq.moe_workspace_bytes(T, topk, E) - 16,), dtype=torch.uint8, device=DEV)
    # (the expert weights are sized for each call: the binding checks sizes
    # before the library sees the call)
    for kw, args in [({"workspace": short}, (E, topk, K)), ({}, (0, topk, K)), ({}, (E, 0, K)),
                     ({}, (E, topk, 240)), ({}, (2049, topk, K))]:
        e, k_top, kk = args
        we = _dev(w) if e <= E else torch.zeros((e * N * mmq.row_bytes(fmt, kk),), dtype=torch.uint8, device=DEV)
        with pytest.raises(mmq.MMQError):
            mmq.moe_gemm(fmt, xq, we, e, ids, k_top, T, N, kk, out, **kw)
        del we
    torch.cuda.synchronize()
    assert np.isnan(out.cpu().numpy()).all()


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K])
@pytest.mark.parametrize("gemm", [g[0] for g in inputs.MOE_GEMMS])
def test_moe_full_size_sampled_rows(fmt, gemm):
    """The Qwen3-30B-A3B-shaped layer (128 experts, 8 per token, 2048
    tokens) at full size, on routed rows sampled across the output."""
    name, N, K, rows_from = next(g for g in inputs.MOE_GEMMS if g[0] == gemm)
    E, topk, T = inputs.MOE_SHAPE["n_experts"], inputs.MOE_SHAPE["topk"], inputs.MOE_T
    ids = inputs.moe_ids(T, E, topk, inputs.moe_seed("ids"))
    if rows_from == "routed":   # down: one activation row per routed row, topk 1
        T, topk, ids = T * topk, 1, ids.reshape(-1, 1)
    _say(f"moe full size fmt={fmt} {name} T={T} topk={topk} N={N} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(T, K, inputs.moe_seed(f"{name}_x")))
    w = _weights(fmt, E, N, K, inputs.moe_seed(f"{name}_w"))
    got = _run(fmt, xq, w, E, ids, topk, T, N, K)
    assert not np.isnan(got).any(), "routed row left unwritten"
    rows = np.unique(np.random.default_rng(7).integers(0, T * topk, size=48))
    ref = oracle.moe_gemm(fmt, xq, w, ids, topk, T, N, K, E, nthreads=16, rows=rows)
    _check(fmt, got[rows], ref)


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K])
def test_moe_routed_reuse_for_down_projection(fmt):
    """gate/up routes T tokens to topk experts; the down projection then
    reuses those tables with one input row per routed row (T*topk rows,
    topk 1) and equals a fresh routing of the flattened ids."""
    T, E, topk, K1, N1, K2, N2 = 150, 8, 2, 512, 256, 256, 384
    _say(f"moe routed reuse fmt={fmt}")
    ids = inputs.moe_ids(T, E, topk, 160, skew=1.0)
    x1 = oracle.quantize_q8_1(inputs.activations(T, K1, 161))
    w1 = _weights(fmt, E, N1, K1, 162)
    ws = torch.empty((mmq.moe_workspace_bytes(T, topk, E),), dtype=torch.uint8, device=DEV)
    up = torch.full((T * topk, N1), float("nan"), dtype=torch.float32, device=DEV)
    mmq.moe_gemm(fmt, _dev(x1), _dev(w1), E, _dev(ids), topk, T, N1, K1, up, workspace=ws)
    x2 = oracle.quantize_q8_1(inputs.activations(T * topk, K2, 163))
    w2 = _weights(fmt, E, N2, K2, 164)
    down = torch.full((T * topk, N2), float("nan"), dtype=torch.float32, device=DEV)
    mmq.moe_gemm_routed(fmt, _dev(x2), _dev(w2), E, 1, T * topk, N2, K2, ws, down)
    fresh = _run(fmt, x2, w2, E, ids.reshape(-1, 1), 1, T * topk, N2, K2)
    torch.cuda.synchronize()
    got = down.cpu().numpy()
    assert not np.isnan(got).any()
    assert np.array_equal(got.view(np.uint32), fresh.view(np.uint32))
    _check(fmt, got, oracle.moe_gemm(fmt, x2, w2, ids.reshape(-1, 1), 1, T * topk, N2, K2, E, nthreads=16))


def test_moe_routed_without_matching_tables_is_refused():
    """A routed call on a workspace that holds no routing of its sizes is
    refused on the host (nothing launched); a workspace whose tables the
    caller overwrote after routing passes that check but computes nothing
    (the kernel checks the header the routing kernel wrote)."""
    fmt, T, E, topk, N, K = mmq.FMT_Q8_0, 64, 4, 2, 128, 256
    _say("moe routed: no matching tables")
    xq = _dev(oracle.quantize_q8_1(inputs.activations(T, K, 170)))
    w = _dev(_weights(fmt, E, N, K, 171))
    ws = torch.zeros((mmq.moe_workspace_bytes(T, topk, E) + 256,), dtype=torch.uint8, device=DEV)
    out = torch.full((T * topk, N), float("nan"), dtype=torch.float32, device=DEV)
    with pytest.raises(mmq.MMQError, match="no routing"):
        mmq.moe_gemm_routed(fmt, xq, w, E, topk, T, N, K, ws, out)      # never routed
    ids = _dev(inputs.moe_ids(T, E, topk, 172))
    mmq.moe_gemm(fmt, xq, w, E, ids, topk, T, N, K, out, workspace=ws)  # routed for 128 rows, 4 experts
    out2 = torch.full((T * topk // 2, N), float("nan"), dtype=torch.float32, device=DEV)
    with pytest.raises(mmq.MMQError, match="routed for 128 rows"):
        mmq.moe_gemm_routed(fmt, xq, w, E, 1, T, N, K, ws, out2)      # 64 routed rows
    out3 = torch.full((T * topk, N), float("nan"), dtype=torch.float32, device=DEV)
    w5 = torch.zeros(((E + 1) * N * mmq.row_bytes(fmt, K),), dtype=torch.uint8, device=DEV)
    with pytest.raises(mmq.MMQError, match="routed for 128 rows"):
        mmq.moe_gemm_routed(fmt, xq, w5, E + 1, topk, T, N, K, ws, out3)  # 5 experts
    torch.cuda.synchronize()
    assert torch.isnan(out2).all() and torch.isnan(out3).all()
    assert not torch.isnan(out).any()
    ws.zero_()                                                           # the header is gone
    out4 = torch.full((T * topk, N), float("nan"), dtype=torch.float32, device=DEV)
    mmq.moe_gemm_routed(fmt, xq, w, E, topk, T, N, K, ws, out4)
    torch.cuda.synchronize()
    assert torch.isnan(out4).all()


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K, mmq.FMT_Q5_K, mmq.FMT_Q6_K])
def test_moe_remainder_boundaries(fmt):
    """Experts whose last partial tile holds exactly 32 rows (the largest
    remainder the small-remainder launch takes), 33 (a row tile of the tile
    launch), none (a multiple of 128), 17 after two full tiles, and experts
    of 32 rows and of 1 row in all, plus an empty one; N ragged over the
    128-row groups and, for Q8_0, K/32 odd (rows off the dword grid, a last
    unit of one block).  Rows of experts with at most 32 rows are computed by
    the small-remainder launch alone, in the oracle's order for every format
    (K-quants too: min term per sub-block), so they match it bit for bit."""
    counts = [32, 33, 128, 160, 161, 1, 0, 256 + 17]
    E, topk = len(counts), 1
    T = sum(counts)
    ids = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(190).shuffle(ids)
    ids = ids.reshape(T, 1)
    N = 200
    K = 288 if fmt == mmq.FMT_Q8_0 else 512
    _say(f"moe remainder boundaries fmt={fmt} T={T} N={N} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(T, K, 191))
    w = _weights(fmt, E, N, K, 192)
    got = _run(fmt, xq, w, E, ids, topk, T, N, K)
    ref = oracle.moe_gemm(fmt, xq, w, ids, topk, T, N, K, E, nthreads=16)
    _check(fmt, got, ref)
    small = np.isin(ids[:, 0], [e for e, c in enumerate(counts) if 0 < c <= 32])
    assert small.sum() == 33
    assert np.array_equal(got[small].view(np.uint32), ref[small].view(np.uint32))


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K, mmq.FMT_Q5_K, mmq.FMT_Q6_K])
@pytest.mark.parametrize("T,N,K", [(1, 1536, 2048), (4, 768, 2048), (3, 2048, 768)])
def test_moe_decode_sized_is_bit_identical(fmt, T, N, K):
    """A few tokens, 8 of 128 experts each (the Qwen3-30B-A3B router's
    shape): every expert holds at most T rows, so the small-remainder launch
    computes everything and the tile launch nothing, and every row is the
    oracle's bit for bit."""
    E, topk = 128, 8
    _say(f"moe decode-sized fmt={fmt} T={T} N={N} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(T, K, 200 + T))
    w = _weights(fmt, E, N, K, 201)
    ids = inputs.moe_ids(T, E, topk, 202 + T)
    got = _run(fmt, xq, w, E, ids, topk, T, N, K)
    ref = oracle.moe_gemm(fmt, xq, w, ids, topk, T, N, K, E, nthreads=16)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt,T,E,topk", [(mmq.FMT_Q8_0, 300, 2048, 1),   # the most experts: most of them empty
                                          (mmq.FMT_Q4_K, 20, 64, 64),     # the largest topk: every expert per token
                                          (mmq.FMT_Q8_0, 129, 1, 1)])     # one expert: a plain gathered GEMM
def test_moe_extreme_expert_counts(fmt, T, E, topk):
    N, K = 160, 256
    _say(f"moe extremes fmt={fmt} T={T} E={E} topk={topk}")
    xq = oracle.quantize_q8_1(inputs.activations(T, K, 180 + E))
    w = _weights(fmt, E, N, K, 181 + topk)
    ids = inputs.moe_ids(T, E, topk, 182)
    got = _run(fmt, xq, w, E, ids, topk, T, N, K)
    _check(fmt, got, oracle.moe_gemm(fmt, xq, w, ids, topk, T, N, K, E, nthreads=16))
