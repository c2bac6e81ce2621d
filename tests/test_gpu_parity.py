"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Bars: q8_1 bytes and int32 block dots bit-exact; fp32 outputs within 1e-5 of
the oracle by the normalized measure in tests/metrics.py (Q8_0 is also
bit-identical by construction: same per-block arithmetic in the same order).
Every output buffer is pre-filled with a NaN sentinel, so an element the
kernel never wrote fails the test ("13 . r7-r8 raw-byte MMQ kernel",
section 3.3: prove the kernel ran).
"""
import sys

import numpy as np
import pytest
import torch

import block_quantized_int8_q8_amd as mmq
import oracle
from block_quantized_int8_q8_amd import inputs
from tests import golden_cases, metrics, npdecode

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _nan_out(M, N):
    return torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)


def _gpu_quantize(x: np.ndarray) -> np.ndarray:
    M, K = x.shape
    y = torch.full((M, K // 32, 36), 0xA5, dtype=torch.uint8, device=DEV)
    mmq.quantize_q8_1(_to_dev(x), y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# ------------------------------------------------------------------ quantize

@pytest.mark.parametrize("M,K,seed", [(1, 32, 1), (3, 64, 2), (64, 512, 3), (129, 3584, 4),
                                      (2048, 3584, inputs.seed_for(2, 0)), (7, 18944, 5)])
def test_quantize_bit_exact(M, K, seed):
    _say(f"quantize M={M} K={K} seed={seed}")
    x = inputs.activations(M, K, seed)
    assert np.array_equal(_gpu_quantize(x), oracle.quantize_q8_1(x))


def test_quantize_special_blocks():
    _say("quantize special blocks")
    xs, d_bits, s_bits, codes = golden_cases.q8_1_blocks()
    rows = [xs.reshape(1, -1)]
    r = np.random.default_rng(0)
    scale = np.float32(2.0 ** -3)
    ties = np.zeros((1, 32), np.float32)
    ties[0, :31] = (np.arange(31) + 0.5) * scale * np.where(np.arange(31) % 2, 1, -1)
    ties[0, 31] = 127 * scale
    tiny = (r.standard_normal((1, 64)) * 1e-39).astype(np.float32)   # fp32 subnormal inputs
    huge = (r.standard_normal((1, 64)) * 1e37).astype(np.float32)
    sparse = np.zeros((1, 96), np.float32)
    sparse[0, 40] = -1e-3
    for x in rows + [ties, tiny, huge, sparse]:
        assert np.array_equal(_gpu_quantize(x), oracle.quantize_q8_1(x))
    y = _gpu_quantize(xs.reshape(1, -1))[0]
    assert np.array_equal(y[:, 0:2].copy().view("<u2")[:, 0], d_bits)
    assert np.array_equal(y[:, 2:4].copy().view("<u2")[:, 0], s_bits)
    assert np.array_equal(y[:, 4:].view(np.int8).astype(np.int64), codes)


# ------------------------------------------------------------------ block dots

def _weights(fmt, N, K, seed):
    gen = {mmq.FMT_Q8_0: inputs.q8_0_weights, mmq.FMT_Q4_K: inputs.q4_K_weights, mmq.FMT_Q5_K: inputs.q5_K_weights,
           mmq.FMT_Q6_K: inputs.q6_K_weights}
    return gen[fmt](N, K, seed)


FMTS = [mmq.FMT_Q8_0, mmq.FMT_Q4_K, mmq.FMT_Q5_K, mmq.FMT_Q6_K]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (200, 300, 768), (128, 128, 512), (33, 517, 256)])
def test_block_dots_bit_exact(fmt, M, N, K):
    _say(f"dots fmt={fmt} M={M} N={N} K={K}")
    x = inputs.q8_1_blocks(M, K, 10 + M)
    w = _weights(fmt, N, K, 20 + N)
    per = K // 16 if fmt == mmq.FMT_Q6_K else K // 32   # Q6_K: one dot per 16-element scale group
    dots = torch.full((M, N, per), -(2 ** 31), dtype=torch.int32, device=DEV)
    mmq.debug_block_dots(fmt, _to_dev(x), _to_dev(w), M, N, K, dots)
    torch.cuda.synchronize()
    ref = {mmq.FMT_Q8_0: oracle.block_dots_q8_0, mmq.FMT_Q4_K: oracle.block_dots_q4_K,
           mmq.FMT_Q5_K: oracle.block_dots_q5_K, mmq.FMT_Q6_K: oracle.group_dots_q6_K}[fmt](x, w, M, N, K)
    assert np.array_equal(dots.cpu().numpy(), ref)


# ------------------------------------------------------------------ GEMMs

def _run_gemm(fmt, xq, w, M, N, K):
    out = _nan_out(M, N)
    mmq.gemm(fmt, _to_dev(xq), _to_dev(w), M, N, K, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert not np.isnan(o).any(), "output element left unwritten"
    return o


def _oracle_gemm(fmt, xq, w, M, N, K, rows=None):
    f = {mmq.FMT_Q8_0: oracle.gemm_q8_0, mmq.FMT_Q4_K: oracle.gemm_q4_K, mmq.FMT_Q5_K: oracle.gemm_q5_K,
         mmq.FMT_Q6_K: oracle.gemm_q6_K}[fmt]
    return f(xq, w, M, N, K, nthreads=16, rows=rows)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (64, 256, 512), (200, 300, 768), (129, 257, 1024),
                                   (300, 130, 2048),
                                   # K-quants: M=96 N=33000 runs the idle-wave skipping tile kernel
                                   # (one wave row of four idle; 258 column tiles), M=2000 the
                                   # full-tile one with a ragged tile
                                   (96, 33000, 512), (2000, 300, 512)])
def test_gemm_matches_oracle(fmt, M, N, K):
    _say(f"gemm fmt={fmt} M={M} N={N} K={K}")
    x = inputs.activations(M, K, 30 + M)
    xq = oracle.quantize_q8_1(x)
    w = _weights(fmt, N, K, 40 + N)
    got = _run_gemm(fmt, xq, w, M, N, K)
    ref = _oracle_gemm(fmt, xq, w, M, N, K)
    if _kernel(fmt, M, N, K) in ("mv", "sm"):
        _check_reordered(fmt, got, ref, xq, w, M, N, K)
        return
    rep = metrics.report(got, ref)
    _say(rep)
    assert rep["normalized_max_error"] <= metrics.TOL
    if fmt in (mmq.FMT_Q8_0, mmq.FMT_Q6_K) and _split_k(fmt, M, N, K) == 1:
        # one workgroup per output tile: the oracle's arithmetic in its order
        assert rep["bit_identical_fraction"] == 1.0


U = 2.0 ** -24


def _exact_and_scale(fmt, xq, w, M, N, K):
    """The exact value of every output (block terms summed in fp64) and the
    sum of the absolute block terms, from the independent numpy decoders."""
    kb = K // 32
    xd, xs, xc = npdecode.q8_1_fields(xq.reshape(M, kb, 36))
    if fmt == mmq.FMT_Q6_K:
        # one term per 16-element group: weight scale d*sc, centred codes
        d, sc, codes = npdecode.q6_K_fields(w.reshape(N, K // 256, -1))
        ng = K // 16
        I = np.matmul(xc.reshape(M, ng, 16).transpose(1, 0, 2).astype(np.float64),
                      (codes - 32).reshape(N, ng, 16).transpose(1, 2, 0).astype(np.float64))
        ws = (d[..., None] * sc).reshape(N, ng)
        main = np.repeat(xd, 2, axis=1).T[:, :, None] * ws.T[:, None, :] * I
        return main.sum(0), np.abs(main).sum(0)
    if fmt == mmq.FMT_Q8_0:
        wd, wc = npdecode.q8_0_fields(w.reshape(N, kb, 34))
    else:
        fields = npdecode.q4_K_fields if fmt == mmq.FMT_Q4_K else npdecode.q5_K_fields
        d, dmin, sc, mn, codes = fields(w.reshape(N, K // 256, -1))
        wc = codes.reshape(N, kb, 32)
        wd = (d[..., None] * sc).reshape(N, kb)
    # exact int block dots as fp64 matrix products, one per block
    I = np.matmul(xc.transpose(1, 0, 2).astype(np.float64), wc.transpose(1, 2, 0).astype(np.float64))
    main = xd.T[:, :, None] * wd.T[:, None, :] * I          # [kb, M, N]
    if fmt == mmq.FMT_Q8_0:
        return main.sum(0), np.abs(main).sum(0)
    dm = (dmin[..., None] * mn).reshape(N, kb)
    mins = xs.T[:, :, None] * dm.T[:, None, :]
    return (main - mins).sum(0), (np.abs(main) + np.abs(mins)).sum(0)


def _check_reordered(fmt, got, ref, xq, w, M, N, K):
    """A result summed in another order than the oracle's: every element
    within the fp32 accumulation bound of the exact value (the bound the
    oracle itself is pinned to), and the 1e-5 normalized error against the
    oracle wherever the output has enough elements for its rms to set the
    scale (a single cancellation-dominated sum can differ from the oracle's
    by more than 1e-5 of itself in any order but the oracle's)."""
    exact, absterm = _exact_and_scale(fmt, xq, w, M, N, K)
    err = np.abs(got.astype(np.float64) - exact)
    assert (err <= (K // 32 + 2) * U * absterm + 1e-300).all()
    rep = metrics.report(got, ref)
    _say(rep)
    if M * N >= 64:
        assert rep["normalized_max_error"] <= metrics.TOL


def _kernel(fmt, M, N, K):
    import re
    return re.search(r"kernel=(\w+)", mmq.plan_describe(fmt, M, N, K)[1]).group(1)


def _split_k(fmt, M, N, K):
    import re
    return int(re.search(r"split_k=(\d+)", mmq.plan_describe(fmt, M, N, K)[1]).group(1))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(200, 64, 3584), (250, 257, 1024), (200, 300, 2048), (200, 100, 18944),
                                   (512, 512, 3584)])
def test_split_k_gemm_matches_oracle(fmt, M, N, K):
    """Shapes with too few output tiles for the device run split-K: without
    a workspace, two slices add their partial sums into the zeroed output
    with fp32 atomics (the summation order differs from the oracle's, so the
    tolerance applies and bit identity does not).  Every element must still
    be written, and a second run gives the same bits (a two-term sum onto
    zero does not depend on which slice lands first)."""
    splits = _split_k(fmt, M, N, K)
    _say(f"split-K gemm fmt={fmt} M={M} N={N} K={K} split_k={splits}")
    assert splits == 2 and _kernel(fmt, M, N, K) == "mmq"
    x = inputs.activations(M, K, 50 + M)
    xq = oracle.quantize_q8_1(x)
    w = _weights(fmt, N, K, 60 + N)
    got = _run_gemm(fmt, xq, w, M, N, K)
    rep = metrics.report(got, _oracle_gemm(fmt, xq, w, M, N, K))
    _say(rep)
    assert rep["normalized_max_error"] <= metrics.TOL
    assert np.array_equal(_run_gemm(fmt, xq, w, M, N, K).view(np.uint32), got.view(np.uint32))


def _ws_split_k(fmt, M, N, K):
    import re
    return int(re.search(r"ws_split_k=(\d+)", mmq.plan_describe(fmt, M, N, K)[1]).group(1))


def _run_multi(fmt, xq_dev, w_dev, Ns, M, K, workspace=None):
    outs = [_nan_out(M, n) for n in Ns]
    mmq.gemm_multi(fmt, xq_dev, w_dev, list(Ns), M, K, outs, workspace=workspace)
    torch.cuda.synchronize()
    res = [o.cpu().numpy() for o in outs]
    assert not any(np.isnan(o).any() for o in res), "output element left unwritten"
    return res


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,Ns,K", [(200, (64,), 3584), (200, (100,), 18944), (200, (300,), 2048),
                                    (512, (512,), 3584), (512, (3584,), 18944), (512, (3584, 512, 512), 3584),
                                    (300, (600,), 3616)])
def test_split_workspace_matches_oracle_and_repeats(fmt, M, Ns, K):
    """Split-K through a caller workspace (more than two slices): the slices
    store their partial tiles and the last one of each tile sums them in
    slice order.  Every output element within tolerance of the oracle; the
    same bits again on a second call whose workspace was first filled with
    0xFF (garbage counters and partials: the launch zeroes its counters),
    and on a third; the call without a workspace (at most two slices) also
    repeats bit for bit."""
    if fmt != mmq.FMT_Q8_0 and K % 256:
        pytest.skip("K-quants need whole super-blocks")
    if len(Ns) == 1:
        assert _ws_split_k(fmt, M, Ns[0], K) > 2
    need = mmq.gemm_workspace_bytes(fmt, list(Ns), M, K)
    _say(f"split workspace fmt={fmt} M={M} Ns={Ns} K={K} bytes={need}")
    assert need > 0
    x = inputs.activations(M, K, 150 + M)
    xq = oracle.quantize_q8_1(x)
    ws = [_weights(fmt, n, K, 160 + g) for g, n in enumerate(Ns)]
    xq_dev, w_dev = _to_dev(xq), [_to_dev(w) for w in ws]
    work = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    first = _run_multi(fmt, xq_dev, w_dev, Ns, M, K, work)
    for g, (n, w) in enumerate(zip(Ns, ws)):
        rep = metrics.report(first[g], _oracle_gemm(fmt, xq, w, M, n, K))
        _say(g, rep)
        assert rep["normalized_max_error"] <= metrics.TOL
    for _ in range(2):
        work.fill_(0xFF)
        again = _run_multi(fmt, xq_dev, w_dev, Ns, M, K, work)
        assert all(np.array_equal(a.view(np.uint32), b.view(np.uint32)) for a, b in zip(first, again))
    plain = _run_multi(fmt, xq_dev, w_dev, Ns, M, K)
    assert all(np.array_equal(a.view(np.uint32), b.view(np.uint32))
               for a, b in zip(plain, _run_multi(fmt, xq_dev, w_dev, Ns, M, K)))


def test_split_workspace_refusals():
    """A workspace smaller than the plan needs, or not 16-byte aligned, is
    refused before anything is launched (the outputs keep their NaN
    sentinel); a shape that does not split needs none and computes exactly
    what the call without a workspace computes."""
    fmt, M, N, K = mmq.FMT_Q4_K, 512, 3584, 3584
    need = mmq.gemm_workspace_bytes(fmt, [N], M, K)
    assert need > 0
    x = inputs.activations(M, K, 170)
    xq_dev = _to_dev(oracle.quantize_q8_1(x))
    w_dev = [_to_dev(_weights(fmt, N, K, 171))]
    for work, why in ((torch.zeros(need - 1, dtype=torch.uint8, device=DEV), "workspace holds"),
                      (torch.zeros(need + 16, dtype=torch.uint8, device=DEV)[1:], "aligned")):
        out = _nan_out(M, N)
        with pytest.raises(mmq.MMQError, match=why):
            mmq.gemm_multi(fmt, xq_dev, w_dev, [N], M, K, [out], workspace=work)
        torch.cuda.synchronize()
        assert torch.isnan(out).all()
    M2 = 2048
    assert mmq.gemm_workspace_bytes(fmt, [N], M2, K) == 0
    xq2 = _to_dev(oracle.quantize_q8_1(inputs.activations(M2, K, 172)))
    a = _run_multi(fmt, xq2, w_dev, [N], M2, K, torch.zeros(0, dtype=torch.uint8, device=DEV))
    b = _run_multi(fmt, xq2, w_dev, [N], M2, K)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_on_random_q8_1_fields(fmt):
    """Fields not tied to each other (s independent of the codes): the
    contraction must read d, s and the codes exactly as stored."""
    M, N, K = 150, 200, 512
    _say(f"gemm random fields fmt={fmt}")
    xq = inputs.q8_1_blocks(M, K, 77)
    w = _weights(fmt, N, K, 78)
    got = _run_gemm(fmt, xq, w, M, N, K)
    ref = _oracle_gemm(fmt, xq, w, M, N, K)
    assert metrics.normalized_max_error(got, ref) <= metrics.TOL


def test_gemm_hand_cases():
    _say("gemm hand cases")
    x, w, K, expect = golden_cases.gemm_q8_0_case()
    # K = 64: two blocks, half a k-step of the tile kernel
    xq = _gpu_quantize(x)
    assert _run_gemm(mmq.FMT_Q8_0, xq, w, 1, 1, K)[0, 0] == expect
    # the batch-decode kernel (9 <= M <= 32 in one row block, 33 in two) and
    # the tile kernel (M = 193) as well: the same row repeated
    for m in (9, 33, 193):
        xm = np.repeat(x, m, axis=0)
        assert (_run_gemm(mmq.FMT_Q8_0, _gpu_quantize(xm), w, m, 1, K)[:, 0] == expect).all()
    x, w, K, expect = golden_cases.gemm_q4_K_case()
    xq = _gpu_quantize(x)
    assert _run_gemm(mmq.FMT_Q4_K, xq, w, 1, 1, K)[0, 0] == expect
    for m in (9, 33, 193):
        xm = np.repeat(x, m, axis=0)
        assert (_run_gemm(mmq.FMT_Q4_K, _gpu_quantize(xm), w, m, 1, K)[:, 0] == expect).all()
    x, w, K, expect = golden_cases.gemm_q5_K_case()
    xq = _gpu_quantize(x)
    assert _run_gemm(mmq.FMT_Q5_K, xq, w, 1, 1, K)[0, 0] == expect
    for m in (9, 33, 193):
        xm = np.repeat(x, m, axis=0)
        assert (_run_gemm(mmq.FMT_Q5_K, _gpu_quantize(xm), w, m, 1, K)[:, 0] == expect).all()


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_configs_full_output(cfg):
    """Benchmark shapes, full launch: GPU quantize then GPU GEMM on device
    (the benchmarked path); the oracle checks the quantized bytes and every
    output element ("13 . r7-r8 raw-byte MMQ kernel", section 4: every cell
    against the host reference)."""
    fmt_name, M, N, K = inputs.CONFIGS[cfg]
    fmt = mmq.FMT_Q8_0 if fmt_name == "q8_0" else mmq.FMT_Q4_K
    _say(f"full config {cfg}: {fmt_name} M={M} N={N} K={K}")
    x = inputs.activations(M, K, inputs.seed_for(cfg, 0))
    w = _weights(fmt, N, K, inputs.seed_for(cfg, 1))
    xd = _to_dev(x)
    xq_dev = mmq.quantize_q8_1(xd)
    out = _nan_out(M, N)
    (mmq.gemm_q8_0 if fmt == mmq.FMT_Q8_0 else mmq.gemm_q4_K)(xq_dev, _to_dev(w), M, N, K, out)
    torch.cuda.synchronize()
    xq = oracle.quantize_q8_1(x)
    assert np.array_equal(xq_dev.cpu().numpy(), xq)
    del xq_dev, xd
    o = out.cpu().numpy()
    del out
    assert not np.isnan(o).any()
    rep = metrics.report(o, _oracle_gemm(fmt, xq, w, M, N, K))
    _say(rep)
    assert rep["normalized_max_error"] <= metrics.TOL
    if fmt == mmq.FMT_Q8_0:
        assert rep["bit_identical_fraction"] == 1.0


def test_q5_K_full_size_sampled_rows():
    """Q5_K at the 7B gate/up shape (M=2048 N=18944 K=3584), full launch,
    sampled output rows against the oracle."""
    fmt, M, N, K = mmq.FMT_Q5_K, 2048, 18944, 3584
    _say(f"Q5_K full size M={M} N={N} K={K}")
    x = inputs.activations(M, K, 7001)
    w = _weights(fmt, N, K, 7002)
    xq_dev = mmq.quantize_q8_1(_to_dev(x))
    out = _nan_out(M, N)
    mmq.gemm_q5_K(xq_dev, _to_dev(w), M, N, K, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert not np.isnan(o).any()
    xq = xq_dev.cpu().numpy()
    rows = [0, 1, 1000, M - 128, M - 1]
    rep = metrics.report(o[rows], _oracle_gemm(fmt, np.ascontiguousarray(xq[rows]), w, len(rows), N, K))
    _say(rep)
    assert rep["normalized_max_error"] <= metrics.TOL


@pytest.mark.parametrize("M", inputs.LAYER_M)
def test_layer_gemm_set(M):
    """The seven Q4_K projection GEMMs of one 7B layer at M tokens, run as
    the benchmark runs them: one GPU quantize pass per distinct input and one
    mmq_gemm_multi launch per input group (q+k+v, o, gate+up, down).  The
    q8_1 bytes in full; every output element at M <= 2048, sampled rows
    (first, last, last row tile, random) at M = 8192."""
    shapes = {g: (n, k) for g, n, k in inputs.LAYER_7B}
    for name, K, gemms in inputs.LAYER_INPUTS:
        _say(f"layer M={M}: input {name} K={K}")
        x = inputs.activations(M, K, inputs.layer_activation_seed(M, name))
        xq_dev = mmq.quantize_q8_1(_to_dev(x))
        torch.cuda.synchronize()
        xq = oracle.quantize_q8_1(x)
        assert np.array_equal(xq_dev.cpu().numpy(), xq)
        del x
        if M <= 2048:
            rows = list(range(M))
        else:
            rows = sorted(set([0, M - 1, M - 128, M // 2] + list(np.random.default_rng(M).integers(0, M, 4))))
        sub = xq if len(rows) == M else np.ascontiguousarray(xq[rows])
        ws = [inputs.q4_K_weights(shapes[g][0], K, inputs.layer_weight_seed(g)) for g in gemms]
        Ns = [shapes[g][0] for g in gemms]
        assert all(shapes[g][1] == K for g in gemms)
        outs = [_nan_out(M, n) for n in Ns]
        need = mmq.gemm_workspace_bytes(mmq.FMT_Q4_K, Ns, M, K)
        work = torch.empty(need, dtype=torch.uint8, device=DEV) if need > 0 else None
        _say(f"layer M={M}: gemm set {'+'.join(gemms)} N={Ns} K={K} workspace={need}")
        mmq.gemm_multi(mmq.FMT_Q4_K, xq_dev, [_to_dev(w) for w in ws], Ns, M, K, outs, workspace=work)
        torch.cuda.synchronize()
        for g, n, w, out in zip(gemms, Ns, ws, outs):
            o = out.cpu().numpy()
            assert not np.isnan(o).any(), f"{g}: output element left unwritten"
            rep = metrics.report(o[rows] if len(rows) < M else o, oracle.gemm_q4_K(sub, w, len(rows), n, K, nthreads=16))
            _say(g, rep)
            assert rep["normalized_max_error"] <= metrics.TOL
        del xq_dev, outs
        torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,Ns,K", [(200, (384, 128, 130), 1024), (129, (257,), 512),
                                     (2048, (3584, 512, 512), 3584), (512, (18944, 18944), 3584)])
def test_gemm_multi_matches_oracle(fmt, M, Ns, K):
    """One launch over several weight matrices sharing the q8_1 input: every
    output within tolerance of the oracle (sampled rows at the large shapes),
    every element written."""
    _say(f"gemm multi fmt={fmt} M={M} Ns={Ns} K={K}")
    x = inputs.activations(M, K, 70 + M)
    xq = oracle.quantize_q8_1(x)
    ws = [_weights(fmt, n, K, 80 + g) for g, n in enumerate(Ns)]
    outs = [_nan_out(M, n) for n in Ns]
    mmq.gemm_multi(fmt, _to_dev(xq), [_to_dev(w) for w in ws], list(Ns), M, K, outs)
    torch.cuda.synchronize()
    rows = list(range(M)) if M <= 256 else sorted({0, 1, M // 2, M - 128, M - 1})
    sub = np.ascontiguousarray(xq[rows])
    for g, (n, w) in enumerate(zip(Ns, ws)):
        o = outs[g].cpu().numpy()
        assert not np.isnan(o).any(), f"GEMM {g}: output element left unwritten"
        rep = metrics.report(o[rows], _oracle_gemm(fmt, sub, w, len(rows), n, K))
        _say(g, rep)
        assert rep["normalized_max_error"] <= metrics.TOL


def test_gemm_multi_unsplit_member_equals_single_launch():
    """Without split-K a member of a set computes exactly what its own launch
    computes (same tiles, same arithmetic)."""
    M, K = 2048, 3584
    Ns = (3584, 1024)
    _say(f"gemm multi vs single M={M} Ns={Ns}")
    assert _split_k(mmq.FMT_Q8_0, M, Ns[0], K) == 1
    x = inputs.activations(M, K, 90)
    xq = _to_dev(oracle.quantize_q8_1(x))
    ws = [_to_dev(_weights(mmq.FMT_Q8_0, n, K, 91 + g)) for g, n in enumerate(Ns)]
    outs = mmq.gemm_multi(mmq.FMT_Q8_0, xq, ws, list(Ns), M, K)
    single = mmq.gemm_q8_0(xq, ws[0], M, Ns[0], K)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], single)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 8])
@pytest.mark.parametrize("N,K", [(1, 256), (300, 768), (3584, 3584), (129, 18944)])
def test_matvec_matches_oracle(fmt, M, N, K):
    """Decode-sized inputs (M <= 8) run the matrix-vector kernel (the
    long-K shape at M = 8: the batch-decode kernel): every element written
    and checked as a reordered sum (the blocks of a row are split over 64
    lanes, so bit identity is not expected)."""
    assert _kernel(fmt, M, N, K) == ("sm" if M == 8 and K > 8192 else "mv")
    _say(f"matvec fmt={fmt} M={M} N={N} K={K}")
    x = inputs.activations(M, K, 110 + M)
    xq = oracle.quantize_q8_1(x)
    w = _weights(fmt, N, K, 120 + N)
    got = _run_gemm(fmt, xq, w, M, N, K)
    _check_reordered(fmt, got, _oracle_gemm(fmt, xq, w, M, N, K), xq, w, M, N, K)


def test_kernel_boundaries():
    """M = 8 is the last matvec size, 9 and 32 the first and last
    batch-decode sizes in one row block, 33 and 192 the first and last in
    row blocks of 32 (a narrow GEMM: 5 column tiles), 193 the first tiled
    one; all agree with the oracle on the same weights."""
    fmt, N, K = mmq.FMT_Q4_K, 640, 2048
    w = _weights(fmt, N, K, 130)
    for M, kern in ((8, "mv"), (9, "sm"), (32, "sm"), (33, "sm"), (192, "sm"), (193, "mmq")):
        assert _kernel(fmt, M, N, K) == kern
        xq = oracle.quantize_q8_1(inputs.activations(M, K, 131))
        rep = metrics.report(_run_gemm(fmt, xq, w, M, N, K), _oracle_gemm(fmt, xq, w, M, N, K))
        _say(M, kern, rep)
        assert rep["normalized_max_error"] <= metrics.TOL


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,Ns,K", [(8, (257, 130, 33), 512), (5, (3, 1, 2), 256), (6, (1, 129), 8192)])
def test_matvec_set_rows_straddling_members(fmt, M, Ns, K):
    """M >= 5 runs two output rows per wave, so with odd member widths a
    wave's two rows belong to different GEMMs of the set (and the last wave
    may have one row past the end): every member equals its own launch bit
    for bit and passes the reordered-sum check against the oracle."""
    assert _kernel(fmt, M, Ns[0], K) == "mv"
    _say(f"matvec set fmt={fmt} M={M} Ns={Ns} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 140 + M))
    ws = [_weights(fmt, n, K, 150 + g) for g, n in enumerate(Ns)]
    outs = [_nan_out(M, n) for n in Ns]
    mmq.gemm_multi(fmt, _to_dev(xq), [_to_dev(w) for w in ws], list(Ns), M, K, outs)
    torch.cuda.synchronize()
    for g, (n, w) in enumerate(zip(Ns, ws)):
        o = outs[g].cpu().numpy()
        assert not np.isnan(o).any(), f"GEMM {g}: output element left unwritten"
        single = mmq.gemm(fmt, _to_dev(xq), _to_dev(w), M, n, K)
        torch.cuda.synchronize()
        assert np.array_equal(o.view(np.uint32), single.cpu().numpy().view(np.uint32))
        _check_reordered(fmt, o, _oracle_gemm(fmt, xq, w, M, n, K), xq, w, M, n, K)


@pytest.mark.parametrize("fmt", FMTS)
def test_matvec_layer_set_decode(fmt):
    """The 7B layer's projections at one token: q+k+v and gate+up through
    one matvec launch each, o and down alone; each member equal to its own
    launch, all within tolerance of the oracle."""
    M = 1
    shapes = {g: (n, k) for g, n, k in inputs.LAYER_7B}
    for name, K, gemms in inputs.LAYER_INPUTS:
        _say(f"matvec layer fmt={fmt} {name} {gemms}")
        xq = oracle.quantize_q8_1(inputs.activations(M, K, inputs.layer_activation_seed(2048, name)))
        ws = [_weights(fmt, shapes[g][0], K, inputs.layer_weight_seed(g)) for g in gemms]
        Ns = [shapes[g][0] for g in gemms]
        outs = mmq.gemm_multi(fmt, _to_dev(xq), [_to_dev(w) for w in ws], Ns, M, K)
        torch.cuda.synchronize()
        for g, (n, w) in enumerate(zip(Ns, ws)):
            o = outs[g].cpu().numpy()
            single = mmq.gemm(fmt, _to_dev(xq), _to_dev(w), M, n, K)
            torch.cuda.synchronize()
            assert np.array_equal(o.view(np.uint32), single.cpu().numpy().view(np.uint32))
            rep = metrics.report(o, _oracle_gemm(fmt, xq, w, M, n, K))
            _say(gemms[g], rep)
            assert rep["normalized_max_error"] <= metrics.TOL


def test_gemm_multi_refusals_leave_outputs_untouched():
    _say("gemm multi refusals")
    M, K = 64, 512
    xq = _to_dev(oracle.quantize_q8_1(inputs.activations(M, K, 95)))
    w = _to_dev(_weights(mmq.FMT_Q8_0, 256, K, 96))
    outs = [_nan_out(M, 256), _nan_out(M, 256)]
    with pytest.raises(mmq.MMQError, match="count"):
        mmq.gemm_multi(mmq.FMT_Q8_0, xq, [w] * 9, [256] * 9, M, K, [_nan_out(M, 256) for _ in range(9)])
    with pytest.raises(mmq.MMQError, match="multiple of 32"):
        mmq.gemm_multi(mmq.FMT_Q8_0, xq, [w, w], [256, 256], M, K - 16, outs)
    with pytest.raises(mmq.MMQError, match=">= 1"):
        mmq.gemm_multi(mmq.FMT_Q8_0, xq, [w, w], [256, 0], M, K, outs)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.isnan(o).all()


def test_nondefault_stream():
    _say("non-default stream")
    M, N, K = 96, 160, 512
    x = inputs.activations(M, K, 5)
    w = inputs.q4_K_weights(N, K, 6)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xd = _to_dev(x)
        wd = _to_dev(w)
        xq = mmq.quantize_q8_1(xd, stream=s)
        out = _nan_out(M, N)
        mmq.gemm_q4_K(xq, wd, M, N, K, out, stream=s)
    s.synchronize()
    ref = oracle.gemm_q4_K(oracle.quantize_q8_1(x), w, M, N, K)
    assert metrics.normalized_max_error(out.cpu().numpy(), ref) <= metrics.TOL


# ------------------------------------------------------------------ refusals

def test_refusals_leave_output_untouched():
    _say("refusals")
    M, N, K = 64, 128, 512
    xq = _to_dev(inputs.q8_1_blocks(M, K, 1))
    w = _to_dev(inputs.q8_0_weights(N, K, 2))
    out = _nan_out(M, N)
    try:
        mmq.set_extra_lds(200 * 1024)
        with pytest.raises(mmq.MMQError, match="LDS"):
            mmq.gemm_q8_0(xq, w, M, N, K, out)
        with pytest.raises(mmq.MMQError, match="LDS"):
            mmq.debug_block_dots(mmq.FMT_Q8_0, xq, w, M, N, K)
    finally:
        mmq.set_extra_lds(0)
    with pytest.raises(mmq.MMQError, match="multiple of 32"):
        mmq.gemm_q8_0(xq, w, M, N, K - 16, out)
    with pytest.raises(mmq.MMQError, match="multiple of 256"):
        mmq.gemm_q4_K(xq, w, M, N // 4, K - 32, out)
    with pytest.raises(mmq.MMQError, match="aligned"):
        mmq.gemm_q8_0(xq.view(-1)[4:4 + 36 * M * 15].view(M, 15, 36), w, M, N, 480 + 0 * K, out)
    with pytest.raises(mmq.MMQError, match=">= 1"):
        mmq.gemm_q8_0(xq, w, 0, N, K, out)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    # a normal call afterwards works and writes everything
    mmq.gemm_q8_0(xq, w, M, N, K, out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()


@pytest.mark.parametrize("fmt", FMTS)
def test_device_plans_read_the_kernels_attributes(fmt):
    """On the device the guard reads each launched kernel's registers and
    scratch (hipFuncGetAttributes) before planning: the tile kernels fit two
    workgroups per CU (<= 128 VGPRs, no scratch, or they would be refused),
    the matvec kernels at least one."""
    import re
    for M, N, K, kern in [(2048, 3584, 3584, "mmq"), (2048, 18944, 3584, "mmq"), (96, 33000, 512, "mmq"),
                          (1, 3584, 3584, "mv"), (8, 4608, 3584, "mv")]:
        ok, desc = mmq.plan_describe(fmt, M, N, K)
        _say(desc)
        assert ok and f"kernel={kern}" in desc, desc
        wg, vg = (int(v) for v in re.search(r"wg_per_cu=(\d+) vgprs=(\d+)", desc).groups())
        assert vg > 0 and (wg == 2 and vg <= 128 if kern == "mmq" else wg >= 1), desc


def test_quantize_refusals():
    _say("quantize refusals")
    x = torch.zeros((4, 48), dtype=torch.float32, device=DEV)
    with pytest.raises(mmq.MMQError, match="multiple of 32"):
        mmq.quantize_q8_1(x, torch.empty((4, 2, 36), dtype=torch.uint8, device=DEV))
    ok, desc = mmq.plan_describe(mmq.FMT_Q4_K, 2048, 18944, 3584)
    assert ok, desc


@pytest.mark.parametrize("fmt,M,N,K", [(mmq.FMT_Q4_K, 1, 4608, 3584),      # matvec
                                       (mmq.FMT_Q8_0, 512, 512, 3584),     # split-K: zero fill + atomics
                                       (mmq.FMT_Q5_K, 300, 640, 1024),     # tiled
                                       (mmq.FMT_Q4_K, 16, 3584, 18944)])   # batch decode, split-K
def test_graph_capture_replays_match_eager(fmt, M, N, K):
    """The library's launches captured in a HIP graph (quantize + GEMM on the
    capture stream): every replay, with eager work and synchronizations in
    between, reproduces the eager output (split-K replays within the
    tolerance, since their atomics add in any order)."""
    _say(f"graph capture fmt={fmt} M={M} N={N} K={K}")
    x = _to_dev(inputs.activations(M, K, 140 + M))
    w = _to_dev(_weights(fmt, N, K, 141))
    xq = torch.empty((M, K // 32, 36), dtype=torch.uint8, device=DEV)
    out = _nan_out(M, N)
    mmq.quantize_q8_1(x, xq)
    mmq.gemm(fmt, xq, w, M, N, K, out)
    torch.cuda.synchronize()
    eager = out.clone()
    split = _kernel(fmt, M, N, K) == "mmq" and _split_k(fmt, M, N, K) > 1
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            mmq.quantize_q8_1(x, xq)
            mmq.gemm(fmt, xq, w, M, N, K, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        xq.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert not np.isnan(got).any(), f"replay {rep}: output left unwritten"
        if split:
            assert metrics.normalized_max_error(got, eager.cpu().numpy()) <= metrics.TOL
        else:
            assert torch.equal(out, eager), f"replay {rep} differs from the eager output"


def test_two_host_threads_two_streams():
    """Two host threads, each with its own stream, launch quantize + GEMM
    (tiled and matvec) concurrently; each result equals the same call made
    alone."""
    import threading
    _say("two threads, two streams")
    cases = [(mmq.FMT_Q4_K, 256, 640, 1024, 150), (mmq.FMT_Q8_0, 3, 1000, 2048, 151)]
    data = []
    for fmt, M, N, K, seed in cases:
        x = _to_dev(inputs.activations(M, K, seed))
        w = _to_dev(_weights(fmt, N, K, seed + 1))
        ref = mmq.gemm(fmt, mmq.quantize_q8_1(x), w, M, N, K)
        data.append((fmt, M, N, K, x, w, ref))
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            fmt, M, N, K, x, w, ref = data[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(20):
                    xq = mmq.quantize_q8_1(x, stream=s)
                    out = mmq.gemm(fmt, xq, w, M, N, K, stream=s)
                s.synchronize()
                if not torch.equal(out, ref):
                    errors.append(f"case {i}: result differs")
        except Exception as e:   # reported below, in the main thread
            errors.append(f"case {i}: {e!r}")

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(len(data))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors


# ------------------------------------------------------- Q8_0 at any whole number of 32-blocks
#
# "When the Product Won't Collapse" (section 2) sums over 32-element blocks,
# so Q8_0 takes any K % 32 == 0.  With K/32 odd, every other weight row (and
# every other MoE expert matrix) starts 2 bytes off the dword grid, and the
# tile kernel's last k-step holds 1-3 blocks.

ODD_K = [32, 96, 288, 3616]


@pytest.mark.parametrize("K", ODD_K)
@pytest.mark.parametrize("M,N", [(33, 65), (200, 301)])
def test_q8_0_block_dots_any_whole_blocks(M, N, K):
    _say(f"q8_0 dots any K: M={M} N={N} K={K}")
    x = inputs.q8_1_blocks(M, K, 200 + M)
    w = inputs.q8_0_weights(N, K, 210 + N)
    dots = torch.full((M, N, K // 32), -(2 ** 31), dtype=torch.int32, device=DEV)
    mmq.debug_block_dots(mmq.FMT_Q8_0, _to_dev(x), _to_dev(w), M, N, K, dots)
    torch.cuda.synchronize()
    assert np.array_equal(dots.cpu().numpy(), oracle.block_dots_q8_0(x, w, M, N, K))


@pytest.mark.parametrize("K", [96, 288, 3616])
def test_q8_0_gemm_any_whole_blocks_bit_identical(K):
    """320 output tiles (no split): the whole output equals the oracle bit
    for bit, with ragged rows and columns."""
    M, N = 1200, 4000
    assert _split_k(mmq.FMT_Q8_0, M, N, K) == 1 and _kernel(mmq.FMT_Q8_0, M, N, K) == "mmq"
    _say(f"q8_0 gemm any K: M={M} N={N} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 220 + K))
    w = inputs.q8_0_weights(N, K, 230 + K)
    got = _run_gemm(mmq.FMT_Q8_0, xq, w, M, N, K)
    rep = metrics.report(got, _oracle_gemm(mmq.FMT_Q8_0, xq, w, M, N, K))
    _say(rep)
    assert rep["bit_identical_fraction"] == 1.0


@pytest.mark.parametrize("M,N,K", [(200, 100, 3616), (250, 130, 2080)])
def test_q8_0_split_k_any_whole_blocks(M, N, K):
    assert _split_k(mmq.FMT_Q8_0, M, N, K) > 1 and _kernel(mmq.FMT_Q8_0, M, N, K) == "mmq"
    _say(f"q8_0 split-K any K: M={M} N={N} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 240 + M))
    w = inputs.q8_0_weights(N, K, 250 + N)
    rep = metrics.report(_run_gemm(mmq.FMT_Q8_0, xq, w, M, N, K), _oracle_gemm(mmq.FMT_Q8_0, xq, w, M, N, K))
    _say(rep)
    assert rep["normalized_max_error"] <= metrics.TOL


@pytest.mark.parametrize("K", [32, 288, 3616])
@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("N", [1, 130])
def test_q8_0_matvec_any_whole_blocks(M, N, K):
    assert _kernel(mmq.FMT_Q8_0, M, N, K) == "mv"
    _say(f"q8_0 matvec any K: M={M} N={N} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 260 + M))
    w = inputs.q8_0_weights(N, K, 270 + N)
    got = _run_gemm(mmq.FMT_Q8_0, xq, w, M, N, K)
    _check_reordered(mmq.FMT_Q8_0, got, _oracle_gemm(mmq.FMT_Q8_0, xq, w, M, N, K), xq, w, M, N, K)


def test_q8_0_gemm_multi_any_whole_blocks():
    """A Q8_0 set on the tile kernel (M > 192) with K % 128 != 0, unsplit:
    every member bit-identical to the oracle."""
    M, Ns, K = 250, (257, 130), 288
    _say(f"q8_0 gemm multi any K: M={M} Ns={Ns} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 280))
    ws = [inputs.q8_0_weights(n, K, 281 + g) for g, n in enumerate(Ns)]
    outs = mmq.gemm_multi(mmq.FMT_Q8_0, _to_dev(xq), [_to_dev(w) for w in ws], list(Ns), M, K,
                          [_nan_out(M, n) for n in Ns])
    torch.cuda.synchronize()
    for n, w, o in zip(Ns, ws, outs):
        rep = metrics.report(o.cpu().numpy(), _oracle_gemm(mmq.FMT_Q8_0, xq, w, M, n, K))
        _say(rep)
        assert rep["bit_identical_fraction"] == 1.0


# ------------------------------------------------------------------ batch decode

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [9, 16, 17, 31, 32])
@pytest.mark.parametrize("N,K", [(300, 768), (37, 2048), (3584, 18944)])
def test_batch_decode_matches_oracle(fmt, M, N, K):
    """Batch-decode sizes run the small-M kernel (32 weight rows per
    workgroup, four K-slices added in order, split over two workgroups for
    the narrow long-K shape): every element written and each within the
    fp32 bound of the exact value and the 1e-5 normalized error (a reordered
    sum); ragged N leaves a partial last group of 32 rows, 300 x 768 an odd
    chunk count per K-slice."""
    assert _kernel(fmt, M, N, K) == "sm"
    _say(f"batch decode fmt={fmt} M={M} N={N} K={K} split={_split_k(fmt, M, N, K)}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 300 + M))
    w = _weights(fmt, N, K, 310 + N)
    got = _run_gemm(fmt, xq, w, M, N, K)
    _check_reordered(fmt, got, _oracle_gemm(fmt, xq, w, M, N, K), xq, w, M, N, K)


@pytest.mark.parametrize("M", [12, 32, 70])
@pytest.mark.parametrize("K", [32, 96, 288, 3616])
def test_batch_decode_q8_0_any_whole_blocks(M, K):
    """Q8_0 at batch-decode sizes with K % 128 != 0: the last chunk of 4
    blocks holds 1-3 (K = 32: a single block, three of the four K-slices
    empty)."""
    N = 130
    assert _kernel(mmq.FMT_Q8_0, M, N, K) == "sm"
    _say(f"batch decode q8_0 any K: M={M} N={N} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 320 + K))
    w = inputs.q8_0_weights(N, K, 330 + K)
    got = _run_gemm(mmq.FMT_Q8_0, xq, w, M, N, K)
    _check_reordered(mmq.FMT_Q8_0, got, _oracle_gemm(mmq.FMT_Q8_0, xq, w, M, N, K), xq, w, M, N, K)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [33, 47, 64, 100, 128])
@pytest.mark.parametrize("N,K", [(300, 768), (37, 2048), (3584, 18944)])
def test_batch_decode_row_blocks_match_oracle(fmt, M, N, K):
    """Above 32 rows a GEMM of fewer 128-column tiles than CUs runs the
    batch-decode kernel over row blocks of 32 (one workgroup per weight-row
    group and row block, the last block partial for M = 33, 47 and 100):
    every element written and within the reordered-sum bounds."""
    if K == 18944 and M not in (47, 128):
        pytest.skip("the long-K shape at two sizes only (oracle time)")
    assert _kernel(fmt, M, N, K) == "sm"
    _say(f"batch decode row blocks fmt={fmt} M={M} N={N} K={K} split={_split_k(fmt, M, N, K)}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 360 + M))
    w = _weights(fmt, N, K, 370 + N)
    got = _run_gemm(fmt, xq, w, M, N, K)
    _check_reordered(fmt, got, _oracle_gemm(fmt, xq, w, M, N, K), xq, w, M, N, K)


@pytest.mark.parametrize("fmt", FMTS)
def test_layer_set_at_72_rows(fmt):
    """The 7B layer's projections at 72 tokens: gate+up (296 column tiles)
    on the tile kernel, the narrow sets on the batch-decode kernel in three
    row blocks; every member within tolerance of the oracle, every element
    written."""
    M = 72
    shapes = {g: (n, k) for g, n, k in inputs.LAYER_7B}
    for name, K, gemms in inputs.LAYER_INPUTS:
        xq = oracle.quantize_q8_1(inputs.activations(M, K, inputs.layer_activation_seed(2048, name)))
        ws = [_weights(fmt, shapes[g][0], K, inputs.layer_weight_seed(g)) for g in gemms]
        Ns = [shapes[g][0] for g in gemms]
        _say(f"layer at 72 rows fmt={fmt} {name} {gemms}")
        outs = _run_multi(fmt, _to_dev(xq), [_to_dev(w) for w in ws], Ns, M, K)
        for g, (n, w) in enumerate(zip(Ns, ws)):
            rep = metrics.report(outs[g], _oracle_gemm(fmt, xq, w, M, n, K))
            _say(gemms[g], rep)
            assert rep["normalized_max_error"] <= metrics.TOL


@pytest.mark.parametrize("fmt", FMTS)
def test_batch_decode_set_members_equal_single_launches(fmt):
    """A GEMM set at M = 20 with member widths that are not multiples of 32:
    each member owns whole 32-row groups, equals its own launch bit for bit
    and passes the reordered-sum check."""
    M, Ns, K = 20, (257, 130, 33), 512
    _say(f"batch decode set fmt={fmt} M={M} Ns={Ns} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 340))
    ws = [_weights(fmt, n, K, 350 + g) for g, n in enumerate(Ns)]
    outs = [_nan_out(M, n) for n in Ns]
    mmq.gemm_multi(fmt, _to_dev(xq), [_to_dev(w) for w in ws], list(Ns), M, K, outs)
    torch.cuda.synchronize()
    for n, w, o in zip(Ns, ws, outs):
        o = o.cpu().numpy()
        assert not np.isnan(o).any(), "output element left unwritten"
        single = _run_gemm(fmt, xq, w, M, n, K)
        assert np.array_equal(o.view(np.uint32), single.view(np.uint32))
        _check_reordered(fmt, o, _oracle_gemm(fmt, xq, w, M, n, K), xq, w, M, n, K)


@pytest.mark.parametrize("fmt", FMTS)
def test_batch_decode_layer_set(fmt):
    """The 7B layer's projections at 16 tokens through the batch-decode
    kernel (q+k+v and gate+up as sets, down split over two workgroups):
    every member equal to its own launch wherever the two plans split K
    alike (the split is decided for the set as a whole), all within
    tolerance of the oracle."""
    M = 16
    shapes = {g: (n, k) for g, n, k in inputs.LAYER_7B}
    for name, K, gemms in inputs.LAYER_INPUTS:
        _say(f"batch decode layer fmt={fmt} {name} {gemms}")
        xq = oracle.quantize_q8_1(inputs.activations(M, K, inputs.layer_activation_seed(2048, name)))
        ws = [_weights(fmt, shapes[g][0], K, inputs.layer_weight_seed(g)) for g in gemms]
        Ns = [shapes[g][0] for g in gemms]
        assert _kernel(fmt, M, Ns[0], K) == "sm"
        # the set's plan is the plan of one GEMM over its whole 32-row groups
        set_split = _split_k(fmt, M, sum(-(-n // 32) * 32 for n in Ns), K)
        outs = mmq.gemm_multi(fmt, _to_dev(xq), [_to_dev(w) for w in ws], Ns, M, K)
        torch.cuda.synchronize()
        for g, (n, w) in enumerate(zip(Ns, ws)):
            o = outs[g].cpu().numpy()
            single = mmq.gemm(fmt, _to_dev(xq), _to_dev(w), M, n, K)
            torch.cuda.synchronize()
            if _split_k(fmt, M, n, K) == set_split:
                assert np.array_equal(o.view(np.uint32), single.cpu().numpy().view(np.uint32))
            rep = metrics.report(o, _oracle_gemm(fmt, xq, w, M, n, K))
            _say(gemms[g], rep)
            assert rep["normalized_max_error"] <= metrics.TOL


# ------------------------------------------------------------------ Q6_K

def test_q6_K_hand_case():
    """The hand-summed fixture (tests/golden/gemm_hand.json, q6_K): one
    super-block, sixteen scale groups, through the GPU quantize and GEMM."""
    x, w, K, expect = golden_cases.gemm_q6_K_case()
    xq = _gpu_quantize(x)
    assert _run_gemm(mmq.FMT_Q6_K, xq, w, 1, 1, K)[0, 0] == expect
    for m in (9, 33, 193):
        xm = np.repeat(x, m, axis=0)
        assert (_run_gemm(mmq.FMT_Q6_K, _gpu_quantize(xm), w, m, 1, K)[:, 0] == expect).all()


@pytest.mark.parametrize("M,N,K", [(33, 37888, 3584), (100, 37888, 1024), (1000, 4608, 2304)])
def test_q6_K_bit_identical(M, N, K):
    """Unsplit tile-kernel shapes (more than 256 output tiles) apply each
    16-element group's scale in the oracle's arithmetic and order: every
    output bit-identical."""
    _say(f"q6_K bit-identical M={M} N={N} K={K}")
    assert _kernel(mmq.FMT_Q6_K, M, N, K) == "mmq" and _split_k(mmq.FMT_Q6_K, M, N, K) == 1
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 180 + M))
    w = inputs.q6_K_weights(N, K, 181)
    got = _run_gemm(mmq.FMT_Q6_K, xq, w, M, N, K)
    ref = oracle.gemm_q6_K(xq, w, M, N, K, nthreads=16)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_q6_K_full_size_sampled_rows():
    """Q6_K at the 7B up-projection shape (2048 x 18944 x 3584): sampled rows
    bit-identical to the oracle, every element written."""
    M, N, K = 2048, 18944, 3584
    _say(f"q6_K full size M={M} N={N} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 190))
    w = inputs.q6_K_weights(N, K, 191)
    got = _run_gemm(mmq.FMT_Q6_K, xq, w, M, N, K)
    rows = sorted(set([0, 1, M - 1, M - 128, M // 2] + list(np.random.default_rng(192).integers(0, M, 3))))
    ref = oracle.gemm_q6_K(np.ascontiguousarray(xq[rows]), w, len(rows), N, K, nthreads=16)
    assert np.array_equal(got[rows].view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", [mmq.FMT_Q4_K, mmq.FMT_Q5_K])
@pytest.mark.parametrize("M,N,K", [(3, 16500, 2048), (5, 16417, 768), (7, 20000, 3584), (8, 333, 256)])
def test_matvec_on_matrix_core(fmt, M, N, K):
    """Few rows of a K-quant on the matrix core (mv_mfma=1): 32 weight rows
    per workgroup, the activation rows as the MFMA's other operand, a
    quarter of the blocks per wave.  Every output written, each within the
    fp32 bound of the exact value and the 1e-5 normalized error (reading
    R20); ragged N leaves a partial last group of 32 rows."""
    import re
    desc = mmq.plan_describe(fmt, M, N, K)[1]
    assert "kernel=mv" in desc and "mv_mfma=1" in desc, desc
    _say(f"matvec on matrix core fmt={fmt} M={M} N={N} K={K}")
    xq = oracle.quantize_q8_1(inputs.activations(M, K, 200 + M))
    w = _weights(fmt, N, K, 201)
    got = _run_gemm(fmt, xq, w, M, N, K)
    _check_reordered(fmt, got, _oracle_gemm(fmt, xq, w, M, N, K), xq, w, M, N, K)
