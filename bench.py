#!/usr/bin/env python3
"""Benchmark: q8_1 quantize + block-quantized int8 MMQ on one MI355X.

One step = one pass of the whole path over one batch: quantize the fp32
activations to q8_1, then the MMQ GEMM against the block-quantized weights.
Inputs are seeded synthetic tensors resident in HBM before timing starts.
The Q8_0 headline reads its weights in the tile-packed form (the same Q8_0
bytes reordered once, before timing, by mmq_pack_q8_0; the time that takes
is reported as `pack_ms`), and the same configuration on row-major weights
is timed beside it (`--row-major` puts that one in the headline instead).

Prints ONE JSON line.  `value` is effective int8 TOPS of the whole step,
2*M*N*K / (quantize + GEMM time); the roofline object reports the GEMM
kernel alone against the MI355X dense int8 matrix-core peak, timed with HIP
events on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective int8 MMQ TOPS at 7B prefill shapes (M=2048); % of MFMA int8 peak"
PEAK_INT8_TOPS = 5000.0          # MI355X dense int8 matrix-core peak, TOP/s
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, GB/s


def _code_only(text: str) -> str:
    """C++ source without its comments and blank space, so that the hash
    below follows the code the compiler sees, not its prose (string literals
    in the kernel sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash() -> str:
    """Hash of the kernel sources' code (comments and layout ignored): the
    committed HBM-traffic counters are reported only while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_quantized_int8_q8_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            h.update(_code_only(open(os.path.join(csrc, name)).read()).encode())
    return h.hexdigest()[:16]


def traffic_for(kernel: str):
    """HBM bytes per launch from committed rocprofv3 PMC counters, if they were
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def make_inputs(cfg):
    """`cfg`: a numbered configuration, or "fmt:MxNxK" (seeds 7000 + 1, 2)."""
    from block_quantized_int8_q8_amd import inputs
    if isinstance(cfg, int):
        fmt, M, N, K = inputs.CONFIGS[cfg]
        sx, sw = inputs.seed_for(cfg, 0), inputs.seed_for(cfg, 1)
    else:
        fmt, shape = cfg.split(":")
        M, N, K = (int(v) for v in shape.split("x"))
        sx, sw = inputs.seed_for(7, 1), inputs.seed_for(7, 2)
    x = inputs.activations(M, K, sx)
    gen = {"q8_0": inputs.q8_0_weights, "q4_K": inputs.q4_K_weights, "q5_K": inputs.q5_K_weights,
           "q6_K": inputs.q6_K_weights}[fmt]
    return fmt, M, N, K, x, gen(N, K, sw)


def make_inputs_fmt(cfg) -> str:
    """The weight format of a configuration (without generating its inputs)."""
    from block_quantized_int8_q8_amd import inputs
    return inputs.CONFIGS[cfg][0] if isinstance(cfg, int) else cfg.split(":")[0]


def _fmt_code(fmt: str) -> int:
    import block_quantized_int8_q8_amd as mmq
    return {"q8_0": mmq.FMT_Q8_0, "q4_K": mmq.FMT_Q4_K, "q5_K": mmq.FMT_Q5_K, "q6_K": mmq.FMT_Q6_K}[fmt]


def time_config(cfg, steps: int, warmup: int, check: bool = True, cold: bool = False, packed: bool = False):
    """Time one configuration.  `packed` (Q8_0): the weights are reordered
    once into the tile-packed form (mmq_pack_q8_0, timed on its own as
    `pack_ms`) before anything is timed, and every GEMM reads that form."""
    import torch
    import block_quantized_int8_q8_amd as mmq

    fmt, M, N, K, x, w = make_inputs(cfg)
    dev = torch.device("cuda:0")
    xd = torch.from_numpy(x).to(dev)
    wd = torch.from_numpy(w).to(dev)
    xq = torch.empty((M, K // 32, 36), dtype=torch.uint8, device=dev)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    code = _fmt_code(fmt)
    pack_ms = None
    if packed:
        assert fmt == "q8_0", "the packed form is a Q8_0 layout"
        wpk = mmq.pack_q8_0(wd, N, K)
        torch.cuda.synchronize()
        pack_ms = graph_time(lambda: mmq.pack_q8_0(wd, N, K, wpk), 20, reps=5)
        del wd
        wd = wpk

        def gemm(xq_, w_, M_, N_, K_, out_, stream=None):
            return mmq.gemm_q8_0_packed(xq_, w_, M_, N_, K_, out_, stream=stream)
    else:
        def gemm(*a, **k):
            return mmq.gemm(code, *a, **k)

    stream = torch.cuda.current_stream()

    def step():
        mmq.quantize_q8_1(xd, xq, stream=stream)
        gemm(xq, wd, M, N, K, out, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timed right after the warm-up (a pause for the parity check first would
    # let the clocks drop); the check reads the last timed launch's output.
    # The step (quantize then GEMM on one stream) is timed with two events
    # around all the steps, with nothing recorded in between; the GEMM and
    # the quantize pass alone the same way, back to back (these are the
    # kernels' own durations: an event recorded before each launch leaves a
    # gap the kernel trace does not show).
    def span(fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    t0 = time.perf_counter()
    step_eager_ms = span(step)
    wall = time.perf_counter() - t0
    # the same step captured once as a HIP graph and replayed (the launch
    # sequence without the host in the loop): the step figure reported

    def step_in_graph():
        mmq.quantize_q8_1(xd, xq)
        gemm(xq, wd, M, N, K, out)

    step_ms = graph_time(step_in_graph, steps)
    g_avg = span(lambda: gemm(xq, wd, M, N, K, out, stream=stream))
    # the quantize pass (~6 us at 2048 x 3584) is shorter than the host takes
    # to issue a launch, so back-to-back eager launches would time the host:
    # ten launches captured in a HIP graph, replayed (as the step above)
    q_avg = graph_time(lambda: mmq.quantize_q8_1(xd, xq), steps, reps=10)
    # per launch, evented (median and minimum; each includes the record gap)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        gemm(xq, wd, M, N, K, out, stream=stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    g_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)]
    ops = 2.0 * M * N * K
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    parity = check_parity(fmt, M, N, K, x, w, xq, out) if check else None
    cold_ms = None
    if cold:
        # one launch after writing 512 MB elsewhere: the weights and the q8_1
        # activations are no longer in the 256 MB last-level cache
        scrub = torch.empty(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
        scrub.fill_(1.0)
        a.record(stream)
        gemm(xq, wd, M, N, K, out, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        cold_ms = a.elapsed_time(b)
        del scrub
    return {
        "cfg": cfg, "fmt": fmt, "M": M, "N": N, "K": K,
        "ms_per_step": step_ms, "ms_per_step_eager": step_eager_ms, "step_timing": "HIP graph replay",
        "wall_s": wall,
        "tops_step": ops / (step_ms * 1e-3) / 1e12,
        "gemm_ms_avg": g_avg, "gemm_ms_evented_avg": float(np.mean(g_ms)), "gemm_ms_evented_min": float(np.min(g_ms)),
        "gemm_ms_evented_median": float(np.median(g_ms)), "gemm_ms_cold": cold_ms,
        "gemm_tops": ops / (g_avg * 1e-3) / 1e12,
        "quant_ms_avg": q_avg,
        "quant_gbs": (4.0 + 36.0 / 32.0) * M * K / (q_avg * 1e-3) / 1e9,
        "parity": parity,
        "packed": packed,
        "pack_ms": pack_ms,
    }


def check_parity(fmt, M, N, K, x, w, xq_dev, out_dev, full_rows: int = 2048):
    """The timed output against the oracle: every row when M <= full_rows
    (all the M=2048 configurations), else sampled rows.  The oracle run is
    timed (quantize + GEMM, all host cores): for the configurations other
    than the headline it is their one-run CPU baseline."""
    import oracle
    from tests import metrics
    threads = min(16, os.cpu_count() or 1)
    t0 = time.perf_counter()
    xq = oracle.quantize_q8_1(x)
    q_ok = bool(np.array_equal(xq_dev.cpu().numpy(), xq))
    o = out_dev.cpu().numpy()
    rows = list(range(M)) if M <= full_rows else \
        sorted(set([0, M - 1, M // 2] + list(np.random.default_rng(0).integers(0, M, 5))))
    f = {"q8_0": oracle.gemm_q8_0, "q4_K": oracle.gemm_q4_K, "q5_K": oracle.gemm_q5_K, "q6_K": oracle.gemm_q6_K}[fmt]
    t1 = time.perf_counter()
    ref = f(xq if len(rows) == M else np.ascontiguousarray(xq[rows]), w, len(rows), N, K, nthreads=threads)
    t2 = time.perf_counter()
    rep = metrics.report(o if len(rows) == M else o[rows], ref)
    oracle_s = (t1 - t0) + (t2 - t1) if len(rows) == M else None
    return {
        "quantize_bit_exact": q_ok,
        "unwritten": int(np.isnan(o).sum()),
        "rows_checked": len(rows),
        "normalized_max_error": rep["normalized_max_error"],
        "elementwise_max_rel": rep["elementwise_max_rel"],
        "count_over_tol_elementwise": rep["count_over_tol_elementwise"],
        "bit_identical_fraction": rep["bit_identical_fraction"],
        "ok": bool(q_ok and not np.isnan(o).any() and rep["normalized_max_error"] <= metrics.TOL),
        # the oracle's quantize (including its byte comparison) and full GEMM, one run
        "oracle_s": oracle_s,
        "oracle_threads": oracle.threads_used(threads),
    }


def time_layer(M: int, steps: int, warmup: int, check: bool = True):
    """The seven Q4_K projection GEMMs of one 7B layer at M tokens: one
    quantize pass per distinct input, and the GEMMs that share it (q, k, v;
    gate, up) in one launch; one step is the whole set in order on one
    stream.  Timed as HIP graph replays (the step, and each input group's
    GEMM launch: `gemm_ms`); `ms_per_layer_eager` is the same step issued
    launch by launch from the host."""
    import torch
    import block_quantized_int8_q8_amd as mmq
    from block_quantized_int8_q8_amd import inputs

    dev = torch.device("cuda:0")
    shapes = {g: (n, k) for g, n, k in inputs.LAYER_7B}
    stream = torch.cuda.current_stream()
    host_x, xs, xqs, ws, outs, w_host = {}, {}, {}, {}, {}, {}
    for name, K, gemms in inputs.LAYER_INPUTS:
        host_x[name] = inputs.activations(M, K, inputs.layer_activation_seed(M, name))
        xs[name] = torch.from_numpy(host_x[name]).to(dev)
        xqs[name] = torch.empty((M, K // 32, 36), dtype=torch.uint8, device=dev)
        for g in gemms:
            N, _ = shapes[g]
            w_host[g] = inputs.q4_K_weights(N, K, inputs.layer_weight_seed(g))
            ws[g] = torch.from_numpy(w_host[g]).to(dev)
            outs[g] = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)

    groups = [(name, K, gemms) for name, K, gemms in inputs.LAYER_INPUTS]
    # one split-K workspace for the whole layer: its launches run one after
    # another on one stream, so they never use it at the same time
    need = max(mmq.gemm_workspace_bytes(mmq.FMT_Q4_K, [shapes[g][0] for g in gemms], M, K)
               for _, K, gemms in groups)
    work = torch.empty((max(need, 0),), dtype=torch.uint8, device=dev)

    def run_gemms(name, K, gemms, stream=None):
        mmq.gemm_multi(mmq.FMT_Q4_K, xqs[name], [ws[g] for g in gemms], [shapes[g][0] for g in gemms],
                       M, K, [outs[g] for g in gemms], stream=stream, workspace=work)

    def step(ev=None):
        # one quantize per distinct input, then its GEMMs in one launch
        for i, (name, K, gemms) in enumerate(groups):
            mmq.quantize_q8_1(xs[name], xqs[name], stream=stream)
            if ev is not None:
                ev[i][0].record(stream)
            run_gemms(name, K, gemms, stream=stream)
            if ev is not None:
                ev[i][1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    parity = None
    if check:
        import oracle
        from tests import metrics
        # run to run: the outputs of one more step, bit for bit
        before = {g: outs[g].clone() for g in outs}
        step()
        torch.cuda.synchronize()
        repeat = all(torch.equal(before[g].view(torch.int32), outs[g].view(torch.int32)) for g in outs)
        del before
        worst, unwritten = 0.0, 0
        for name, K, gemms in inputs.LAYER_INPUTS:
            rows = [0, M // 2, M - 1]
            xq = oracle.quantize_q8_1(host_x[name][rows])
            for g in gemms:
                N, _ = shapes[g]
                o = outs[g].cpu().numpy()
                unwritten += int(np.isnan(o).sum())
                worst = max(worst, metrics.normalized_max_error(
                    o[rows], oracle.gemm_q4_K(xq, w_host[g], len(rows), N, K)))
        parity = {"rows_checked_per_gemm": 3, "unwritten": unwritten,
                  "normalized_max_error": worst, "repeat_bit_identical": repeat,
                  "ok": bool(unwritten == 0 and worst <= metrics.TOL and repeat)}
    # eager: launches issued by the host as the step runs (host issue time
    # shows up as idle gaps at small M)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / steps

    # the GPU time: the step, and each group's GEMM launch, as HIP graph replays
    def group_call(name, K, gemms):
        return lambda: step_group(name, K, gemms)

    def step_group(name, K, gemms):
        run_gemms(name, K, gemms)

    def eager_step():
        for name, K, gemms in groups:
            mmq.quantize_q8_1(xs[name], xqs[name])
            step_group(name, K, gemms)

    def separate_step():
        # the variant without sharing: every GEMM quantizes its own input and
        # runs in a launch of its own (7 quantize passes, 7 GEMM launches)
        for name, K, gemms in groups:
            for g in gemms:
                mmq.quantize_q8_1(xs[name], xqs[name])
                run_gemms(name, K, [g])

    step_ms = graph_time(eager_step, steps)
    separate_ms = graph_time(separate_step, steps)
    gemm_ms = {"+".join(gemms): graph_time(group_call(name, K, gemms), steps) for name, K, gemms in groups}
    ops = sum(2.0 * M * n * k for _, n, k in inputs.LAYER_7B)
    return {
        "M": M, "ms_per_layer": step_ms, "ms_per_layer_eager": eager_ms, "timing": "HIP graph replay",
        "split_k_workspace_bytes": need,
        "ms_per_layer_7_passes_7_launches": separate_ms,
        "tops_layer": ops / (step_ms * 1e-3) / 1e12,
        "gemm_tops": ops / (sum(gemm_ms.values()) * 1e-3) / 1e12,
        "gemm_ms": gemm_ms,
        "parity": parity,
    }


def graph_time(fn, n: int, reps: int = 4) -> float:
    """ms per call of `fn` (launches on the current stream): `reps` calls
    captured once in a HIP graph, the graph replayed `n` times between two
    events (host launch cost kept out of the figure)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(reps):
                fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):   # warm
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(max(1, n)):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (max(1, n) * reps)


def time_decode(M: int, fmt_name: str, steps: int, warmup: int, check: bool = True):
    """The 7B layer's projections at decode size (the matvec kernels up to 8
    tokens, the batch-decode kernel above: up to 32 for every GEMM, up to 192
    for the narrow ones), one format: one
    quantize per distinct input and one GEMM launch per input group (q+k+v,
    o, gate+up, down).  These kernels stream every weight byte once, so
    their roofline is HBM: `weight_gbs` is weight bytes / GEMM time.  The
    step runs `layers` copies of the layer's weights (more bytes than the
    256 MB last-level cache holds twice over), as a model's layers would,
    so that every weight byte comes from HBM."""
    import torch
    import block_quantized_int8_q8_amd as mmq
    from block_quantized_int8_q8_amd import inputs

    dev = torch.device("cuda:0")
    fmt = _fmt_code(fmt_name)
    wgen = {"q8_0": inputs.q8_0_weights, "q4_K": inputs.q4_K_weights, "q5_K": inputs.q5_K_weights,
           "q6_K": inputs.q6_K_weights}[fmt_name]
    shapes = {g: (n, k) for g, n, k in inputs.LAYER_7B}
    groups = []
    for name, K, gemms in inputs.LAYER_INPUTS:
        x = inputs.activations(M, K, inputs.layer_activation_seed(2048, name))
        ws_host = [wgen(shapes[g][0], K, inputs.layer_weight_seed(g)) for g in gemms]
        groups.append({
            "gemms": gemms, "K": K, "Ns": [shapes[g][0] for g in gemms], "x_host": x, "w_host": ws_host,
            "x": torch.from_numpy(x).to(dev), "xq": torch.empty((M, K // 32, 36), dtype=torch.uint8, device=dev),
            "out": [torch.full((M, shapes[g][0]), float("nan"), dtype=torch.float32, device=dev) for g in gemms],
        })
    layer_bytes = sum(w.nbytes for g in groups for w in g["w_host"])
    layers = max(2, -(-2 * 256 * 2 ** 20 // layer_bytes))
    for g in groups:   # per layer, its own device copy of the weights
        g["w"] = [[torch.from_numpy(w).to(dev) for w in g["w_host"]] for _ in range(layers)]

    def step():
        for layer in range(layers):
            for g in groups:
                mmq.quantize_q8_1(g["x"], g["xq"])
                mmq.gemm_multi(fmt, g["xq"], g["w"][layer], g["Ns"], M, g["K"], g["out"])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    parity = None
    if check:
        import oracle
        from tests import metrics
        worst, unwritten = 0.0, 0
        f = {mmq.FMT_Q8_0: oracle.gemm_q8_0, mmq.FMT_Q4_K: oracle.gemm_q4_K, mmq.FMT_Q5_K: oracle.gemm_q5_K,
             mmq.FMT_Q6_K: oracle.gemm_q6_K}[fmt]
        for g in groups:
            xq = oracle.quantize_q8_1(g["x_host"])
            for n, w, o in zip(g["Ns"], g["w_host"], g["out"]):
                o = o.cpu().numpy()
                unwritten += int(np.isnan(o).sum())
                worst = max(worst, metrics.normalized_max_error(o, f(xq, w, M, n, g["K"], nthreads=16)))
        parity = {"outputs_checked": "all", "unwritten": unwritten, "normalized_max_error": worst,
                  "ok": bool(unwritten == 0 and worst <= metrics.TOL)}
    # A decode step is a few microseconds of GPU work per launch, less than
    # the host needs to issue a launch, so it is timed as HIP graph replays
    # (the launches captured once): the whole step, and each group's GEMM
    # launch over the layer copies.
    ref_out = [[o.clone() for o in g["out"]] for g in groups]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(step_graph, stream=side):
            step()
        group_graphs = []
        for g in groups:
            gg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gg, stream=side):
                for layer in range(layers):
                    mmq.gemm_multi(fmt, g["xq"], g["w"][layer], g["Ns"], M, g["K"], g["out"])
            group_graphs.append(gg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def timed(graph):
        for _ in range(3):   # warm
            graph.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (steps * layers)

    layer_ms = timed(step_graph)
    gemm_ms = {"+".join(g["gemms"]): timed(gg) for g, gg in zip(groups, group_graphs)}
    # replays recompute the same outputs: they must equal the eager ones
    replay_ok = all(torch.equal(o, r) for g, rs in zip(groups, ref_out) for o, r in zip(g["out"], rs))
    if parity is not None:
        parity["graph_replays_equal_eager"] = bool(replay_ok)
        parity["ok"] = bool(parity["ok"] and replay_ok)
    wbytes = {"+".join(g["gemms"]): float(sum(w.nbytes for w in g["w_host"])) for g in groups}
    return {
        "format": fmt_name.upper(), "M": M, "ms_per_layer": layer_ms, "timing": "HIP graph replay",
        "layer_copies": layers,
        "weight_bytes": sum(wbytes.values()),
        "gemm_ms": gemm_ms,
        "weight_gbs": {k: wbytes[k] / (gemm_ms[k] * 1e-3) / 1e9 for k in gemm_ms},
        "weight_gbs_all_gemms": sum(wbytes.values()) / (sum(gemm_ms.values()) * 1e-3) / 1e9,
        "weight_gbs_layer": sum(wbytes.values()) / (layer_ms * 1e-3) / 1e9,
        "parity": parity,
    }


def time_moe(fmt_name: str, steps: int, warmup: int, check: bool = True):
    """The expert GEMMs of one Qwen3-30B-A3B-shaped MoE layer (128 experts,
    8 per token) at 2048 prefill tokens, in one format: quantize the token
    rows, the gate+up indexed GEMM (routing included), quantize the routed
    rows' down-projection input, the down indexed GEMM.  The routing is
    seeded top-8 over uniform expert scores; the down input is synthetic
    (the activation function between the two GEMMs is not part of the
    path).  `moe_ms` is per indexed GEMM, gate+up's including the routing
    kernel, which down reuses."""
    import torch
    import block_quantized_int8_q8_amd as mmq
    from block_quantized_int8_q8_amd import inputs

    dev = torch.device("cuda:0")
    fmt = _fmt_code(fmt_name)
    wgen = {"q8_0": inputs.q8_0_weights, "q4_K": inputs.q4_K_weights, "q5_K": inputs.q5_K_weights,
           "q6_K": inputs.q6_K_weights}[fmt_name]
    E, topk0, T0 = inputs.MOE_SHAPE["n_experts"], inputs.MOE_SHAPE["topk"], inputs.MOE_T
    ids0 = inputs.moe_ids(T0, E, topk0, inputs.moe_seed("ids"))
    stream = torch.cuda.current_stream()
    legs = []
    for name, N, K, rows_from in inputs.MOE_GEMMS:
        T, topk, ids = (T0, topk0, ids0) if rows_from == "token" else (T0 * topk0, 1, ids0.reshape(-1, 1))
        x = inputs.activations(T, K, inputs.moe_seed(f"{name}_x"))
        w = wgen(E * N, K, inputs.moe_seed(f"{name}_w"))
        legs.append({
            "name": name, "T": T, "topk": topk, "N": N, "K": K, "x_host": x, "w_host": w, "ids_host": ids,
            "x": torch.from_numpy(x).to(dev), "xq": torch.empty((T, K // 32, 36), dtype=torch.uint8, device=dev),
            "w": torch.from_numpy(w).to(dev), "ids": torch.from_numpy(np.ascontiguousarray(ids)).to(dev),
            "out": torch.full((T * topk, N), float("nan"), dtype=torch.float32, device=dev),
            "ws": torch.empty((mmq.moe_workspace_bytes(T, topk, E),), dtype=torch.uint8, device=dev),
        })

    def step(ev=None):
        # down reuses gate+up's routing tables (same routed rows, one input
        # row each): one routing kernel per layer
        for i, g in enumerate(legs):
            mmq.quantize_q8_1(g["x"], g["xq"], stream=stream)
            if ev is not None:
                ev[i][0].record(stream)
            if i == 0:
                mmq.moe_gemm(fmt, g["xq"], g["w"], E, g["ids"], g["topk"], g["T"], g["N"], g["K"], g["out"],
                             workspace=legs[0]["ws"], stream=stream)
            else:
                mmq.moe_gemm_routed(fmt, g["xq"], g["w"], E, g["topk"], g["T"], g["N"], g["K"], legs[0]["ws"],
                                    g["out"], stream=stream)
            if ev is not None:
                ev[i][1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    parity = None
    if check:
        import oracle
        from tests import metrics
        worst, unwritten = 0.0, 0
        for g in legs:
            o = g["out"].cpu().numpy()
            unwritten += int(np.isnan(o).sum())
            R = g["T"] * g["topk"]
            rows = [0, R // 3, R // 2, R - 1]
            toks = sorted({r // g["topk"] for r in rows})
            xq = oracle.quantize_q8_1(g["x_host"][toks])
            # the sampled tokens re-indexed 0..len(toks)-1 with all their routed rows
            sub_ids = g["ids_host"][toks]
            ref = oracle.moe_gemm(fmt, xq, g["w_host"], sub_ids, g["topk"], len(toks), g["N"], g["K"], E)
            got = np.concatenate([o[t * g["topk"]:(t + 1) * g["topk"]] for t in toks])
            worst = max(worst, metrics.normalized_max_error(got, ref))
        parity = {"tokens_checked_per_gemm": 4, "unwritten": unwritten, "normalized_max_error": worst,
                  "ok": bool(unwritten == 0 and worst <= metrics.TOL)}
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in legs] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        step(ev[i])
    end.record(stream)
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / steps
    moe_ms = {g["name"]: float(np.mean([ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(steps)]))
              for j, g in enumerate(legs)}
    ops = {g["name"]: 2.0 * g["T"] * g["topk"] * g["N"] * g["K"] for g in legs}
    wbytes = {g["name"]: float(g["w_host"].nbytes) for g in legs}
    return {
        "format": fmt_name.upper(), "tokens": T0, "experts": E, "topk": topk0,
        "ms_per_layer": step_ms,
        "tops_layer": sum(ops.values()) / (step_ms * 1e-3) / 1e12,
        "moe_ms": moe_ms,
        "moe_tops": {k: ops[k] / (moe_ms[k] * 1e-3) / 1e12 for k in moe_ms},
        # every expert's weights are read at least once per launch
        "expert_weight_gbs": {k: wbytes[k] / (moe_ms[k] * 1e-3) / 1e9 for k in moe_ms},
        "parity": parity,
    }


def oracle_baseline(rec):
    """The one full oracle run of a configuration's parity check (quantize +
    GEMM over every row, all host cores) as its CPU baseline; None when the
    check was skipped or sampled rows only."""
    par = rec.get("parity") or {}
    if not par.get("oracle_s"):
        return None
    M, N, K = rec["M"], rec["N"], rec["K"]
    return {"value": 2.0 * M * N * K / par["oracle_s"] / 1e12, "unit": "TOP/s", "cores": par["oracle_threads"],
            "kind": "oracle", "sample": f"all {M} rows (quantize + full GEMM), one run, {par['oracle_s']:.2f} s",
            "vs_gpu_gemm": rec["gemm_tops"] / (2.0 * M * N * K / par["oracle_s"] / 1e12)}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg: int, target_s: float = 15.0):
    """The oracle (quantize + GEMM) on the host cores, on a bounded sample of
    the same workload (all rows when they finish within `target_s`): the
    median of the all-core runs that fit in about `target_s` (at most 15),
    plus a single-thread row sample and the quantize pass timed on its own.
    Reported, not a target."""
    import oracle
    fmt, M, N, K, x, w = make_inputs(cfg)
    threads = min(16, os.cpu_count() or 1)
    f = {"q8_0": oracle.gemm_q8_0, "q4_K": oracle.gemm_q4_K, "q5_K": oracle.gemm_q5_K, "q6_K": oracle.gemm_q6_K}[fmt]
    used = oracle.threads_used(threads)

    def run(rows, nthreads):
        t0 = time.perf_counter()
        xq = oracle.quantize_q8_1(x[:rows])
        f(xq, w, rows, N, K, nthreads=nthreads)
        return time.perf_counter() - t0

    probe = max(1, min(M, 2 * used))
    t_probe = run(probe, threads)
    rows = int(max(probe, min(M, probe * target_s / max(t_probe, 1e-6))))
    rows = max(used, rows - rows % used) if rows >= used else rows
    times = [run(rows, threads)]
    while len(times) < 15 and sum(times) + times[0] <= target_s:
        times.append(run(rows, threads))
    t = float(np.median(times))
    r1 = min(M, 64)   # one thread, on a row sample
    t1 = run(r1, 1)
    t0 = time.perf_counter()
    oracle.quantize_q8_1(x)
    tq = time.perf_counter() - t0
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {
        "value": 2.0 * rows * N * K / t / 1e12,
        "unit": "TOP/s",
        "cores": used,
        "kind": "oracle",
        "sample": f"{rows} of {M} activation rows (quantize + full-N GEMM), median of {len(times)} runs, "
                  f"{t:.2f} s each",
        "single_thread_tops": 2.0 * r1 * N * K / t1 / 1e12,
        "single_thread_sample": f"{r1} rows, {t1:.2f} s",
        "quantize_gbs": (4.0 + 36.0 / 32.0) * M * K / tq / 1e9,
        "cpu_model": _cpu_model(),
        "nproc": os.cpu_count(),
        "affinity_cpus": affinity,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="benchmark shape (2: Q8_0 2048x3584x3584)")
    ap.add_argument("--extra-configs", default="3,4", help="other shapes timed in the same run")
    ap.add_argument("--extra-shapes", default="q5_K:2048x18944x3584,q6_K:2048x18944x3584",
                    help="fmt:MxNxK GEMMs timed in the same run ('' for none)")
    ap.add_argument("--layer-m", default="512,2048,8192",
                    help="token counts at which the 7B layer GEMM set is timed ('' for none)")
    ap.add_argument("--decode", default="q4_K:1,q8_0:1,q4_K:8,q6_K:1,q4_K:16,q4_K:32,q4_K:64",
                    help="format:M pairs of the timed decode-size layer ('' for none)")
    ap.add_argument("--moe", default="q4_K,q8_0",
                    help="weight formats of the timed 128-expert MoE layer ('' for none)")
    ap.add_argument("--row-major", action="store_true",
                    help="time the headline Q8_0 GEMM on row-major weights instead of the tile-packed form")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the library and this benchmark run on one GPU; --gpus {args.gpus} is not "
              "supported (the path would shard by output columns, with no reduction between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import block_quantized_int8_q8_amd as mmq
    mmq.lib()   # fail loudly when the library is missing

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def progress(what):
        print(f"bench.py: {what} done", file=sys.stderr, flush=True)

    packed = not args.row_major and make_inputs_fmt(args.config) == "q8_0"
    main_rec = time_config(args.config, args.steps, args.warmup, check=not args.no_check, cold=True,
                           packed=packed)
    progress(f"config {args.config}")
    extra = {}
    if packed:
        # the same configuration on row-major weights (mmq_gemm_q8_0), for comparison
        r = time_config(args.config, args.steps, args.warmup, check=not args.no_check)
        extra[f"config{args.config}_row_major"] = {
            k: r[k] for k in ("fmt", "M", "N", "K", "ms_per_step", "tops_step", "gemm_ms_avg", "gemm_tops",
                              "quant_gbs", "parity")}
        extra[f"config{args.config}_row_major"]["gemm_frac_of_int8_peak"] = r["gemm_tops"] / PEAK_INT8_TOPS
        progress(f"config {args.config} row-major")
    for c in [int(v) for v in args.extra_configs.split(",") if v.strip()]:
        if c != args.config:
            r = time_config(c, max(5, args.steps // 5), 2, check=not args.no_check)
            extra[f"config{c}"] = {k: r[k] for k in ("fmt", "M", "N", "K", "ms_per_step", "tops_step",
                                                      "gemm_ms_avg", "gemm_tops", "quant_gbs", "parity")}
            extra[f"config{c}"]["gemm_frac_of_int8_peak"] = r["gemm_tops"] / PEAK_INT8_TOPS
            extra[f"config{c}"]["cpu_baseline"] = oracle_baseline(r)
            progress(f"config {c}")

    for spec in [v.strip() for v in args.extra_shapes.split(",") if v.strip()]:
        r = time_config(spec, max(5, args.steps // 5), 2, check=not args.no_check)
        extra[spec] = {k: r[k] for k in ("fmt", "M", "N", "K", "ms_per_step", "tops_step", "gemm_ms_avg",
                                         "gemm_tops", "quant_gbs", "parity")}
        extra[spec]["gemm_frac_of_int8_peak"] = r["gemm_tops"] / PEAK_INT8_TOPS
        extra[spec]["cpu_baseline"] = oracle_baseline(r)
        progress(spec)

    for m in [int(v) for v in args.layer_m.split(",") if v.strip()]:
        extra[f"layer_M{m}"] = time_layer(m, max(3, args.steps // 10), 1, check=not args.no_check)
        progress(f"layer M={m}")

    for spec in [v.strip() for v in args.decode.split(",") if v.strip()]:
        f, m = spec.split(":")
        extra[f"decode_{f}_M{m}"] = time_decode(int(m), f, max(10, args.steps // 2), 2, check=not args.no_check)
        progress(f"decode {spec}")

    for f in [v.strip() for v in args.moe.split(",") if v.strip()]:
        extra[f"moe_{f}"] = time_moe(f, max(3, args.steps // 5), 1, check=not args.no_check)
        progress(f"moe {f}")

    kname = ("k_mmq<Q8_0,packed>" if packed else "k_mmq<Q8_0>") if main_rec["fmt"] == "q8_0" else "k_mmq<Q4_K>"
    achieved = main_rec["gemm_tops"]
    # The per-block scale costs 32 VALU operations per 32x32x32 MFMA; measured
    # alone (registers only, 4 waves per SIMD) that epilogue takes 159 cycles
    # per MFMA against the MFMA's own 32, which caps this method at 32/159 of
    # the int8 peak on this part.
    epilogue_ceiling = PEAK_INT8_TOPS * 32.0 / 159.0
    roofline = {
        "bound": "mfma",
        "achieved": achieved,
        "peak": PEAK_INT8_TOPS,
        "unit": "TOP/s",
        "frac": achieved / PEAK_INT8_TOPS,
        "traffic": traffic_for(kname),
        "kernel": kname,
        "kernel_ms_avg": main_rec["gemm_ms_avg"],
    }
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.config)
    progress("cpu baseline")
    M, N, K = main_rec["M"], main_rec["N"], main_rec["K"]
    line = {
        "metric": METRIC,
        "value": main_rec["tops_step"],
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": f"{main_rec['fmt'].upper()} x q8_1 MMQ M={M} N={N} K={K} (quantize + GEMM)",
            "M": M, "N": N, "K": K, "format": main_rec["fmt"].upper(),
            "weights": ("Q8_0 in the tile-packed form: the same bytes reordered once before timing "
                        "(mmq_pack_q8_0, pack_ms); row-major figures under extra" if packed else "row-major"),
            "parallelism": "single GPU",
        },
        "pack_ms": main_rec["pack_ms"],
        "frac_of_int8_peak_step": main_rec["tops_step"] / PEAK_INT8_TOPS,
        "step_timing": "quantize + GEMM captured once as a HIP graph, replayed; eager launches: "
                       f"{main_rec['ms_per_step_eager'] * 1e3:.1f} us per step",
        "epilogue_ceiling": {"tops": epilogue_ceiling, "gemm_frac": main_rec["gemm_tops"] / epilogue_ceiling,
                             "basis": "32 MFMA cycles / 159 cycles of scale epilogue per 32x32x32 block product"},
        "gemm_ms": {k: main_rec[k] for k in ("gemm_ms_avg", "gemm_ms_evented_median", "gemm_ms_evented_min",
                                             "gemm_ms_cold")},
        "gemm_tops": main_rec["gemm_tops"],
        "quantize_gbs": main_rec["quant_gbs"],
        "quantize_frac_of_hbm": main_rec["quant_gbs"] / PEAK_HBM_GBS,
        "parity": main_rec["parity"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
