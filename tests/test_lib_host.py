"""Host-side checks of the GPU library that need no GPU: every symbol the
header declares is exported, and the launch guard (pure host planning)
refuses what it must ("13 . r7-r8 raw-byte MMQ kernel", sections 3.3 and 6:
an over-capacity plan is refused before launch, never run silently)."""
import os
import re

import pytest

import block_quantized_int8_q8_amd as mmq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LDS_GFX950 = 160 * 1024


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "mmq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mmq_[A-Za-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = mmq.lib()
    syms = declared_symbols()
    assert len(syms) >= 9
    for s in syms:
        assert hasattr(L, s), s
    assert set(mmq.EXPORTS) == set(syms)


def test_library_carries_gfx950_code_only():
    blob = open(mmq.LIB_PATH, "rb").read()
    assert b"gfx950" in blob
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert b"amdgcn-amd-amdhsa--" + other not in blob


@pytest.mark.parametrize("fmt,M,N,K", [
    (mmq.FMT_Q8_0, 2048, 3584, 3584),
    (mmq.FMT_Q4_K, 2048, 18944, 3584), (mmq.FMT_Q4_K, 2048, 3584, 18944),
    (mmq.FMT_Q4_K, 8192, 512, 3584), (mmq.FMT_Q8_0, 193, 1, 256),
])
def test_plans_for_benchmark_shapes_fit(fmt, M, N, K):
    ok, desc = mmq.plan_for_limits(fmt, M, N, K, LDS_GFX950, 256)
    assert ok, desc
    assert "kernel=mmq" in desc
    lds = int(re.search(r"lds=(\d+)", desc).group(1))
    assert lds <= 80 * 1024          # two workgroups fit in one CU's 160 KiB
    gx, gy = map(int, re.search(r"grid=(\d+)x(\d+)", desc).groups())
    assert gx == -(-N // 128) and gy == -(-M // 128)


@pytest.mark.parametrize("M,N,K,split,steps", [
    (2048, 3584, 3584, 1, 28),      # 448 tiles: enough to occupy 256 CUs x 2
    (2048, 18944, 3584, 1, 28),
    (512, 512, 3584, 7, 4),         # 16 tiles: 7 slices of 4 k-steps (the minimum)
    (512, 3584, 3584, 3, 10),       # 112 tiles: ~one workgroup per CU
    (512, 3584, 18944, 4, 37),      # 112 tiles of 148 k-steps: two per CU, 4 slices
    (512, 4608, 3584, 3, 10),       # the q+k+v set (144 tiles): 3 slices of >= 8 k-steps
    (2048, 512, 3584, 4, 7),        # 64 tiles
    (8192, 512, 3584, 1, 28),       # 256 tiles: one per CU already
    (200, 256, 512, 1, 4),          # 4 k-steps: too short to split
    (200, 100, 18944, 37, 4),       # two tiles, 148 k-steps
])
def test_split_k_planning(M, N, K, split, steps):
    """With a workspace (ws_*) the split follows the occupancy rule; without
    one the same shapes split into at most two slices (fp32 atomics onto a
    zeroed output, reproducible only for two terms)."""
    for fmt in (mmq.FMT_Q8_0, mmq.FMT_Q4_K):
        ok, desc = mmq.plan_for_limits(fmt, M, N, K, LDS_GFX950, 256)
        assert ok, desc
        k_steps = K // 128
        got = tuple(int(v) for v in re.search(r" ws_split_k=(\d+) ws_steps_per_split=(\d+)", desc).groups())
        assert got == (split, steps), desc
        assert (split - 1) * steps < k_steps <= split * steps   # no empty slice
        tiles = -(-M // 128) * -(-N // 128)
        ws = int(re.search(r"ws_bytes=(\d+)", desc).group(1))
        assert ws == (0 if split == 1 else -(-4 * tiles // 256) * 256 + tiles * split * 128 * 128 * 4), desc
        plain = (2, -(-k_steps // 2)) if split > 1 else (1, k_steps)
        got = tuple(int(v) for v in re.search(r" split_k=(\d+) steps_per_split=(\d+)", desc).groups())
        assert got == plain, desc
        assert f"split_ws=0" in desc


def test_split_workspace_bound():
    """The workspace a split plan needs stays under 2 x CUs x 64 KiB plus the
    counters, over tile counts from 1 to past the split threshold."""
    for n_tiles in range(1, 300):
        ok, desc = mmq.plan_for_limits(mmq.FMT_Q4_K, 128, 128 * n_tiles, 1 << 20, LDS_GFX950, 256)
        assert ok, desc
        ws = int(re.search(r"ws_bytes=(\d+)", desc).group(1))
        assert ws <= 2 * 256 * 65536 + 4096, (n_tiles, desc)


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K])
def test_guard_refuses_over_capacity_lds(fmt):
    ok, desc = mmq.plan_for_limits(fmt, 2048, 3584, 3584, LDS_GFX950, 256)
    need = int(re.search(r"lds=(\d+)", desc).group(1))
    assert mmq.plan_for_limits(fmt, 2048, 3584, 3584, need, 256)[0]
    ok, why = mmq.plan_for_limits(fmt, 2048, 3584, 3584, need - 1, 256)
    assert not ok and "LDS" in why and "refused" in why


def test_extra_lds_hook_forces_refusal():
    try:
        mmq.set_extra_lds(LDS_GFX950)
        ok, why = mmq.plan_for_limits(mmq.FMT_Q8_0, 64, 256, 512, LDS_GFX950, 256)
        assert not ok and "LDS" in why
    finally:
        mmq.set_extra_lds(0)
    assert mmq.plan_for_limits(mmq.FMT_Q8_0, 64, 256, 512, LDS_GFX950, 256)[0]


@pytest.mark.parametrize("fmt,M,N,K,needle", [
    (mmq.FMT_Q8_0, 64, 256, 272, "multiple of 32"),
    (mmq.FMT_Q4_K, 64, 256, 512 + 32, "super-blocks"),
    (mmq.FMT_Q8_0, 0, 256, 512, ">= 1"),
    (mmq.FMT_Q8_0, 64, 0, 512, ">= 1"),
    (mmq.FMT_Q8_0, 64, 256, 0, ">= 1"),
    (7, 64, 256, 512, "format"),
    (mmq.FMT_Q8_0, 1 << 31, 256, 512, "int32"),
    (mmq.FMT_Q8_0, 64, 256, 1 << 24, "at most"),
    (mmq.FMT_Q8_0, (65536 * 128), 256, 512, "row tiles"),
])
def test_guard_refuses_bad_shapes(fmt, M, N, K, needle):
    ok, why = mmq.plan_for_limits(fmt, M, N, K, LDS_GFX950, 256)
    assert not ok and needle in why, why


@pytest.mark.parametrize("M,K", [(64, 32), (200, 96), (2048, 288), (2048, 3616), (5, 3616), (100, 3616),
                                 (160, 3616), (193, 3616)])
def test_q8_0_plans_any_whole_number_of_blocks(M, K):
    """Q8_0 contracts over any whole number of 32-blocks ("When the Product
    Won't Collapse", section 2): the tile kernel's last k-step may hold 1-3
    blocks, the matvec's last unit one block.  The K-quants keep whole
    super-blocks."""
    ok, desc = mmq.plan_for_limits(mmq.FMT_Q8_0, M, 300, K, LDS_GFX950, 256)
    assert ok, desc
    kb = K // 32
    assert f"tail={int(kb % 4 != 0 and M > 192)}" in desc, desc
    steps = int(re.search(r"k_steps=(\d+)", desc).group(1))
    if M <= 8:
        assert "kernel=mv" in desc and steps == (kb + 1) // 2
    elif M <= 192:   # N = 300: a narrow GEMM, the batch-decode kernel
        assert "kernel=sm" in desc and steps == -(-kb // 4)
    else:
        assert "kernel=mmq" in desc and steps == -(-kb // 4)
        split, sps = (int(v) for v in re.search(r"split_k=(\d+) steps_per_split=(\d+)", desc).groups())
        assert (split - 1) * sps < steps <= split * sps
    assert not mmq.plan_for_limits(mmq.FMT_Q4_K, M, 300, K, LDS_GFX950, 256)[0]


def test_guard_refuses_without_compute_units():
    ok, why = mmq.plan_for_limits(mmq.FMT_Q8_0, 64, 256, 512, LDS_GFX950, 0)
    assert not ok and "compute units" in why


@pytest.mark.parametrize("T,topk,E,tiles", [(2048, 8, 128, 128 + 128), (1, 8, 128, 0 + 8), (37, 3, 8, 0 + 8),
                                            (16384, 1, 128, 128 + 128), (0, 2, 4, 0), (5, 1, 3, 0 + 3)])
def test_moe_workspace_bytes(T, topk, E, tiles):
    """A 32-byte header, the tile table (16 B per possible 128-row tile:
    floor(R/128) + min(E, R)), the small-remainder list (16 B per expert)
    and the sorted routed-row ids (4 B each, padded to 16)."""
    R = T * topk
    assert mmq.moe_workspace_bytes(T, topk, E) == 32 + 16 * tiles + 16 * E + -(-4 * R // 16) * 16


@pytest.mark.parametrize("T,topk,E", [(-1, 2, 4), (4, 0, 4), (4, 65, 128), (4, 2, 0), (4, 2, 2049),
                                      (2 ** 31, 1, 4)])
def test_moe_workspace_bytes_refuses(T, topk, E):
    assert mmq.moe_workspace_bytes(T, topk, E) == -1


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K])
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (1, 3584, 3584), (2, 4608, 3584), (5, 7, 512), (8, 18944, 3584), (3, 5, 18944),
                                   (3, 18944, 3584)])
def test_decode_sizes_plan_the_matvec_kernel(fmt, M, N, K):
    """M <= 8: the matvec kernel, four waves per 256-thread workgroup, one
    output row per wave for M <= 4 and two for M >= 5 (the wave's rows share
    each activation load), no LDS, no split; Q4_K at M = 8 (K <= 8192) on the
    matrix core instead: 32 weight rows per workgroup, 4 KiB of LDS for its
    four K-slices' partial sums."""
    ok, desc = mmq.plan_for_limits(fmt, M, N, K, LDS_GFX950, 256)
    if fmt == mmq.FMT_Q8_0 and M >= 4 and N >= 16384:   # the batch-decode kernel (below)
        assert ok and "kernel=sm" in desc, desc
        return
    assert ok and "kernel=mv" in desc, desc
    gx, gy = map(int, re.search(r"grid=(\d+)x(\d+)", desc).groups())
    assert "threads=256" in desc and "split_k=1" in desc
    if fmt == mmq.FMT_Q4_K and (M == 8 or (M >= 3 and N >= 16384)) and K <= 8192:
        assert "mv_mfma=1" in desc and "lds=4096" in desc, desc
        assert (gx, gy) == (-(-N // 32), 1)
    else:
        rows = 1 if M <= 4 else 2
        assert f"mv_rows_per_wave={rows}" in desc and "mv_mfma=0" in desc and "lds=0" in desc, desc
        assert (gx, gy) == (-(-N // (4 * rows)), 1)
    # the same shape with one more row runs the batch-decode kernel, up to
    # M = 192 for these narrow GEMMs, and from M = 193 on the tile kernel
    assert "kernel=sm" in mmq.plan_for_limits(fmt, 9, N, K, LDS_GFX950, 256)[1]
    assert "kernel=sm" in mmq.plan_for_limits(fmt, 192, N, K, LDS_GFX950, 256)[1]
    assert "kernel=mmq" in mmq.plan_for_limits(fmt, 193, N, K, LDS_GFX950, 256)[1]


W_UNITS = {mmq.FMT_Q8_0: 9, mmq.FMT_Q4_K: 5, mmq.FMT_Q5_K: 7, mmq.FMT_Q6_K: 10}


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K, mmq.FMT_Q5_K, mmq.FMT_Q6_K])
@pytest.mark.parametrize("M", [9, 16, 17, 24, 25, 32, 33, 64, 100, 128, 192])
@pytest.mark.parametrize("N,K", [(3584, 18944), (37888, 3584), (4608, 3584), (300, 256), (1, 2048)])
def test_batch_decode_sizes_plan_the_small_m_kernel(fmt, M, N, K):
    """9 <= M <= 32, and up to 192 for GEMMs of fewer 128-column tiles than
    CUs: the batch-decode kernel, one 256-thread workgroup per 32 weight
    rows (and row block of 32 activation rows above M = 32), 16 activation
    rows staged up to M = 16 and 32 above; two
    LDS stages per wave of activation codes and headers (144 B per row) and
    the 32 weight rows' 16-byte units padded to whole 64-lane DMA
    instructions; K in chunks of 4 blocks, split over two workgroups when
    the workgroups fill at most half of the resident slots and K is long
    (256 blocks and more) or the workgroups are fewer than half the CUs
    (with 64 blocks and more); Q4_K with 16 staged rows takes whole
    super-blocks per chunk instead."""
    ok, desc = mmq.plan_for_limits(fmt, M, N, K, LDS_GFX950, 256)
    if M > 32 and -(-N // 128) >= 256:   # a wide GEMM above 32 rows: the tile kernel
        assert ok and "kernel=mmq" in desc, desc
        return
    assert ok and "kernel=sm" in desc and "threads=256" in desc, desc
    ar = 16 if M <= 16 else 32
    assert f"tile={ar}x32" in desc, desc
    gx, gy = map(int, re.search(r"grid=(\d+)x(\d+)", desc).groups())
    groups = -(-N // 32)
    # above 32 rows: one workgroup per (group, row block of 32), the groups
    # padded to whole groups of 8
    assert (gx, gy) == ((groups if M <= 32 else -(-groups // 8) * 8 * -(-M // 32)), 1)
    # chunks of 4 blocks, or of whole super-blocks (Q4_K, 16 staged rows)
    cb = 8 if fmt == mmq.FMT_Q4_K and ar == 16 else 4
    units = 9 if cb == 8 else W_UNITS[fmt]
    assert f"blocks_per_stage={cb}" in desc, desc
    lds = int(re.search(r"lds=(\d+)", desc).group(1))
    assert lds == 2 * 4 * (ar * cb * 36 + 1024 * -(-32 * units // 64))
    chunks = int(re.search(r"k_steps=(\d+)", desc).group(1))
    assert chunks == -(-(K // 32) // cb)
    wg = int(re.search(r"wg_per_cu=(\d+)", desc).group(1))
    assert wg == min(4, (160 * 1024) // lds)   # one wave per SIMD each, 128 registers
    split = int(re.search(r"split_k=(\d+)", desc).group(1))
    assert split == (2 if 2 * gx <= wg * 256 and (K // 32 >= 256 or (2 * gx <= 256 and K // 32 >= 64)) else 1)
    assert "ws_bytes=0" in desc


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K, mmq.FMT_Q5_K, mmq.FMT_Q6_K])
@pytest.mark.parametrize("M", range(1, 9))
@pytest.mark.parametrize("N,K", [(37888, 3584), (3584, 18944), (4608, 3584), (3584, 3584)])
def test_decode_sizes_take_the_batch_decode_kernel_where_measured_faster(fmt, M, N, K):
    """M <= 8: the batch-decode kernel on the wide and long-K launches where
    it measured faster than the matvecs (Q8_0 from M = 4; Q6_K wide from
    M = 4, long-K from M = 7; Q4_K and Q5_K long-K from M = 6), the
    matvecs everywhere else."""
    wide, long_k = N >= 16384, K > 8192
    want = {mmq.FMT_Q8_0: M >= 4 and (wide or long_k),
            mmq.FMT_Q6_K: (M >= 4 and wide) or (M >= 7 and long_k)}.get(fmt, M >= 6 and long_k)
    ok, desc = mmq.plan_for_limits(fmt, M, N, K, LDS_GFX950, 256)
    assert ok and f"kernel={'sm' if want else 'mv'}" in desc, desc


def test_batch_decode_set_counts_32_row_groups():
    """A GEMM set at batch-decode sizes: each member takes whole 32-row
    groups (a workgroup never holds rows of two members)."""
    ok, desc = mmq.plan_for_limits(mmq.FMT_Q4_K, 16, 3584 + 33, 3584, LDS_GFX950, 256)
    assert ok and "grid=114x1" in desc, desc
    ok, desc = mmq.plan_for_limits(mmq.FMT_Q4_K, 64, 3584 + 33, 3584, LDS_GFX950, 256)
    assert ok and "grid=240x1" in desc, desc   # 114 groups padded to 120, two row blocks


@pytest.mark.parametrize("M,q8_skips,kquant_skips", [
    (33, True, True), (64, True, True), (96, True, True),  # one row tile, 1-2 of its 4 wave rows past M
    (97, False, False), (128, False, False),               # every wave row holds rows
    (192, True, True),                                     # 2 of 8 wave rows idle: the 1/4 share
    (200, True, False), (2000, True, False),               # 1 idle wave row
    (2048, False, False), (8192, False, False)])
def test_idle_wave_skip_planning(M, q8_skips, kquant_skips):
    """Waves whose 32 rows all lie past M skip their MFMAs and epilogues.
    The skipping kernel runs full tiles 1-2 % slower, so it is chosen for
    Q8_0 whenever a wave row is idle, and for the K-quants only when idle
    wave rows make up at least 1/4 of the launch's.  The matvec kernel
    (M <= 8) has no row tiles."""
    for fmt, want in [(mmq.FMT_Q8_0, q8_skips), (mmq.FMT_Q4_K, kquant_skips), (mmq.FMT_Q5_K, kquant_skips)]:
        # 296 column tiles: the tile kernel at every M here
        ok, desc = mmq.plan_for_limits(fmt, M, 37888, 3584, LDS_GFX950, 256)
        assert ok and "kernel=mmq" in desc and f"skip_idle_waves={int(want)}" in desc, desc


def test_q5_K_plans_like_q4_K():
    """Q5_K stages the same LDS layout as Q4_K (codes unpacked to one byte,
    scales, split min operand): 80 KiB, two workgroups per CU."""
    for M, N, K in [(2048, 18944, 3584), (512, 512, 3584), (1, 3584, 3584)]:
        a = mmq.plan_for_limits(mmq.FMT_Q5_K, M, N, K, LDS_GFX950, 256)
        b = mmq.plan_for_limits(mmq.FMT_Q4_K, M, N, K, LDS_GFX950, 256)
        assert a[0] and b[0]
        assert a[1].replace("Q5_K", "Q4_K") == b[1]
    assert "lds=81920" in mmq.plan_for_limits(mmq.FMT_Q5_K, 2048, 18944, 3584, LDS_GFX950, 256)[1]
    ok, why = mmq.plan_for_limits(mmq.FMT_Q5_K, 64, 256, 512 + 32, LDS_GFX950, 256)
    assert not ok and "super-blocks" in why


def test_refusal_reasons_are_per_thread():
    """A refusal decided before any device call (here a null pointer or an
    unknown format) leaves its reason in a thread-local string: two threads
    refusing for different reasons each read their own."""
    import ctypes
    import threading
    L = mmq.lib()
    seen = {}

    def worker(name, fmt):
        for _ in range(200):
            rc = L.mmq_gemm_multi(fmt, None, 1, None, None, None, 64, 256, None)
            assert rc == 0
            seen.setdefault(name, set()).add(mmq.last_error())

    a = threading.Thread(target=worker, args=("null", mmq.FMT_Q8_0))
    b = threading.Thread(target=worker, args=("fmt", 7))
    a.start(); b.start(); a.join(); b.join()
    assert seen["null"] == {"null pointer argument"}
    assert seen["fmt"] == {"unknown weight format 7"}


def _t(dtype, n):
    import torch
    return torch.zeros(n, dtype=dtype)


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K, mmq.FMT_Q5_K])
def test_binding_refuses_short_buffers(fmt):
    """The C ABI takes bare pointers, so the binding checks every buffer
    against the shape before the call: a short activation, weight, output,
    id or block-dot buffer is a ValueError naming it (here on CPU tensors,
    which the same check reaches before the device check)."""
    import torch
    u8, f32, i32 = torch.uint8, torch.float32, torch.int32
    M, N, K = 9, 5, 512
    xq_n, w_n, o_n = M * (K // 32) * 36, N * mmq.row_bytes(fmt, K), M * N
    good = dict(xq=_t(u8, xq_n), w=_t(u8, w_n), out=_t(f32, o_n))
    cases = [("xq", _t(u8, xq_n - 1)), ("w", _t(u8, w_n - 1)), ("out", _t(f32, o_n - 1)),
             ("xq", _t(torch.int8, xq_n)), ("out", _t(torch.float16, o_n))]
    for name, bad in cases:
        args = dict(good, **{name: bad})
        with pytest.raises(ValueError, match=name):
            mmq.gemm(fmt, args["xq"], args["w"], M, N, K, args["out"])
    with pytest.raises(ValueError, match="GPU"):   # sizes fine: the device check is next
        mmq.gemm(fmt, good["xq"], good["w"], M, N, K, good["out"])
    with pytest.raises(ValueError, match="w"):
        mmq.gemm_multi(fmt, good["xq"], [good["w"], _t(u8, 3 * mmq.row_bytes(fmt, K))], [N, 4], M, K,
                       [good["out"], _t(f32, M * 4)])
    with pytest.raises(ValueError, match="dots"):
        mmq.debug_block_dots(fmt, good["xq"], good["w"], M, N, K, _t(i32, M * N * (K // 32) - 1))
    T, topk, E = 6, 2, 3
    mw = _t(u8, E * N * mmq.row_bytes(fmt, K))
    mo = _t(f32, T * topk * N)
    ws = _t(u8, 1024)
    ids = _t(i32, T * topk)
    mx = _t(u8, T * (K // 32) * 36)
    with pytest.raises(ValueError, match="ids"):
        mmq.moe_gemm(fmt, mx, mw, E, _t(i32, T * topk - 1), topk, T, N, K, mo, ws)
    with pytest.raises(ValueError, match="expert weights"):
        mmq.moe_gemm(fmt, mx, _t(u8, (E - 1) * N * mmq.row_bytes(fmt, K)), E, ids, topk, T, N, K, mo, ws)
    with pytest.raises(ValueError, match="out"):
        mmq.moe_gemm_routed(fmt, mx, mw, E, topk, T, N, K, ws, _t(f32, T * topk * N - 1))


def test_binding_refuses_short_quantize_buffers():
    import torch
    M, K = 3, 96
    with pytest.raises(ValueError, match="x"):
        mmq.quantize_q8_1(torch.zeros(M, K, dtype=torch.float64))
    with pytest.raises(ValueError, match="q8_1"):
        mmq.quantize_q8_1(torch.zeros(M, K), _t(torch.uint8, M * 3 * 36 - 1))


def _split(desc):
    return int(re.search(r"split_k=(\d+)", desc).group(1))


def test_guard_plans_with_the_kernels_registers():
    """The resident workgroups per CU come from the launched kernel's own
    registers (read from the device with hipFuncGetAttributes; injected
    here): 128 VGPRs give four waves per SIMD, two 8-wave workgroups per CU;
    129-168 give one, which changes the split-K decision; more than 256 fit
    no workgroup and are refused ("13 . r7-r8 raw-byte MMQ kernel", 3.3 and
    6: every capacity the launch depends on is checked before it)."""
    shape = (mmq.FMT_Q8_0, 1280, 2560, 3584)   # 200 output tiles
    ok, desc = mmq.plan_for_limits(*shape, LDS_GFX950, 256)
    assert ok and "wg_per_cu=2 vgprs=128" in desc and _split(desc) == 2, desc
    ok, desc = mmq.plan_for_limits(*shape, LDS_GFX950, 256, vgprs=129)
    assert ok and "wg_per_cu=1 vgprs=129" in desc and _split(desc) == 1, desc
    ok, desc = mmq.plan_for_limits(*shape, LDS_GFX950, 256, vgprs=256)
    assert ok and "wg_per_cu=1" in desc, desc
    ok, why = mmq.plan_for_limits(*shape, LDS_GFX950, 256, vgprs=257)
    assert not ok and "no workgroup" in why and "refused" in why, why
    # LDS bounds residency too: a 100 KiB limit leaves one 76 KiB workgroup per CU
    ok, desc = mmq.plan_for_limits(*shape, 100 * 1024, 256)
    assert ok and "wg_per_cu=1" in desc, desc


@pytest.mark.parametrize("M", [1, 8, 9, 32, 33, 2048])
def test_guard_refuses_kernels_that_spill(M):
    """A kernel that needs scratch missed its register budget: refused
    before launch, for the tile and the matvec kernel alike."""
    ok, why = mmq.plan_for_limits(mmq.FMT_Q4_K, M, 3584, 3584, LDS_GFX950, 256, vgprs=128, scratch=16)
    assert not ok and "scratch" in why and "refused" in why, why
    assert ("matvec" in why) == (M <= 8) and ("batch-decode" in why) == (9 <= M <= 192)


@pytest.mark.parametrize("M", [1, 3, 4, 8, 9, 32, 33, 192, 193, 2048])
def test_q6_K_plans(M):
    """Q6_K (16-element scale groups, no min term): the Q8_0 LDS layout for
    the tile kernel (the group scales fill the scale area), the matvec for
    M <= 3, the batch-decode kernel for 4 <= M <= 192 at this width
    (18944 rows; 148 column tiles, fewer than the CUs), whole
    super-blocks."""
    ok, desc = mmq.plan_for_limits(mmq.FMT_Q6_K, M, 18944, 3584, LDS_GFX950, 256)
    assert ok and "fmt=Q6_K" in desc, desc
    if M <= 3:
        assert "kernel=mv" in desc, desc
    elif M <= 192:
        assert "kernel=sm" in desc, desc
    else:
        assert "kernel=mmq" in desc and int(re.search(r"lds=(\d+)", desc).group(1)) == 77824, desc
    ok, why = mmq.plan_for_limits(mmq.FMT_Q6_K, M, 300, 3584 + 32, LDS_GFX950, 256)
    assert not ok and "super-blocks" in why
    assert mmq.row_bytes(mmq.FMT_Q6_K, 3584) == 14 * 210
