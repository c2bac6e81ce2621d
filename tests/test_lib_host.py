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
    (mmq.FMT_Q8_0, 64, 256, 512), (mmq.FMT_Q8_0, 2048, 3584, 3584),
    (mmq.FMT_Q4_K, 2048, 18944, 3584), (mmq.FMT_Q4_K, 2048, 3584, 18944),
    (mmq.FMT_Q4_K, 8192, 512, 3584), (mmq.FMT_Q8_0, 9, 1, 256),
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
    (64, 256, 512, 1, 4),           # 4 k-steps: too short to split
    (100, 100, 18944, 37, 4),       # one tile, 148 k-steps
])
def test_split_k_planning(M, N, K, split, steps):
    for fmt in (mmq.FMT_Q8_0, mmq.FMT_Q4_K):
        ok, desc = mmq.plan_for_limits(fmt, M, N, K, LDS_GFX950, 256)
        assert ok, desc
        got = tuple(int(v) for v in re.search(r"split_k=(\d+) steps_per_split=(\d+)", desc).groups())
        assert got == (split, steps), desc
        k_steps = K // 128
        assert (split - 1) * steps < k_steps <= split * steps   # no empty slice


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
    (mmq.FMT_Q8_0, 64, 256, 288, "multiple of 256"),
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


def test_guard_refuses_without_compute_units():
    ok, why = mmq.plan_for_limits(mmq.FMT_Q8_0, 64, 256, 512, LDS_GFX950, 0)
    assert not ok and "compute units" in why


@pytest.mark.parametrize("T,topk,E,tiles", [(2048, 8, 128, 128 + 128), (1, 8, 128, 0 + 8), (37, 3, 8, 0 + 8),
                                            (16384, 1, 128, 128 + 128), (0, 2, 4, 0)])
def test_moe_workspace_bytes(T, topk, E, tiles):
    """A 16-byte header, the tile table (16 B per possible 128-row tile:
    floor(R/128) + min(E, R)) and the sorted routed-row ids (4 B each,
    padded to 16)."""
    R = T * topk
    assert mmq.moe_workspace_bytes(T, topk, E) == 16 + 16 * tiles + -(-4 * R // 16) * 16


@pytest.mark.parametrize("T,topk,E", [(-1, 2, 4), (4, 0, 4), (4, 65, 128), (4, 2, 0), (4, 2, 2049),
                                      (2 ** 31, 1, 4)])
def test_moe_workspace_bytes_refuses(T, topk, E):
    assert mmq.moe_workspace_bytes(T, topk, E) == -1


@pytest.mark.parametrize("fmt", [mmq.FMT_Q8_0, mmq.FMT_Q4_K])
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (1, 3584, 3584), (2, 4608, 3584), (5, 7, 512), (8, 18944, 3584), (3, 5, 18944)])
def test_decode_sizes_plan_the_matvec_kernel(fmt, M, N, K):
    """M <= 8: the matvec kernel, four waves per 256-thread workgroup, one
    output row per wave for M <= 4 and two for M >= 5 (the wave's rows share
    each activation load), no LDS, no split."""
    ok, desc = mmq.plan_for_limits(fmt, M, N, K, LDS_GFX950, 256)
    assert ok and "kernel=mv" in desc, desc
    rows = 1 if M <= 4 else 2
    assert f"mv_rows_per_wave={rows}" in desc, desc
    gx, gy = map(int, re.search(r"grid=(\d+)x(\d+)", desc).groups())
    assert (gx, gy) == (-(-N // (4 * rows)), 1)
    assert "threads=256" in desc and "lds=0" in desc and "split_k=1" in desc
    # the same shape with one more row is tiled
    assert "kernel=mmq" in mmq.plan_for_limits(fmt, 9, N, K, LDS_GFX950, 256)[1]


@pytest.mark.parametrize("M,kquant_skips", [
    (9, True), (64, True), (96, True),      # one row tile, 1-3 of its 4 wave rows past M
    (97, False), (128, False),              # every wave row holds rows
    (192, True),                            # 2 of 8 wave rows idle: the 1/4 share
    (200, False), (2000, False), (2048, False), (8192, False)])
def test_idle_wave_skip_planning(M, kquant_skips):
    """Waves whose 32 rows all lie past M skip their MFMAs and epilogues:
    always for Q8_0, and for the K-quants only when idle wave rows make up
    at least 1/4 of the launch's (their skipping kernel runs full tiles a
    little slower).  The matvec kernel (M <= 8) has no row tiles."""
    for fmt, want in [(mmq.FMT_Q8_0, True), (mmq.FMT_Q4_K, kquant_skips), (mmq.FMT_Q5_K, kquant_skips)]:
        ok, desc = mmq.plan_for_limits(fmt, M, 3584, 3584, LDS_GFX950, 256)
        assert ok and f"skip_idle_waves={int(want)}" in desc, desc


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
