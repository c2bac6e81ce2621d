"""CPU oracle for block-quantized int8 MMQ -- test infrastructure only.

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark import this package.  The GPU library never does, and this package
never imports the GPU library: the two share no code.

The arithmetic lives in ``mmq_oracle.c`` (plain C, built with gcc
``-O2 -ffp-contract=off`` and no fast-math); this module only builds it and
marshals numpy arrays.  Every function states the passage it follows in the
C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mmq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q8_1_BYTES = 36
Q8_0_BYTES = 34
Q4_K_BYTES = 144
Q5_K_BYTES = 176
Q6_K_BYTES = 210


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    cmd = [
        "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
        "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
        _SRC, "-o", _LIB + ".tmp", "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f32_to_f16_array.argtypes = [p, p, i64]
        L.oracle_f16_to_f32_array.argtypes = [p, p, i64]
        L.oracle_moe_gemm.argtypes = [i32, p, p, p, i32, p, i64, i64, i64, i32, i64, i64, i32]
        L.oracle_moe_gemm.restype = i32
        L.oracle_quantize_q8_1.argtypes = [p, p, i64, i64]
        L.oracle_quantize_q8_1.restype = i32
        L.oracle_q4k_scale_min.argtypes = [p, i32, p, p]
        L.oracle_q4k_pack_scale_min.argtypes = [p, p, p]
        L.oracle_q4k_pack_scale_min.restype = i32
        L.oracle_q4k_code.argtypes = [p, i32]
        L.oracle_q4k_code.restype = i32
        L.oracle_dequant_q4_K_block.argtypes = [p, p]
        L.oracle_q5k_code.argtypes = [p, i32]
        L.oracle_q5k_code.restype = i32
        for name in ("oracle_q6k_code", "oracle_q6k_scale"):
            getattr(L, name).argtypes = [p, i32]
            getattr(L, name).restype = i32
        L.oracle_dequant_q6_K_block.argtypes = [p, p]
        L.oracle_group_dots_q6_K.argtypes = [p, p, p, i64, i64, i64]
        L.oracle_group_dots_q6_K.restype = i32
        for name in ("oracle_block_dots_q8_0", "oracle_block_dots_q4_K", "oracle_block_dots_q5_K"):
            getattr(L, name).argtypes = [p, p, p, i64, i64, i64]
            getattr(L, name).restype = i32
        for name in ("oracle_gemm_q8_0", "oracle_gemm_q4_K", "oracle_gemm_q5_K", "oracle_gemm_q6_K"):
            getattr(L, name).argtypes = [p, p, p, i64, i64, i64, i32]
            getattr(L, name).restype = i32
        for name in ("oracle_gemm_q8_0_rows", "oracle_gemm_q4_K_rows", "oracle_gemm_q5_K_rows",
                     "oracle_gemm_q6_K_rows"):
            getattr(L, name).argtypes = [p, p, p, i64, i64, i64, i64, i64, i32]
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------- fp16

def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().oracle_f16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


# ---------------------------------------------------------------- quantize

def quantize_q8_1(x: np.ndarray) -> np.ndarray:
    """fp32 M x K -> uint8 M x (K/32) x 36 (q8_1 blocks)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    y = np.zeros((M, K // 32, Q8_1_BYTES), dtype=np.uint8)
    rc = lib().oracle_quantize_q8_1(_ptr(x), _ptr(y), M, K)
    if rc != 0:
        raise ValueError(f"oracle_quantize_q8_1 failed ({rc}): non-finite input or bad shape")
    return y


# ---------------------------------------------------------------- Q4_K helpers

def q4k_scale_min(s12: np.ndarray, j: int) -> tuple[int, int]:
    s12 = np.ascontiguousarray(s12, dtype=np.uint8)
    assert s12.size == 12
    sc, mn = ctypes.c_uint8(), ctypes.c_uint8()
    lib().oracle_q4k_scale_min(_ptr(s12), j, ctypes.byref(sc), ctypes.byref(mn))
    return sc.value, mn.value


def q4k_pack_scale_min(sc, mn) -> np.ndarray:
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    mn = np.ascontiguousarray(mn, dtype=np.uint8)
    out = np.zeros(12, dtype=np.uint8)
    if lib().oracle_q4k_pack_scale_min(_ptr(sc), _ptr(mn), _ptr(out)) != 0:
        raise ValueError("Q4_K scales and mins must lie in 0..63")
    return out


def q4k_code(superblock: np.ndarray, e: int) -> int:
    superblock = np.ascontiguousarray(superblock, dtype=np.uint8)
    assert superblock.size == Q4_K_BYTES
    return lib().oracle_q4k_code(_ptr(superblock), e)


def q5k_code(superblock: np.ndarray, e: int) -> int:
    """5-bit code of element e of a Q5_K super-block (reading R21 in the C source)."""
    superblock = np.ascontiguousarray(superblock, dtype=np.uint8)
    assert superblock.size == Q5_K_BYTES
    return lib().oracle_q5k_code(_ptr(superblock), e)


def q6k_code(superblock: np.ndarray, e: int) -> int:
    """6-bit code (0..63) of element e of a Q6_K super-block (reading R22 in the C source)."""
    superblock = np.ascontiguousarray(superblock, dtype=np.uint8)
    assert superblock.size == Q6_K_BYTES
    return lib().oracle_q6k_code(_ptr(superblock), e)


def q6k_scale(superblock: np.ndarray, g: int) -> int:
    """int8 scale of 16-element group g of a Q6_K super-block (reading R22)."""
    superblock = np.ascontiguousarray(superblock, dtype=np.uint8)
    assert superblock.size == Q6_K_BYTES
    return lib().oracle_q6k_scale(_ptr(superblock), g)


def dequant_q6_K_block(superblock: np.ndarray) -> np.ndarray:
    superblock = np.ascontiguousarray(superblock, dtype=np.uint8)
    assert superblock.size == Q6_K_BYTES
    out = np.empty(256, dtype=np.float32)
    lib().oracle_dequant_q6_K_block(_ptr(superblock), _ptr(out))
    return out


def dequant_q4_K_block(superblock: np.ndarray) -> np.ndarray:
    superblock = np.ascontiguousarray(superblock, dtype=np.uint8)
    out = np.empty(256, dtype=np.float32)
    lib().oracle_dequant_q4_K_block(_ptr(superblock), _ptr(out))
    return out


# ---------------------------------------------------------------- dots / GEMMs

def block_dots_q8_0(x, w, M, N, K) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    out = np.zeros((M, N, K // 32), dtype=np.int32)
    rc = lib().oracle_block_dots_q8_0(_ptr(x), _ptr(w), _ptr(out), M, N, K)
    if rc != 0:
        raise ValueError(f"bad shape ({rc})")
    return out


def block_dots_q4_K(x, w, M, N, K) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    out = np.zeros((M, N, K // 32), dtype=np.int32)
    rc = lib().oracle_block_dots_q4_K(_ptr(x), _ptr(w), _ptr(out), M, N, K)
    if rc != 0:
        raise ValueError(f"bad shape ({rc})")
    return out


def block_dots_q5_K(x, w, M, N, K) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    out = np.zeros((M, N, K // 32), dtype=np.int32)
    rc = lib().oracle_block_dots_q5_K(_ptr(x), _ptr(w), _ptr(out), M, N, K)
    if rc != 0:
        raise ValueError(f"bad shape ({rc})")
    return out


def group_dots_q6_K(x, w, M, N, K) -> np.ndarray:
    """Q6_K: the exact dot of each 16-element scale group, codes centred (R23)."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    out = np.zeros((M, N, K // 16), dtype=np.int32)
    rc = lib().oracle_group_dots_q6_K(_ptr(x), _ptr(w), _ptr(out), M, N, K)
    if rc != 0:
        raise ValueError(f"bad shape ({rc})")
    return out


def gemm_q8_0(x, w, M, N, K, nthreads: int = 0, rows=None) -> np.ndarray:
    """q8_1 activations x Q8_0 weights -> fp32 M x N (or the row range ``rows``)."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    out = np.zeros((M, N), dtype=np.float32)
    m0, m1 = (0, M) if rows is None else rows
    rc = lib().oracle_gemm_q8_0_rows(_ptr(x), _ptr(w), _ptr(out), M, N, K, m0, m1, nthreads)
    if rc < 0:
        raise ValueError(f"bad shape ({rc})")
    return out


def gemm_q4_K(x, w, M, N, K, nthreads: int = 0, rows=None) -> np.ndarray:
    """q8_1 activations x Q4_K weights -> fp32 M x N (or the row range ``rows``)."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    out = np.zeros((M, N), dtype=np.float32)
    m0, m1 = (0, M) if rows is None else rows
    rc = lib().oracle_gemm_q4_K_rows(_ptr(x), _ptr(w), _ptr(out), M, N, K, m0, m1, nthreads)
    if rc < 0:
        raise ValueError(f"bad shape ({rc})")
    return out


def gemm_q5_K(x, w, M, N, K, nthreads: int = 0, rows=None) -> np.ndarray:
    """q8_1 activations x Q5_K weights -> fp32 M x N (or the row range ``rows``)."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    out = np.zeros((M, N), dtype=np.float32)
    m0, m1 = (0, M) if rows is None else rows
    rc = lib().oracle_gemm_q5_K_rows(_ptr(x), _ptr(w), _ptr(out), M, N, K, m0, m1, nthreads)
    if rc < 0:
        raise ValueError(f"bad shape ({rc})")
    return out


def gemm_q6_K(x, w, M, N, K, nthreads: int = 0, rows=None) -> np.ndarray:
    """q8_1 activations x Q6_K weights -> fp32 M x N (or the row range ``rows``)."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    out = np.zeros((M, N), dtype=np.float32)
    m0, m1 = (0, M) if rows is None else rows
    rc = lib().oracle_gemm_q6_K_rows(_ptr(x), _ptr(w), _ptr(out), M, N, K, m0, m1, nthreads)
    if rc < 0:
        raise ValueError(f"bad shape ({rc})")
    return out


def moe_gemm(fmt: int, x: np.ndarray, w: np.ndarray, ids: np.ndarray, topk: int, T: int, N: int, K: int,
             n_experts: int, nthreads: int = 0, rows=None) -> np.ndarray:
    """Indexed MoE (``oracle_moe_gemm``): out[r] = x[r // topk] times the
    weights of expert ids[r] (experts stored one after another in ``w``).
    ``rows`` selects routed rows (sorted); the result then holds only those."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    R = T * topk
    assert ids.size == R
    out = np.zeros((R, N), dtype=np.float32)
    spans = [(0, R)] if rows is None else [(int(r), int(r) + 1) for r in rows]
    for r0, r1 in spans:
        rc = lib().oracle_moe_gemm(fmt, _ptr(x), _ptr(w), _ptr(ids), topk, _ptr(out), T, N, K, n_experts,
                                   r0, r1, nthreads)
        if rc < 0:
            raise ValueError(f"oracle_moe_gemm rejected the input ({rc})")
    return out if rows is None else out[np.asarray(rows)]


def threads_used(nthreads: int = 0) -> int:
    """Threads the oracle's GEMM runs with for a given request (0 = OpenMP default)."""
    x = np.zeros((1, 1, Q8_1_BYTES), np.uint8)
    w = np.zeros((1, 1, Q8_0_BYTES), np.uint8)
    out = np.zeros((1, 1), np.float32)
    return lib().oracle_gemm_q8_0_rows(_ptr(x), _ptr(w), _ptr(out), 1, 1, 32, 0, 1, nthreads)
