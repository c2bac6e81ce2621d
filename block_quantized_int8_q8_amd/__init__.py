"""Block-quantized int8 MMQ for AMD MI355X (gfx950).

Thin Python binding over ``libmmq.so`` (C ABI in ``include/mmq.h``): argument
marshalling only.  Every step of the path runs in the library's HIP kernels;
PyTorch supplies device memory and the stream.  There is no CPU fallback: if
the library is missing or refuses a call, an exception says why.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmmq.so")

FMT_Q8_0 = 0
FMT_Q4_K = 1
FMT_Q5_K = 2
FMT_Q6_K = 3
Q8_1_BYTES, Q8_0_BYTES, Q4_K_BYTES, Q5_K_BYTES, Q6_K_BYTES = 36, 34, 144, 176, 210

EXPORTS = (
    "mmq_quantize_q8_1", "mmq_gemm_q8_0", "mmq_packed_bytes_q8_0", "mmq_pack_q8_0", "mmq_gemm_q8_0_packed",
    "mmq_gemm_q4_K", "mmq_gemm_q5_K", "mmq_gemm_q6_K", "mmq_gemm_multi", "mmq_gemm_workspace_bytes",
    "mmq_gemm_multi_ws", "mmq_moe_workspace_bytes",
    "mmq_moe_gemm", "mmq_moe_gemm_routed", "mmq_moe_gemm_noalloc", "mmq_debug_block_dots",
    "mmq_last_error", "mmq_plan_describe", "mmq_plan_for_limits",
    "mmq_debug_set_extra_lds", "mmq_version",
)


class MMQError(RuntimeError):
    """The library refused a call (nothing was launched)."""


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmmq.so (built by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.mmq_quantize_q8_1.argtypes = [p, p, i64, i64, p]
        L.mmq_quantize_q8_1.restype = i32
        for name in ("mmq_gemm_q8_0", "mmq_gemm_q4_K", "mmq_gemm_q5_K", "mmq_gemm_q6_K"):
            getattr(L, name).argtypes = [p, p, p, i64, i64, i64, p]
            getattr(L, name).restype = i32
        L.mmq_packed_bytes_q8_0.argtypes = [i64, i64]
        L.mmq_packed_bytes_q8_0.restype = i64
        L.mmq_pack_q8_0.argtypes = [p, i64, i64, p, i64, p]
        L.mmq_pack_q8_0.restype = i32
        L.mmq_gemm_q8_0_packed.argtypes = [p, p, p, i64, i64, i64, p]
        L.mmq_gemm_q8_0_packed.restype = i32
        L.mmq_gemm_multi.argtypes = [i32, p, i32, p, p, p, i64, i64, p]
        L.mmq_gemm_multi.restype = i32
        L.mmq_gemm_workspace_bytes.argtypes = [i32, i32, p, i64, i64]
        L.mmq_gemm_workspace_bytes.restype = i64
        L.mmq_gemm_multi_ws.argtypes = [i32, p, i32, p, p, p, i64, i64, p, i64, p]
        L.mmq_gemm_multi_ws.restype = i32
        L.mmq_moe_workspace_bytes.argtypes = [i64, i32, i32]
        L.mmq_moe_workspace_bytes.restype = i64
        L.mmq_moe_gemm.argtypes = [i32, p, p, i32, p, i32, p, i64, i64, i64, p, i64, p]
        L.mmq_moe_gemm.restype = i32
        L.mmq_moe_gemm_routed.argtypes = [i32, p, p, i32, i32, p, i64, i64, i64, p, i64, p]
        L.mmq_moe_gemm_routed.restype = i32
        L.mmq_moe_gemm_noalloc.argtypes = [i32, p, p, i32, p, i32, p, i64, i64, i64, p]
        L.mmq_moe_gemm_noalloc.restype = i32
        L.mmq_debug_block_dots.argtypes = [i32, p, p, p, i64, i64, i64, p]
        L.mmq_debug_block_dots.restype = i32
        L.mmq_last_error.argtypes = []
        L.mmq_last_error.restype = ctypes.c_char_p
        L.mmq_plan_describe.argtypes = [i32, i64, i64, i64, ctypes.c_char_p, i64]
        L.mmq_plan_describe.restype = i32
        L.mmq_plan_for_limits.argtypes = [i32, i64, i64, i64, i64, i32, i32, i64, ctypes.c_char_p, i64]
        L.mmq_plan_for_limits.restype = i32
        L.mmq_debug_set_extra_lds.argtypes = [i64]
        L.mmq_debug_set_extra_lds.restype = None
        L.mmq_version.argtypes = []
        L.mmq_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().mmq_last_error().decode()


def _check(rc: int, what: str):
    if rc != 1:
        raise MMQError(f"{what}: {last_error()}")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def row_bytes(fmt, K) -> int:
    """Bytes of one weight row of K values in format ``fmt``."""
    if fmt == FMT_Q8_0:
        return (K // 32) * Q8_0_BYTES
    if fmt in (FMT_Q4_K, FMT_Q5_K, FMT_Q6_K):
        return (K // 256) * {FMT_Q4_K: Q4_K_BYTES, FMT_Q5_K: Q5_K_BYTES, FMT_Q6_K: Q6_K_BYTES}[fmt]
    raise ValueError(f"unknown weight format {fmt}")


def _need(t, dtype, count, what):
    """``t`` must be a ``dtype`` tensor holding at least ``count`` elements:
    the library receives bare pointers and trusts the sizes it is given, so a
    short buffer would be read or written past its end on the device."""
    if t.dtype != dtype:
        raise ValueError(f"{what}: expected {dtype}, got {t.dtype}")
    if count > 0 and t.numel() < count:
        raise ValueError(f"{what} holds {t.numel()} elements; the shape needs {count}")


def _dims_ok(*dims) -> bool:
    # sizes are checked only for shapes the library could accept; it refuses
    # the others itself, with its own reason
    return all(int(d) >= 1 for d in dims)


def _ptr(t, dtype=None):
    if not t.is_cuda:
        raise ValueError("tensor must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def quantize_q8_1(x, y=None, stream=None):
    """fp32 [M, K] -> q8_1 uint8 [M, K/32, 36] on the same device."""
    import torch
    M, K = x.shape
    if y is None:
        y = torch.empty((M, K // 32, Q8_1_BYTES), dtype=torch.uint8, device=x.device)
    if _dims_ok(M, K):
        _need(x, torch.float32, M * K, "x")
        _need(y, torch.uint8, M * (K // 32) * Q8_1_BYTES, "y (q8_1)")
    _check(lib().mmq_quantize_q8_1(_ptr(x, torch.float32), _ptr(y, torch.uint8), M, K, _stream(stream)),
           "mmq_quantize_q8_1")
    return y


def _check_gemm_sizes(fmt, xq, w, out, M, N, K):
    import torch
    if _dims_ok(M, N, K):
        _need(xq, torch.uint8, M * (K // 32) * Q8_1_BYTES, "xq (q8_1 activations)")
        _need(w, torch.uint8, N * row_bytes(fmt, K), "w (weights)")
        _need(out, torch.float32, M * N, "out")


def _gemm(fn, name, xq, w, M, N, K, out, stream):
    import torch
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    _check_gemm_sizes(_FN_FMT[fn], xq, w, out, M, N, K)
    _check(getattr(lib(), fn)(_ptr(xq), _ptr(w), _ptr(out, torch.float32), M, N, K, _stream(stream)), name)
    return out


_FN_FMT = {"mmq_gemm_q8_0": FMT_Q8_0, "mmq_gemm_q4_K": FMT_Q4_K, "mmq_gemm_q5_K": FMT_Q5_K,
           "mmq_gemm_q6_K": FMT_Q6_K}


def gemm_q8_0(xq, w, M, N, K, out=None, stream=None):
    """q8_1 [M, K/32, 36] x Q8_0 [N, K/32, 34] -> fp32 [M, N]."""
    return _gemm("mmq_gemm_q8_0", "mmq_gemm_q8_0", xq, w, M, N, K, out, stream)


def packed_bytes_q8_0(N, K) -> int:
    """Bytes of the tile-packed form of an N x K Q8_0 matrix."""
    b = int(lib().mmq_packed_bytes_q8_0(N, K))
    if b < 0:
        raise MMQError(f"mmq_packed_bytes_q8_0: {last_error()}")
    return b


def pack_q8_0(w, N, K, packed=None, stream=None):
    """Q8_0 [N, K/32, 34] -> the tile-packed form (uint8, packed_bytes_q8_0(N, K)),
    reordered on the device; gemm_q8_0_packed reads it."""
    import torch
    nbytes = packed_bytes_q8_0(N, K)
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _need(w, torch.uint8, N * row_bytes(FMT_Q8_0, K), "w (Q8_0 weights)")
    _need(packed, torch.uint8, nbytes, "packed")
    _check(lib().mmq_pack_q8_0(_ptr(w, torch.uint8), N, K, _ptr(packed, torch.uint8), packed.numel(),
                               _stream(stream)), "mmq_pack_q8_0")
    return packed


def gemm_q8_0_packed(xq, packed, M, N, K, out=None, stream=None):
    """q8_1 [M, K/32, 36] x tile-packed Q8_0 (pack_q8_0) -> fp32 [M, N]."""
    import torch
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    if _dims_ok(M, N, K):
        _need(xq, torch.uint8, M * (K // 32) * Q8_1_BYTES, "xq (q8_1 activations)")
        _need(packed, torch.uint8, packed_bytes_q8_0(N, K) if K % 32 == 0 else 0, "packed (Q8_0 weights)")
        _need(out, torch.float32, M * N, "out")
    _check(lib().mmq_gemm_q8_0_packed(_ptr(xq), _ptr(packed), _ptr(out, torch.float32), M, N, K, _stream(stream)),
           "mmq_gemm_q8_0_packed")
    return out


def gemm_q4_K(xq, w, M, N, K, out=None, stream=None):
    """q8_1 [M, K/32, 36] x Q4_K [N, K/256, 144] -> fp32 [M, N]."""
    return _gemm("mmq_gemm_q4_K", "mmq_gemm_q4_K", xq, w, M, N, K, out, stream)


def gemm_q5_K(xq, w, M, N, K, out=None, stream=None):
    """q8_1 [M, K/32, 36] x Q5_K [N, K/256, 176] -> fp32 [M, N]."""
    return _gemm("mmq_gemm_q5_K", "mmq_gemm_q5_K", xq, w, M, N, K, out, stream)


def gemm_q6_K(xq, w, M, N, K, out=None, stream=None):
    """q8_1 [M, K/32, 36] x Q6_K [N, K/256, 210] -> fp32 [M, N]."""
    return _gemm("mmq_gemm_q6_K", "mmq_gemm_q6_K", xq, w, M, N, K, out, stream)


def gemm(fmt, xq, w, M, N, K, out=None, stream=None):
    """The GEMM of weight format ``fmt`` (FMT_Q8_0, FMT_Q4_K, FMT_Q5_K or FMT_Q6_K)."""
    f = {FMT_Q8_0: gemm_q8_0, FMT_Q4_K: gemm_q4_K, FMT_Q5_K: gemm_q5_K, FMT_Q6_K: gemm_q6_K}[fmt]
    return f(xq, w, M, N, K, out, stream)


def gemm_workspace_bytes(fmt, Ns, M, K) -> int:
    """Split-K workspace bytes gemm_multi(..., workspace=...) needs on the
    current device (0: the set does not split; -1: it would be refused)."""
    count = len(Ns)
    npv = (ctypes.c_int64 * max(count, 1))(*[int(n) for n in Ns])
    return int(lib().mmq_gemm_workspace_bytes(fmt, count, npv, M, K))


def gemm_multi(fmt, xq, ws, Ns, M, K, outs=None, stream=None, workspace=None):
    """One launch of several GEMMs sharing the q8_1 activations:
    q8_1 [M, K/32, 36] x ws[g] [N[g], ...] -> outs[g] fp32 [M, N[g]].
    ``workspace``: a uint8 device tensor of at least gemm_workspace_bytes
    bytes, which lets a shape with few output tiles split K further
    (mmq_gemm_multi_ws); None: mmq_gemm_multi."""
    import torch
    count = len(ws)
    if len(Ns) != count or (outs is not None and len(outs) != count):
        raise ValueError("ws, Ns and outs must have the same length")
    if outs is None:
        outs = [torch.empty((M, n), dtype=torch.float32, device=xq.device) for n in Ns]
    for w, o, n in zip(ws, outs, Ns):
        _check_gemm_sizes(fmt, xq, w, o, M, n, K)
    wp = (ctypes.c_void_p * count)(*[_ptr(w).value for w in ws])
    op = (ctypes.c_void_p * count)(*[_ptr(o, torch.float32).value for o in outs])
    npv = (ctypes.c_int64 * count)(*[int(n) for n in Ns])
    if workspace is None:
        _check(lib().mmq_gemm_multi(fmt, _ptr(xq), count, wp, op, npv, M, K, _stream(stream)), "mmq_gemm_multi")
    else:
        _need(workspace, torch.uint8, 0, "workspace")
        _check(lib().mmq_gemm_multi_ws(fmt, _ptr(xq), count, wp, op, npv, M, K, _ptr(workspace),
                                       workspace.numel(), _stream(stream)), "mmq_gemm_multi_ws")
    return outs


def moe_workspace_bytes(T, topk, n_experts) -> int:
    """Device workspace bytes mmq_moe_gemm needs (-1 for arguments it refuses)."""
    return int(lib().mmq_moe_workspace_bytes(T, topk, n_experts))


def _check_moe_sizes(fmt, xq, w, n_experts, topk, T, N, K, out, workspace):
    import torch
    if _dims_ok(T, topk, n_experts, N, K):
        _need(xq, torch.uint8, T * (K // 32) * Q8_1_BYTES, "xq (q8_1 activations)")
        _need(w, torch.uint8, n_experts * N * row_bytes(fmt, K), "w (expert weights)")
        _need(out, torch.float32, T * topk * N, "out")
    if workspace is not None:
        _need(workspace, torch.uint8, 0, "workspace")


def moe_gemm(fmt, xq, w, n_experts, ids, topk, T, N, K, out=None, workspace=None, stream=None):
    """Indexed MoE: q8_1 [T, K/32, 36] x expert weights [E, N, ...] routed by
    int32 ids [T, topk] -> fp32 [T*topk, N] (row t*topk + j = token t times
    expert ids[t, j])."""
    import torch
    if out is None:
        out = torch.empty((T * topk, N), dtype=torch.float32, device=xq.device)
    need = moe_workspace_bytes(T, topk, n_experts)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=xq.device)
    _check_moe_sizes(fmt, xq, w, n_experts, topk, T, N, K, out, workspace)
    if _dims_ok(T, topk):
        _need(ids, torch.int32, T * topk, "ids")
    _check(lib().mmq_moe_gemm(fmt, _ptr(xq), _ptr(w), n_experts, _ptr(ids, torch.int32), topk,
                              _ptr(out, torch.float32), T, N, K, _ptr(workspace, torch.uint8),
                              workspace.numel(), _stream(stream)), "mmq_moe_gemm")
    return out


def moe_gemm_routed(fmt, xq, w, n_experts, topk, T, N, K, workspace, out=None, stream=None):
    """Indexed MoE on the routing tables an earlier ``moe_gemm`` left in
    ``workspace`` (same T*topk routed rows and experts; e.g. the down
    projection: T*topk input rows, topk 1)."""
    import torch
    if out is None:
        out = torch.empty((T * topk, N), dtype=torch.float32, device=xq.device)
    _check_moe_sizes(fmt, xq, w, n_experts, topk, T, N, K, out, workspace)
    _check(lib().mmq_moe_gemm_routed(fmt, _ptr(xq), _ptr(w), n_experts, topk, _ptr(out, torch.float32), T, N, K,
                                     _ptr(workspace, torch.uint8), workspace.numel(), _stream(stream)),
           "mmq_moe_gemm_routed")
    return out


MOE_NOALLOC_MAX_ROUTED = 131072   # T * topk the allocation-free MoE entry point takes at most


def moe_gemm_noalloc(fmt, xq, w, n_experts, ids, topk, T, N, K, out, stream=None):
    """Indexed MoE as ``moe_gemm``, with the routing tables in the library's
    static device scratch instead of a workspace: nothing is allocated,
    here or in the library (``out`` must be given).  Calls that overlap in
    time on one GPU race on that scratch.  T * topk <= MOE_NOALLOC_MAX_ROUTED."""
    import torch
    _check_moe_sizes(fmt, xq, w, n_experts, topk, T, N, K, out, None)
    if _dims_ok(T, topk):
        _need(ids, torch.int32, T * topk, "ids")
    _check(lib().mmq_moe_gemm_noalloc(fmt, _ptr(xq), _ptr(w), n_experts, _ptr(ids, torch.int32), topk,
                                      _ptr(out, torch.float32), T, N, K, _stream(stream)), "mmq_moe_gemm_noalloc")
    return out


def debug_block_dots(fmt, xq, w, M, N, K, dots=None, stream=None):
    """Exact int32 block dots [M, N, K/32] through the GEMM's own staging and
    MFMA code (Q6_K: [M, N, K/16], one per 16-element scale group)."""
    import torch
    per = K // 16 if fmt == FMT_Q6_K else K // 32
    if dots is None:
        dots = torch.empty((M, N, per), dtype=torch.int32, device=xq.device)
    if _dims_ok(M, N, K):
        _need(xq, torch.uint8, M * (K // 32) * Q8_1_BYTES, "xq (q8_1 activations)")
        _need(w, torch.uint8, N * row_bytes(fmt, K), "w (weights)")
        _need(dots, torch.int32, M * N * per, "dots")
    _check(lib().mmq_debug_block_dots(fmt, _ptr(xq), _ptr(w), _ptr(dots, torch.int32), M, N, K,
                                      _stream(stream)), "mmq_debug_block_dots")
    return dots


def plan_describe(fmt, M, N, K) -> tuple[bool, str]:
    buf = ctypes.create_string_buffer(512)
    ok = lib().mmq_plan_describe(fmt, M, N, K, buf, 512)
    return bool(ok), buf.value.decode()


def plan_for_limits(fmt, M, N, K, lds_limit, cu_count, vgprs=0, scratch=0) -> tuple[bool, str]:
    """Pure host planning; ``vgprs``/``scratch``: the launched kernel's
    registers and scratch bytes per lane (0 registers: the built budget)."""
    buf = ctypes.create_string_buffer(512)
    ok = lib().mmq_plan_for_limits(fmt, M, N, K, lds_limit, cu_count, vgprs, scratch, buf, 512)
    return bool(ok), buf.value.decode()


def set_extra_lds(nbytes: int) -> None:
    lib().mmq_debug_set_extra_lds(nbytes)


def version() -> str:
    return lib().mmq_version().decode()
