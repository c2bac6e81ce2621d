"""Independent numpy decoders of the block layouts, used to pin the oracle.

Written from the layout description (q8_1: fp16 d @0, fp16 s @2, int8 codes
@4; Q8_0: fp16 d @0, int8 codes @2; Q4_K: fp16 d @0, fp16 dmin @2, 12 bytes
of 6-bit scales/mins @4, 128 bytes of 4-bit codes @16) with numpy's own
fp16 type, vectorised, and without the oracle's loop structure.
"""
import numpy as np


def f16(b2: np.ndarray) -> np.ndarray:
    """(..., 2) little-endian bytes -> float64 via numpy's binary16."""
    b2 = np.ascontiguousarray(b2, dtype=np.uint8)
    return b2.view("<f2")[..., 0].astype(np.float64)


def q8_1_fields(x):
    """-> (d f64 [M,kb], s f64 [M,kb], codes int64 [M,kb,32])."""
    return f16(x[..., 0:2]), f16(x[..., 2:4]), x[..., 4:36].view(np.int8).astype(np.int64)


def q8_0_fields(w):
    return f16(w[..., 0:2]), w[..., 2:34].view(np.int8).astype(np.int64)


def q4_K_fields(w):
    """-> (d [N,nsb], dmin [N,nsb], sc [N,nsb,8], mn [N,nsb,8], codes [N,nsb,256])."""
    d = f16(w[..., 0:2])
    dmin = f16(w[..., 2:4])
    s = w[..., 4:16].astype(np.int64)
    sc = np.empty(s.shape[:-1] + (8,), np.int64)
    mn = np.empty_like(sc)
    # sub-blocks 0..3: low six bits of bytes 0..3 (scale) and 4..7 (min)
    sc[..., 0:4] = s[..., 0:4] & 63
    mn[..., 0:4] = s[..., 4:8] & 63
    # sub-blocks 4..7: nibbles of bytes 8..11 plus the top two bits of 0..3 / 4..7
    sc[..., 4:8] = (s[..., 8:12] & 15) | ((s[..., 0:4] >> 6) << 4)
    mn[..., 4:8] = (s[..., 8:12] >> 4) | ((s[..., 4:8] >> 6) << 4)
    q = w[..., 16:144].astype(np.int64).reshape(w.shape[:-1] + (4, 32))  # 4 groups of 32 bytes
    lo = q & 15   # group g, byte i, low nibble  -> element 64g + i
    hi = q >> 4   # group g, byte i, high nibble -> element 64g + 32 + i
    codes = np.stack([lo, hi], axis=-2).reshape(w.shape[:-1] + (256,))
    return d, dmin, sc, mn, codes


def q5_K_fields(w):
    """-> (d, dmin, sc, mn, codes 0..31 [N,nsb,256]): the Q4_K fields of bytes
    0..15 and 48..175, plus 16 x bit (e // 32) of high-bit byte e % 32."""
    d = f16(w[..., 0:2])
    dmin = f16(w[..., 2:4])
    s = w[..., 4:16].astype(np.int64)
    sc = np.empty(s.shape[:-1] + (8,), np.int64)
    mn = np.empty_like(sc)
    sc[..., 0:4] = s[..., 0:4] & 63
    mn[..., 0:4] = s[..., 4:8] & 63
    sc[..., 4:8] = (s[..., 8:12] & 15) | ((s[..., 0:4] >> 6) << 4)
    mn[..., 4:8] = (s[..., 8:12] >> 4) | ((s[..., 4:8] >> 6) << 4)
    q = w[..., 48:176].astype(np.int64).reshape(w.shape[:-1] + (4, 32))
    low = np.stack([q & 15, q >> 4], axis=-2).reshape(w.shape[:-1] + (256,))
    qh = w[..., 16:48].astype(np.int64)                                   # [..., 32]
    high = (qh[..., None, :] >> np.arange(8)[:, None]) & 1               # [..., 8 (bit j), 32 (byte l)]
    return d, dmin, sc, mn, low + 16 * high.reshape(w.shape[:-1] + (256,))


def dequant_q5_K(w) -> np.ndarray:
    """-> f64 N x K: d*sc*q - dmin*m with 5-bit q."""
    d, dmin, sc, mn, codes = q5_K_fields(w)
    N, nsb = d.shape
    c = codes.reshape(N, nsb, 8, 32)
    val = (d[..., None, None] * sc[..., None]) * c - (dmin[..., None] * mn)[..., None]
    return val.reshape(N, -1)


def dequant_q8_0(w) -> np.ndarray:
    """-> f64 N x K (exact: fp16 x int8)."""
    d, q = q8_0_fields(w)
    return (d[..., None] * q).reshape(w.shape[0], -1)


def dequant_q4_K(w) -> np.ndarray:
    """-> f64 N x K: d*sc*q - dmin*m (exact in fp64)."""
    d, dmin, sc, mn, codes = q4_K_fields(w)
    N, nsb = d.shape
    c = codes.reshape(N, nsb, 8, 32)
    val = (d[..., None, None] * sc[..., None]) * c - (dmin[..., None] * mn)[..., None]
    return val.reshape(N, -1)


def dequant_q8_1(x) -> np.ndarray:
    d, _, q = q8_1_fields(x)
    return (d[..., None] * q).reshape(x.shape[0], -1)


def q6_K_fields(w):
    """-> (d f64 [N,nsb], sc int64 [N,nsb,16], codes 0..63 int64 [N,nsb,256]).
    Low bits: the 128 bytes @0 as [half 2][row 2][32]; quarter q of a half
    takes row q%2, low nibble for q < 2 and high nibble for q >= 2.  High
    bits: the 64 bytes @128 as [half 2][32]; quarter q takes bits 2q, 2q+1.
    Scales: 16 int8 @192 (one per 16 elements); d: fp16 @208."""
    ql = w[..., 0:128].astype(np.int64).reshape(w.shape[:-1] + (2, 2, 32))
    qh = w[..., 128:192].astype(np.int64).reshape(w.shape[:-1] + (2, 32))
    low = np.stack([ql[..., 0, :] & 15, ql[..., 1, :] & 15, ql[..., 0, :] >> 4, ql[..., 1, :] >> 4], axis=-2)
    high = np.stack([(qh >> (2 * q)) & 3 for q in range(4)], axis=-2)        # [..., half, quarter, 32]
    codes = (low + 16 * high).reshape(w.shape[:-1] + (256,))
    sc = w[..., 192:208].view(np.int8).astype(np.int64)
    return f16(w[..., 208:210]), sc, codes


def dequant_q6_K(w) -> np.ndarray:
    """-> f64 N x K: d*sc*(code - 32) (exact in fp64)."""
    d, sc, codes = q6_K_fields(w)
    N, nsb = d.shape
    c = (codes - 32).reshape(N, nsb, 16, 16)
    return ((d[..., None, None] * sc[..., None]) * c).reshape(N, -1)
