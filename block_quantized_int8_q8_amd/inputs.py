"""Seeded synthetic inputs for the MMQ path.

This module only draws random numbers and places them in the documented
byte layouts.  It holds none of the method's arithmetic (no amax, no
rounding to codes, no scale products, no dot products), so that the CPU
oracle and the GPU library can both be fed from it without sharing code.

Distributions follow the 7B prefill workloads the library is measured on:
  * activations: fp32 standard normal, M x K row-major;
  * Q8_0 weights: int8 codes uniform on [-127, 127], fp16 scale d drawn
    uniform on [1e-3, 1e-2] in fp64 and rounded to fp16 by numpy;
  * Q4_K weights: 4-bit codes uniform on 0..15, the sixteen 6-bit
    scales/mins uniform on 0..63 (12 uniformly random bytes: every bit of
    the 12-byte field feeds exactly one 6-bit value, so uniform bytes give
    uniform values), fp16 d uniform on [1e-3, 1e-2], fp16 dmin uniform on
    [0, 1e-2].
  * Q5_K weights: as Q4_K, plus 32 uniformly random high-bit bytes (each
    code's fifth bit uniform).
  * Q6_K weights: 128 low-bit and 64 high-bit bytes uniformly random (each
    6-bit code uniform on 0..63), the sixteen int8 scales uniform on
    -128..127, fp16 d uniform on [1e-4, 1e-3].
Seeds are ``1000 * config + tensor_id`` with numpy's PCG64.

Block layouts (little-endian):
  q8_1 (36 B):  fp16 d @0, fp16 s @2, 32 x int8 @4
  Q8_0 (34 B):  fp16 d @0, 32 x int8 @2
  Q4_K (144 B): fp16 d @0, fp16 dmin @2, 12 B scales/mins @4, 128 B codes @16
  Q5_K (176 B): fp16 d @0, fp16 dmin @2, 12 B scales/mins @4, 32 B high bits
                @16, 128 B low nibbles @48
  Q6_K (210 B): 128 B low four bits @0, 64 B high two bits @128, 16 x int8
                scales @192, fp16 d @208
"""
from __future__ import annotations

import numpy as np

Q8_1_BYTES = 36
Q8_0_BYTES = 34
Q4_K_BYTES = 144
Q5_K_BYTES = 176
Q6_K_BYTES = 210


def seed_for(config: int, tensor_id: int) -> int:
    return 1000 * config + tensor_id


def _f16_bytes(values: np.ndarray) -> np.ndarray:
    """fp64 draws -> fp16 (numpy round-to-nearest-even) -> 2 little-endian bytes."""
    h = np.asarray(values, dtype=np.float64).astype(np.float16)
    return h.astype("<f2").view(np.uint8).reshape(h.shape + (2,))


def activations(M: int, K: int, seed: int) -> np.ndarray:
    """fp32 M x K, standard normal."""
    return np.random.default_rng(seed).standard_normal((M, K), dtype=np.float32)


def activations_device(M: int, K: int, seed: int, device) -> "torch.Tensor":
    """fp32 M x K, standard normal, drawn on the device by torch's seeded
    generator: for sizes (several GB) the host would take too long to draw.
    The tests read back the rows they check and hand those to the oracle."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((M, K), generator=g, dtype=torch.float32, device=device)


def q8_0_weights(N: int, K: int, seed: int, d_range=(1e-3, 1e-2),
                 d_value: float | None = None) -> np.ndarray:
    """uint8 N x (K/32) x 34.  ``d_value`` fixes every scale (e.g. 1.0)."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    kb = K // 32
    r = np.random.default_rng(seed)
    d = np.full((N, kb), d_value) if d_value is not None else r.uniform(*d_range, size=(N, kb))
    qs = r.integers(-127, 127, size=(N, kb, 32), endpoint=True, dtype=np.int8)
    out = np.empty((N, kb, Q8_0_BYTES), dtype=np.uint8)
    out[..., 0:2] = _f16_bytes(d)
    out[..., 2:34] = qs.view(np.uint8)
    return out


def q4_K_weights(N: int, K: int, seed: int, d_range=(1e-3, 1e-2), dmin_range=(0.0, 1e-2),
                 d_value: float | None = None, dmin_value: float | None = None,
                 scale_bytes: np.ndarray | None = None,
                 code_byte: int | None = None) -> np.ndarray:
    """uint8 N x (K/256) x 144.

    ``d_value`` / ``dmin_value`` fix the super-block scales, ``scale_bytes``
    (12 bytes) fixes the packed scale/min field, ``code_byte`` fixes every
    code byte; whatever is not fixed is drawn at random."""
    if K % 256:
        raise ValueError("K must be a multiple of 256")
    nsb = K // 256
    r = np.random.default_rng(seed)
    d = np.full((N, nsb), d_value) if d_value is not None else r.uniform(*d_range, size=(N, nsb))
    dmin = (np.full((N, nsb), dmin_value) if dmin_value is not None
            else r.uniform(*dmin_range, size=(N, nsb)))
    sc = r.integers(0, 255, size=(N, nsb, 12), endpoint=True, dtype=np.uint8)
    qs = r.integers(0, 255, size=(N, nsb, 128), endpoint=True, dtype=np.uint8)
    if scale_bytes is not None:
        sc[...] = np.asarray(scale_bytes, dtype=np.uint8).reshape(12)
    if code_byte is not None:
        qs[...] = np.uint8(code_byte)
    out = np.empty((N, nsb, Q4_K_BYTES), dtype=np.uint8)
    out[..., 0:2] = _f16_bytes(d)
    out[..., 2:4] = _f16_bytes(dmin)
    out[..., 4:16] = sc
    out[..., 16:144] = qs
    return out


def q5_K_weights(N: int, K: int, seed: int, d_range=(1e-3, 1e-2), dmin_range=(0.0, 1e-2),
                 d_value: float | None = None, dmin_value: float | None = None,
                 scale_bytes: np.ndarray | None = None, code_byte: int | None = None,
                 high_byte: int | None = None) -> np.ndarray:
    """uint8 N x (K/256) x 176: fp16 d, fp16 dmin, 12 scale/min bytes, 32
    high-bit bytes, 128 low-nibble bytes.  ``high_byte`` fixes every high-bit
    byte; the other keywords as for ``q4_K_weights``."""
    if K % 256:
        raise ValueError("K must be a multiple of 256")
    nsb = K // 256
    r = np.random.default_rng(seed)
    d = np.full((N, nsb), d_value) if d_value is not None else r.uniform(*d_range, size=(N, nsb))
    dmin = (np.full((N, nsb), dmin_value) if dmin_value is not None
            else r.uniform(*dmin_range, size=(N, nsb)))
    sc = r.integers(0, 255, size=(N, nsb, 12), endpoint=True, dtype=np.uint8)
    qh = r.integers(0, 255, size=(N, nsb, 32), endpoint=True, dtype=np.uint8)
    qs = r.integers(0, 255, size=(N, nsb, 128), endpoint=True, dtype=np.uint8)
    if scale_bytes is not None:
        sc[...] = np.asarray(scale_bytes, dtype=np.uint8).reshape(12)
    if code_byte is not None:
        qs[...] = np.uint8(code_byte)
    if high_byte is not None:
        qh[...] = np.uint8(high_byte)
    out = np.empty((N, nsb, Q5_K_BYTES), dtype=np.uint8)
    out[..., 0:2] = _f16_bytes(d)
    out[..., 2:4] = _f16_bytes(dmin)
    out[..., 4:16] = sc
    out[..., 16:48] = qh
    out[..., 48:176] = qs
    return out


def q6_K_weights(N: int, K: int, seed: int, d_range=(1e-4, 1e-3), d_value: float | None = None,
                 scale_value: int | None = None, low_byte: int | None = None,
                 high_byte: int | None = None) -> np.ndarray:
    """uint8 N x (K/256) x 210.  ``scale_value`` fixes all sixteen int8
    scales, ``low_byte`` / ``high_byte`` every low-bit / high-bit byte."""
    if K % 256:
        raise ValueError("K must be a multiple of 256")
    nsb = K // 256
    r = np.random.default_rng(seed)
    d = np.full((N, nsb), d_value) if d_value is not None else r.uniform(*d_range, size=(N, nsb))
    ql = r.integers(0, 255, size=(N, nsb, 128), endpoint=True, dtype=np.uint8)
    qh = r.integers(0, 255, size=(N, nsb, 64), endpoint=True, dtype=np.uint8)
    sc = r.integers(-128, 127, size=(N, nsb, 16), endpoint=True, dtype=np.int8)
    if scale_value is not None:
        sc[...] = np.int8(scale_value)
    if low_byte is not None:
        ql[...] = np.uint8(low_byte)
    if high_byte is not None:
        qh[...] = np.uint8(high_byte)
    out = np.empty((N, nsb, Q6_K_BYTES), dtype=np.uint8)
    out[..., 0:128] = ql
    out[..., 128:192] = qh
    out[..., 192:208] = sc.view(np.uint8)
    out[..., 208:210] = _f16_bytes(d)
    return out


def q8_1_blocks(M: int, K: int, seed: int, d_range=(5e-3, 5e-2), s_range=(-2.0, 2.0)) -> np.ndarray:
    """uint8 M x (K/32) x 36 with independent random fields.

    For tests of the contraction alone: the d and s fields are arbitrary fp16
    values and the codes are uniform on [-127, 127]; nothing ties s to the
    codes, because the contraction only reads the fields."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    kb = K // 32
    r = np.random.default_rng(seed)
    d = r.uniform(*d_range, size=(M, kb))
    s = r.uniform(*s_range, size=(M, kb))
    qs = r.integers(-127, 127, size=(M, kb, 32), endpoint=True, dtype=np.int8)
    out = np.empty((M, kb, Q8_1_BYTES), dtype=np.uint8)
    out[..., 0:2] = _f16_bytes(d)
    out[..., 2:4] = _f16_bytes(s)
    out[..., 4:36] = qs.view(np.uint8)
    return out


# The benchmarked shapes (M, N, K) by config number; config 5 is the set of
# seven projection GEMMs of one 7B layer (q, k, v, o, gate, up, down).
CONFIGS = {
    1: ("q8_0", 64, 256, 512),
    2: ("q8_0", 2048, 3584, 3584),
    3: ("q4_K", 2048, 18944, 3584),
    4: ("q4_K", 2048, 3584, 18944),
}

LAYER_7B = [  # (name, N, K) -- hidden 3584, 28 q heads / 4 kv heads of 128, ffn 18944
    ("q", 3584, 3584),
    ("k", 512, 3584),
    ("v", 512, 3584),
    ("o", 3584, 3584),
    ("gate", 18944, 3584),
    ("up", 18944, 3584),
    ("down", 3584, 18944),
]

# Config 5: the layer's GEMMs at these token counts, Q4_K weights.  GEMMs that
# read the same activations share one q8_1 quantize pass: q, k and v read the
# attention input, gate and up the FFN input.
LAYER_M = (512, 2048, 8192)
LAYER_INPUTS = [  # (input name, K, GEMMs reading it)
    ("attn_in", 3584, ("q", "k", "v")),
    ("o_in", 3584, ("o",)),
    ("ffn_in", 3584, ("gate", "up")),
    ("down_in", 18944, ("down",)),
]


def layer_weight_seed(gemm: str) -> int:
    """One weight tensor per projection, the same at every token count."""
    return seed_for(5, 10 + [g for g, _, _ in LAYER_7B].index(gemm))


def layer_activation_seed(M: int, input_name: str) -> int:
    return seed_for(5, 100 + 4 * LAYER_M.index(M) + [n for n, _, _ in LAYER_INPUTS].index(input_name))


# Indexed MoE (a Qwen3-30B-A3B-shaped layer: 128 experts, 8 per token,
# hidden 2048, expert FFN 768).
MOE_SHAPE = {"n_experts": 128, "topk": 8, "hidden": 2048, "ffn": 768}
MOE_T = 2048   # prefill tokens
# The two expert GEMMs of the layer: gate and up fused into one N = 2 * ffn
# matrix per expert, reading the T token rows (topk routed rows per token);
# down reading the T * topk routed rows (one expert each, topk = 1).
MOE_GEMMS = [  # (name, N, K, rows read per routed row: "token" or "routed")
    ("gate_up", 2 * MOE_SHAPE["ffn"], MOE_SHAPE["hidden"], "token"),
    ("down", MOE_SHAPE["hidden"], MOE_SHAPE["ffn"], "routed"),
]


def moe_seed(name: str) -> int:
    """Seeds of the MoE layer's tensors: expert weights, activations, routing."""
    return seed_for(6, ["ids", "gate_up_w", "down_w", "gate_up_x", "down_x"].index(name))


def moe_ids(T: int, n_experts: int, topk: int, seed: int, skew: float = 0.0) -> np.ndarray:
    """int32 [T, topk]: topk distinct experts per token.  Expert e is drawn
    with probability proportional to (e + 1) ** -skew (skew 0: uniform), by
    Gumbel top-k sampling without replacement."""
    if not 1 <= topk <= n_experts:
        raise ValueError("need 1 <= topk <= n_experts")
    r = np.random.default_rng(seed)
    logp = -skew * np.log(np.arange(1, n_experts + 1, dtype=np.float64))
    scores = logp[None, :] + r.gumbel(size=(T, n_experts))
    ids = np.argpartition(-scores, topk - 1, axis=1)[:, :topk]
    return ids.astype(np.int32)

