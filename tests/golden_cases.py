"""Build the inputs described by the hand-derived fixtures in tests/golden/."""
import json
import os

import numpy as np

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def q8_1_blocks():
    """-> (x fp32 [n, 32], expected d bits, s bits, codes [n, 32])."""
    spec = json.load(open(os.path.join(HERE, "q8_1_hand.json")))["blocks"]
    xs, d, s, codes = [], [], [], []
    for b in spec:
        x = np.zeros(32, np.float32)
        c = np.zeros(32, np.int64)
        if b["x"] == "tie":
            i = np.arange(31)
            x[:31] = (i + 0.5) / 4
            x[31] = 31.75
            c[:31] = i + 1
            c[31] = 127
        elif b["x"] == "integer":
            i = np.arange(31)
            x[:31] = i - 16
            x[31] = -127
            c[:] = x
        elif b["x"] == "onehot":
            x[5] = -2.0
            c[5] = -127
        elif b["x"] == "recip":
            x[0], x[1] = 9.0, 4.5
            c[0], c[1] = 127, 64
        xs.append(x)
        d.append(b["d_bits"])
        s.append(b["s_bits"])
        codes.append(c)
    return np.stack(xs), np.array(d, np.uint16), np.array(s, np.uint16), np.stack(codes)


def gemm_q8_0_case():
    """-> (x fp32 [1, K], w Q8_0 bytes [1, kb, 34], K, expected out)."""
    g = json.load(open(os.path.join(HERE, "gemm_hand.json")))["q8_0"]
    K = g["K"]
    x = np.zeros((1, K), np.float32)
    for k, v in g["x_nonzero"]:
        x[0, k] = v
    w = np.zeros((1, K // 32, 34), np.uint8)
    for b, sc in enumerate(g["w_scales"]):
        w[0, b, 0:2] = np.array([sc], "<f2").view(np.uint8)
    for k, v in g["w_nonzero"]:
        w[0, k // 32, 2 + k % 32] = np.int8(v).view(np.uint8)
    return x, w, K, g["out"]


def gemm_q4_K_case(pack_scale_min=None):
    """-> (x fp32 [1, K], w Q4_K bytes [1, 1, 144], K, expected out).

    The 12-byte scale field with every scale 2 and every min 3: bytes 0..3
    hold scale 2, bytes 4..7 hold min 3 (top bits 0), bytes 8..11 hold scale
    2 in the low nibble and min 3 in the high nibble -> 0x32."""
    g = json.load(open(os.path.join(HERE, "gemm_hand.json")))["q4_K"]
    K = g["K"]
    x = np.zeros((1, K), np.float32)
    x[0, ::32] = g["x_first_of_each_block"]
    w = np.zeros((1, 1, 144), np.uint8)
    w[0, 0, 0:2] = np.array([g["d"]], "<f2").view(np.uint8)
    w[0, 0, 2:4] = np.array([g["dmin"]], "<f2").view(np.uint8)
    w[0, 0, 4:8] = g["sc"]
    w[0, 0, 8:12] = g["m"]
    w[0, 0, 12:16] = g["sc"] | (g["m"] << 4)
    w[0, 0, 16:] = g["code"] | (g["code"] << 4)
    return x, w, K, g["out"]


def gemm_q5_K_case():
    """-> (x fp32 [1, K], w Q5_K bytes [1, 1, 176], K, expected out): the
    Q4_K case's fields plus a high-bit plane with only byte 0 non-zero."""
    g = json.load(open(os.path.join(HERE, "gemm_hand.json")))["q5_K"]
    K = g["K"]
    x = np.zeros((1, K), np.float32)
    x[0, ::32] = g["x_first_of_each_block"]
    w = np.zeros((1, 1, 176), np.uint8)
    w[0, 0, 0:2] = np.array([g["d"]], "<f2").view(np.uint8)
    w[0, 0, 2:4] = np.array([g["dmin"]], "<f2").view(np.uint8)
    w[0, 0, 4:8] = g["sc"]
    w[0, 0, 8:12] = g["m"]
    w[0, 0, 12:16] = g["sc"] | (g["m"] << 4)
    w[0, 0, 16] = g["high_byte_0"]
    w[0, 0, 48:] = g["code"] | (g["code"] << 4)
    return x, w, K, g["out"]


def gemm_q6_K_case():
    """-> (x fp32 [1, K], w Q6_K bytes [1, 1, 210], K, expected out): uniform
    low-bit and high-bit bytes, sixteen listed int8 scales, fp16 d."""
    g = json.load(open(os.path.join(HERE, "gemm_hand.json")))["q6_K"]
    K = g["K"]
    x = np.zeros((1, K), np.float32)
    x[0, ::16] = g["x_at_0_and_16_of_each_block"]
    w = np.zeros((1, 1, 210), np.uint8)
    w[0, 0, 0:128] = g["low_byte"]
    w[0, 0, 128:192] = g["high_byte"]
    w[0, 0, 192:208] = np.array(g["scales"], np.int8).view(np.uint8)
    w[0, 0, 208:210] = np.array([g["d"]], "<f2").view(np.uint8)
    return x, w, K, g["out"]
