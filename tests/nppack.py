"""Independent numpy model of the tile-packed Q8_0 layout (mmq_pack_q8_0).

Written from the layout the header states: for every 128-column tile t and
every step s of 4 blocks, one 17408-byte image -- the codes as
[block][column][32 bytes] with the two 16-byte halves swapped for the columns
c (within the tile) whose bits 2 and 3 differ, then the fp16 scales as
[block][column] -- columns past N and blocks past K/32 zero.  Test
infrastructure only: the library packs on the device; these functions say
what its bytes must be.
"""
import numpy as np

TILE, STEP_BLOCKS, IMG = 128, 4, 17408


def packed_bytes(N: int, K: int) -> int:
    kb = K // 32
    return -(-N // TILE) * -(-kb // STEP_BLOCKS) * IMG


def _swapped_columns() -> np.ndarray:
    c = np.arange(TILE)
    return ((c >> 2) & 1) != ((c >> 3) & 1)


def pack(w: np.ndarray, N: int, K: int) -> np.ndarray:
    """Q8_0 bytes (N x K/32 blocks of 34) -> packed bytes (uint8, flat)."""
    kb = K // 32
    tiles, steps = -(-N // TILE), -(-kb // STEP_BLOCKS)
    blocks = np.asarray(w, dtype=np.uint8).reshape(N, kb, 34)
    codes = np.zeros((tiles * TILE, steps * STEP_BLOCKS, 2, 16), np.uint8)
    scales = np.zeros((tiles * TILE, steps * STEP_BLOCKS, 2), np.uint8)
    codes[:N, :kb] = blocks[:, :, 2:].reshape(N, kb, 2, 16)
    scales[:N, :kb] = blocks[:, :, :2]
    # [tile][step][block][column][half][16]
    c = codes.reshape(tiles, TILE, steps, STEP_BLOCKS, 2, 16).transpose(0, 2, 3, 1, 4, 5).copy()
    sw = _swapped_columns()
    c[:, :, :, sw] = c[:, :, :, sw][:, :, :, :, ::-1, :]
    sc = scales.reshape(tiles, TILE, steps, STEP_BLOCKS, 2).transpose(0, 2, 3, 1, 4)
    img = np.concatenate([c.reshape(tiles, steps, -1), sc.reshape(tiles, steps, -1)], axis=2)
    assert img.shape[2] == IMG
    return np.ascontiguousarray(img).reshape(-1)


def unpack(p: np.ndarray, N: int, K: int) -> np.ndarray:
    """The inverse on the valid part: packed bytes -> Q8_0 bytes [N, K/32, 34]."""
    kb = K // 32
    tiles, steps = -(-N // TILE), -(-kb // STEP_BLOCKS)
    img = np.asarray(p, dtype=np.uint8).reshape(tiles, steps, IMG)
    c = img[:, :, :STEP_BLOCKS * TILE * 32].reshape(tiles, steps, STEP_BLOCKS, TILE, 2, 16).copy()
    sw = _swapped_columns()
    c[:, :, :, sw] = c[:, :, :, sw][:, :, :, :, ::-1, :]
    sc = img[:, :, STEP_BLOCKS * TILE * 32:].reshape(tiles, steps, STEP_BLOCKS, TILE, 2)
    codes = c.transpose(0, 3, 1, 2, 4, 5).reshape(tiles * TILE, steps * STEP_BLOCKS, 32)
    scales = sc.transpose(0, 3, 1, 2, 4).reshape(tiles * TILE, steps * STEP_BLOCKS, 2)
    out = np.concatenate([scales[:N, :kb], codes[:N, :kb]], axis=2)
    return np.ascontiguousarray(out)


def padding_is_zero(p: np.ndarray, N: int, K: int) -> bool:
    """Every byte of the packed form that belongs to no (column < N, block < K/32) is zero."""
    kb = K // 32
    tiles, steps = -(-N // TILE), -(-kb // STEP_BLOCKS)
    img = np.asarray(p, dtype=np.uint8).reshape(tiles, steps, IMG)
    c = img[:, :, :STEP_BLOCKS * TILE * 32].reshape(tiles, steps, STEP_BLOCKS, TILE, 32)
    sc = img[:, :, STEP_BLOCKS * TILE * 32:].reshape(tiles, steps, STEP_BLOCKS, TILE, 2)
    col = (np.arange(tiles)[:, None] * TILE + np.arange(TILE)[None, :])            # [tile][column]
    blk = (np.arange(steps)[:, None] * STEP_BLOCKS + np.arange(STEP_BLOCKS)[None, :])  # [step][block]
    pad = (col[:, None, None, :] >= N) | (blk[None, :, :, None] >= kb)             # [tile][step][block][column]
    return not c[pad].any() and not sc[pad].any()
