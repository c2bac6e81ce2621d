"""Host checks of the tile-packed Q8_0 form: the library's size function,
the numpy model of the layout the header states (a permutation of the Q8_0
bytes, zero padding), and the binding's buffer checks.  No GPU needed."""
import numpy as np
import pytest

import block_quantized_int8_q8_amd as mmq
from tests import nppack


@pytest.mark.parametrize("N,K", [(1, 32), (127, 96), (128, 128), (129, 160), (300, 544), (3584, 3584),
                                 (18944, 3584), (3584, 18944), (5, 8388608)])
def test_packed_bytes(N, K):
    tiles, steps = -(-N // 128), -(-(K // 32) // 4)
    assert mmq.packed_bytes_q8_0(N, K) == tiles * steps * 17408 == nppack.packed_bytes(N, K)


@pytest.mark.parametrize("N,K", [(0, 128), (4, 0), (4, 48), (4, 16), (4, 8388608 + 32), (2 ** 31, 32)])
def test_packed_bytes_refuses(N, K):
    with pytest.raises(mmq.MMQError, match="multiple of 32|N must be"):
        mmq.packed_bytes_q8_0(N, K)


@pytest.mark.parametrize("N,K,seed", [(1, 32, 1), (127, 96, 2), (128, 128, 3), (130, 160, 4), (300, 544, 5),
                                      (257, 3616, 6)])
def test_numpy_pack_is_a_permutation_with_zero_padding(N, K, seed):
    rng = np.random.default_rng(seed)
    w = rng.integers(1, 256, size=(N, K // 32, 34), dtype=np.uint8)   # no zero byte: padding stands out
    p = nppack.pack(w, N, K)
    assert p.size == nppack.packed_bytes(N, K)
    assert np.array_equal(nppack.unpack(p, N, K), w)
    assert nppack.padding_is_zero(p, N, K)
    # every valid byte appears exactly once: as many non-zero bytes as the input has
    assert np.count_nonzero(p) == w.size


def test_numpy_pack_places_a_block_where_the_header_says():
    """One hand-placed block: column 13 of tile 1 (n = 141), block 6 (step
    1, block 2 of the step); column 13 has bits 2 and 3 equal (1101b), so its
    halves are not swapped; column 4 (0100b) has them swapped."""
    N, K = 200, 256
    w = np.zeros((N, K // 32, 34), np.uint8)
    w[141, 6, :2] = [0x34, 0x12]
    w[141, 6, 2:] = np.arange(1, 33, dtype=np.uint8)
    w[132, 1, 2:18] = 0xAA      # column 4 of tile 1, block 1, low half
    p = nppack.pack(w, N, K).reshape(2, 2, 17408)
    img = p[1, 1]
    base = 2 * 128 * 32 + 13 * 32
    assert np.array_equal(img[base:base + 32], np.arange(1, 33, dtype=np.uint8))
    s = 4 * 128 * 32 + (2 * 128 + 13) * 2
    assert list(img[s:s + 2]) == [0x34, 0x12]
    img0 = p[1, 0]
    b4 = 1 * 128 * 32 + 4 * 32
    assert (img0[b4 + 16:b4 + 32] == 0xAA).all() and not img0[b4:b4 + 16].any()


def test_binding_refuses_short_packed_buffers():
    import torch
    N, K, M = 130, 256, 3
    nb = mmq.packed_bytes_q8_0(N, K)
    w = torch.zeros(N * mmq.row_bytes(mmq.FMT_Q8_0, K), dtype=torch.uint8)
    with pytest.raises(ValueError, match="w"):
        mmq.pack_q8_0(w[:-1], N, K)
    with pytest.raises(ValueError, match="packed"):
        mmq.pack_q8_0(w, N, K, torch.zeros(nb - 1, dtype=torch.uint8))
    xq = torch.zeros(M * (K // 32) * 36, dtype=torch.uint8)
    out = torch.zeros(M * N, dtype=torch.float32)
    pk = torch.zeros(nb, dtype=torch.uint8)
    with pytest.raises(ValueError, match="packed"):
        mmq.gemm_q8_0_packed(xq, pk[:-1], M, N, K, out)
    with pytest.raises(ValueError, match="xq"):
        mmq.gemm_q8_0_packed(xq[:-1], pk, M, N, K, out)
    with pytest.raises(ValueError, match="out"):
        mmq.gemm_q8_0_packed(xq, pk, M, N, K, out[:-1])
    with pytest.raises(ValueError, match="GPU"):   # sizes fine: the device check is next
        mmq.gemm_q8_0_packed(xq, pk, M, N, K, out)
