"""CPU checks of the host-side unpacker of the bit-plane index that the GPU
plane tests rely on: it must invert the layout's definition (word j of row
(b, l) of tile t holds bit b of table l's codes for keys 512 t + 32 j + e at
bit e), which is packed here key by key."""
import numpy as np

from tests.test_gpu_planes import planes_to_codes


def pack_by_definition(codes, K):
    U, L, n = codes.shape
    T = n // 512
    p = np.zeros((U, T, K, L, 16), np.uint32)
    for u in range(U):
        for l in range(L):
            for i in range(n):
                c = int(codes[u, l, i])
                for b in range(K):
                    if (c >> b) & 1:
                        p[u, i // 512, b, l, (i % 512) // 32] |= np.uint32(1 << (i % 32))
    return p.view(np.int32)


def test_unpacker_inverts_the_layout():
    rng = np.random.default_rng(11)
    for K, L in ((5, 3), (10, 2), (16, 1)):
        codes = rng.integers(0, 1 << K, size=(2, L, 1024), dtype=np.uint32)
        planes = pack_by_definition(codes, K)
        assert np.array_equal(planes_to_codes(planes, K, L), codes), (K, L)


def test_one_word_by_hand():
    codes = np.zeros((1, 2, 512), np.uint32)
    codes[0, 1, 37] = 0b101  # key 37 = word 1, bit 5
    planes = pack_by_definition(codes, 3).view(np.uint32)
    assert planes[0, 0, 0, 1, 1] == 1 << 5 and planes[0, 0, 2, 1, 1] == 1 << 5
    assert planes[0, 0, 1].sum() == 0 and planes[0, 0, :, 0].sum() == 0
    assert np.count_nonzero(planes) == 2
    assert planes_to_codes(planes.view(np.int32), 3, 2)[0, 1, 37] == 0b101
