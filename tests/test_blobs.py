"""The probe tests' blob packer (tests/blobs.py) lays codes and scale/bias
words where the oracle's readers find them."""
import numpy as np
import pytest

import oracle
from blobs import BF16_ONE, pack_blob


@pytest.mark.parametrize("bits", [4, 2])
def test_pack_blob_read_back_by_the_oracle(bits):
    D, I = 128, 64
    rng = np.random.default_rng(bits)
    top = 1 << bits
    gate, up = rng.integers(0, top, size=(I, D)), rng.integers(0, top, size=(I, D))
    down = rng.integers(0, top, size=(D, I))
    sb = []
    for rows, cols in ((I, D), (I, D), (D, I)):
        s = rng.integers(0x3C00, 0x3D00, size=(rows, cols // 64))      # bf16 in [2^-7, 2^-5)
        b = rng.integers(0xBC00, 0xBD00, size=(rows, cols // 64))      # negative, same range
        sb.append((s, b))
    blob = pack_blob(gate, up, down, bits, sb=sb)
    assert blob.size == oracle.blob_bytes(D, I, bits, 64)
    for m, mat in enumerate((gate, up, down)):
        rows, cols = mat.shape
        for i in rng.integers(0, rows, size=6):
            for j in rng.integers(0, cols, size=6):
                assert oracle.q(blob, D, I, bits, m, int(i), int(j)) == mat[i, j]
                s, b = oracle.sb(blob, D, I, bits, 64, m, int(i), int(j))
                hs, hb = int(sb[m][0][i, j // 64]), int(sb[m][1][i, j // 64])
                assert s == np.frombuffer(np.uint32(hs << 16).tobytes(), np.float32)[0]
                assert b == np.frombuffer(np.uint32(hb << 16).tobytes(), np.float32)[0]
    one = pack_blob(gate, up, down, bits)
    assert oracle.sb(one, D, I, bits, 64, 0, 0, 0) == (1.0, 0.0)
    assert BF16_ONE == 0x3F80
