"""Hand-built canonical expert blobs for probe tests.

The canonical blob (include/moe.h) is [gate.q | up.q | down.q | gate.sb |
up.sb | down.sb]: gate and up [I][D], down [D][I], row-major; element c of a
row sits at bit offset c*bits of the row (little-endian words, so byte
c*bits/8, lowest bits first); one 32-bit word per 64-column group of a row,
bf16 scale in the low half and bf16 bias in the high half.  This module only
lays given codes and bf16 words out in that order; it holds none of the
method's arithmetic.
"""
import numpy as np

BF16_ONE = 0x3F80
BF16_ZERO = 0x0000


def pack_codes(q, bits):
    """Rows of unsigned codes [rows][cols] -> packed bytes."""
    q = np.asarray(q, dtype=np.uint8)
    per = 8 // bits
    rows, cols = q.shape
    assert cols % per == 0 and int(q.max(initial=0)) < (1 << bits)
    g = q.reshape(rows, cols // per, per).astype(np.uint32)
    byte = np.zeros((rows, cols // per), np.uint32)
    for k in range(per):
        byte |= g[:, :, k] << (bits * k)
    return byte.astype(np.uint8).reshape(-1)


def pack_sb(scale_bf16, bias_bf16):
    """bf16 bit patterns [rows][groups] -> sb words as bytes."""
    w = (np.asarray(scale_bf16, np.uint32) & 0xFFFF) | ((np.asarray(bias_bf16, np.uint32) & 0xFFFF) << 16)
    return w.astype("<u4").view(np.uint8).reshape(-1)


def pack_blob(gate_q, up_q, down_q, bits, sb=None, group=64):
    """A canonical blob from codes gate/up [I][D] and down [D][I]; sb: None
    (scale 1, bias 0 everywhere) or three (scale, bias) pairs of bf16 bit
    patterns [rows][cols / group]."""
    I, D = np.shape(gate_q)
    assert np.shape(up_q) == (I, D) and np.shape(down_q) == (D, I)
    parts = [pack_codes(gate_q, bits), pack_codes(up_q, bits), pack_codes(down_q, bits)]
    for m, (rows, cols) in enumerate(((I, D), (I, D), (D, I))):
        if sb is None:
            s = np.full((rows, cols // group), BF16_ONE)
            b = np.full((rows, cols // group), BF16_ZERO)
        else:
            s, b = sb[m]
        parts.append(pack_sb(s, b))
    return np.concatenate(parts)
