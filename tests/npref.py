"""Test-side dense references in numpy (independent of the C oracle).

These re-derive the method from its plain definition with whole-matrix numpy
operations, so the oracle's element-at-a-time code can be checked against a
differently structured implementation on small inputs.
"""
import numpy as np

MATS = ("gate", "up", "down")


def dims(D, I, mat):
    return (D, I) if mat in (2, "down") else (I, D)


def unpack(blob, D, I, bits, group):
    """Dense fp64 gate [I][D], up [I][D], down [D][I] from a canonical blob,
    read byte-wise: inside a byte the lowest bits hold the earliest element."""
    blob = np.asarray(blob, dtype=np.uint8)
    per = 8 // bits
    mat_bytes = D * I * bits // 8
    sb0 = 3 * mat_bytes
    sb_words = np.frombuffer(blob[sb0:].tobytes(), dtype="<u4")
    out = {}
    off_sb = 0
    for m, name in enumerate(MATS):
        rows, cols = dims(D, I, name)
        raw = blob[m * mat_bytes:(m + 1) * mat_bytes]
        codes = np.stack([(raw >> (bits * k)) & ((1 << bits) - 1) for k in range(per)], axis=-1)
        q = codes.reshape(rows, cols).astype(np.float64)
        ng = rows * cols // group
        wsb = sb_words[off_sb:off_sb + ng].reshape(rows, cols // group)
        off_sb += ng
        s = ((wsb & 0xFFFF).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        b = ((wsb >> 16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        s_full = np.repeat(s, group, axis=1)
        b_full = np.repeat(b, group, axis=1)
        out[name] = q * s_full + b_full
        out[name + "_q"] = q
    return out


def pack(qs, scales, biases, D, I, bits, group):
    """Inverse of unpack: build a canonical blob from integer codes and bf16
    bit patterns (dicts keyed by matrix name)."""
    per = 8 // bits
    parts = []
    for name in MATS:
        rows, cols = dims(D, I, name)
        q = np.asarray(qs[name], dtype=np.uint8).reshape(rows, cols // per, per)
        byte = np.zeros((rows, cols // per), dtype=np.uint8)
        for k in range(per):
            byte |= (q[:, :, k] << (bits * k)).astype(np.uint8)
        parts.append(byte.reshape(-1))
    for name in MATS:
        s = np.asarray(scales[name], dtype=np.uint32)
        b = np.asarray(biases[name], dtype=np.uint32)
        parts.append(((b << 16) | s).astype("<u4").view(np.uint8).reshape(-1))
    return np.concatenate(parts)


def silu(z):
    return z / (1.0 + np.exp(-z))


def expert(mats, x):
    g = mats["gate"] @ x
    u = mats["up"] @ x
    h = silu(g) * u
    return h, mats["down"] @ h


def bf16_bits(v):
    """bf16 bit pattern of a value that is exactly representable in bf16."""
    f = np.float32(v)
    u = int(f.view(np.uint32))
    assert u & 0xFFFF == 0, f"{v} is not a bf16 value"
    return u >> 16
