"""The seeded input generator: determinism, sub-range regeneration and the
stated distributions (uniform codes, bf16 scale/bias ranges, normals)."""
import numpy as np

import seedgen


def test_blob_deterministic_and_distinct():
    c = seedgen.CONFIGS["tiny"]
    a = seedgen.blob(c, 0, 3)
    assert np.array_equal(a, seedgen.blob(c, 0, 3))
    assert not np.array_equal(a, seedgen.blob(c, 0, 4))
    assert not np.array_equal(a, seedgen.blob(c, 1, 3))
    assert not np.array_equal(a, seedgen.blob(c.replace(seed=c.seed + 1), 0, 3))
    assert a.size == c.blob_bytes


def test_subrange_regeneration():
    k = seedgen.key(1, 2, 3, 0)
    full = seedgen.words(k, 1001)
    assert np.array_equal(full[37:500], seedgen.words(k, 463, w0=37))


def test_code_uniformity():
    c = seedgen.CONFIGS["layer"].replace(D=1024, I=512)
    b = seedgen.blob(c, 0, 0)
    q = b[: 3 * c.D * c.I // 2]
    nib = np.concatenate([q & 15, q >> 4])
    counts = np.bincount(nib, minlength=16)
    exp = nib.size / 16
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < 60, chi2   # 15 dof; p ~ 1e-7 at 60


def test_scale_bias_ranges_and_bf16():
    c = seedgen.CONFIGS["tiny"]
    b = seedgen.blob(c, 0, 1)
    sb = b[3 * c.D * c.I // 2:].view("<u4")
    s = ((sb & 0xFFFF) << 16).astype(np.uint32).view(np.float32)
    bias = ((sb >> 16) << 16).astype(np.uint32).view(np.float32)
    assert s.min() >= np.float32(0.005) * (1 - 2**-8) and s.max() <= 0.02 * (1 + 2**-8)
    assert bias.min() >= -0.1 * (1 + 2**-8) and bias.max() <= 0.0
    assert s.std() > 0.003 and bias.std() > 0.02


def test_bf16_rne():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert seedgen.bf16_rne(1.0 + 2**-8) == 0x3F80
    assert seedgen.bf16_rne(1.0 + 3 * 2**-8) == 0x3F82
    assert seedgen.bf16_rne(-0.5) == 0xBF00


def test_normal_moments():
    x = seedgen.normal(seedgen.key(5, 0, 0, 3), 200001, 0.02)
    assert abs(x.mean()) < 3 * 0.02 / np.sqrt(x.size) * 1.5
    assert abs(x.std() / 0.02 - 1) < 0.01
    assert abs(((x / 0.02) ** 4).mean() - 3) < 0.1
