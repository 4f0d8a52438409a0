"""The quantiser's code arithmetic on the GPU: clamp(rint(t), -127, 127)
(rounding half to even) is computed as the low byte of the binary32 bit
pattern of fl(med3(t, -127, 127) + 1.5 * 2^23).  This scan checks that
identity on the CPU in IEEE binary32 arithmetic: every value within 64 ulps
of each integer and half-integer in [-130, 130], a million random values,
and large and infinite magnitudes."""
import numpy as np


def _codes_magic(vals):
    t = np.minimum(np.maximum(vals, np.float32(-127.0)), np.float32(127.0))
    m = (t + np.float32(12582912.0)).astype(np.float32)
    return (m.view(np.uint32) & 0xff).astype(np.uint8).view(np.int8).astype(np.int16)


def _codes_ref(vals):
    return np.clip(np.rint(vals.astype(np.float64)), -127, 127).astype(np.int16)


def test_code_rounding_identity():
    anchors = np.arange(-260, 261, dtype=np.float32) / np.float32(2.0)  # k / 2
    bits = anchors.view(np.int32)[:, None] + np.arange(-64, 65, dtype=np.int32)[None, :]
    near = bits.ravel().view(np.float32)
    rng = np.random.default_rng(5)
    rnd = (rng.standard_normal(1_000_000) * 100).astype(np.float32)
    big = np.float32(2.0) ** np.arange(-149, 128, dtype=np.float32)
    vals = np.concatenate([near, -near, rnd, big, -big,
                           np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    vals = vals[np.isfinite(vals) | np.isinf(vals)].astype(np.float32)
    got, want = _codes_magic(vals), _codes_ref(vals)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, vals[bad[:8]]


def test_bf16_packed_daz_identity():
    """The library flushes bf16 inputs (DAZ) with packed 16-bit operations:
    e = h & 0x7f80, m = min(e, 0x7f), h & ~(m ^ 0x7f).  Every one of the
    65536 bf16 patterns must give h with only its sign kept when the
    exponent field is zero, and h itself otherwise."""
    h = np.arange(1 << 16, dtype=np.uint32)
    e = h & 0x7F80
    m = np.minimum(e, 0x7F)
    got = h & ~(m ^ 0x7F) & 0xFFFF
    want = np.where(e == 0, h & 0x8000, h)
    assert np.array_equal(got, want)
