"""The INT8 append kernel's decisions against the exact arithmetic of the
definition (group scale s = RNE16(max|x| / 127), codes RNE(x / s)), on the
host for every bf16 value below sampled group maxima (no GPU):
  - rounding the correctly rounded fp32 quotient x / s to the nearest
    integer (ties to even) gives the exact code: x / s is a half-integer
    exactly or at least 2^-12 from one, and the fp32 quotient is within
    2^-18 of it;
  - the group scale from the product with the fp32 1/127 equals the
    oracle's for every maximum;
  - the kernels' division-free code decision equals the exact code."""
import numpy as np


def test_fp32_quotient_gives_the_exact_code():
    b = (np.arange(0x0001, 0x7F80, dtype=np.uint32) << 16).view(np.float32)   # bf16 > 0
    rng = np.random.default_rng(7)
    maxima = np.concatenate([b[::97], b[rng.integers(0, len(b), 200)],
                             np.float32([1.0, 127.0, 254.0, 65504.0 * 127.0])])
    pairs = 0
    for m in maxima:
        q = np.float64(m) / 127.0
        if not 0.0 < q < 65504.0:      # saturated or zero scales code nothing here
            continue
        s = np.float64(np.float16(q))
        if s == 0.0:
            continue
        xs = b[b <= m]
        xs = np.concatenate([xs, -xs])
        exact = np.clip(np.rint(xs.astype(np.float64) / s), -127, 127)
        fp32 = np.clip(np.rint(xs / np.float32(s)).astype(np.float64), -127, 127)
        assert np.array_equal(exact, fp32), float(m)
        pairs += len(xs)
    assert pairs > 1_000_000


def test_fp32_group_scale_equals_the_oracle_scale_for_every_maximum():
    """The append kernels take the group scale RNE16(m / 127) as m times the
    fp32 nearest 1/127, converted to binary16 (nearest even, saturating at
    65504), either through the rounded fp32 product or, where the compiler
    fuses the two into a mixed-precision multiply-add, from the exact
    product rounded once.  For every bf16 magnitude m both give the oracle's
    scale, which rounds the fp64 quotient once; so does the correctly
    rounded fp32 quotient."""
    import oracle as O
    m = (np.arange(0x0000, 0x7F80, dtype=np.uint32) << 16).view(np.float32)   # 0 and all finite
    ref = np.array([O.f64_to_f16_sat(float(x) / 127.0) for x in m], dtype=np.uint16)

    def to16(q):
        return np.where(q >= 65504.0, np.uint16(0x7BFF),
                        np.minimum(q, 65504.0).astype(np.float16).view(np.uint16))

    r = np.float32(1.0) / np.float32(127.0)
    assert np.array_equal(to16(m * r), ref)                                  # fp32 product, then binary16
    assert np.array_equal(to16(m.astype(np.float64) * np.float64(r)), ref)   # exact product, rounded once
    assert np.array_equal(to16(m / np.float32(127.0)), ref)                  # fp32 quotient
    assert (ref == 0x7BFF).sum() > 1000 and ((ref > 0) & (ref < 0x0400)).sum() > 100


def test_reciprocal_quotient_with_exact_tie_test_gives_the_exact_code():
    """The append kernels decide RNE(x / s) from q = x * r, r the hardware
    reciprocal of s (within one ulp of 1/s: all three fp32 neighbours are
    tried here), with rint(q) unless x - h s == 0 for h = floor(q) + 1/2
    (then rint(h)).  For every bf16 x below sampled group maxima that gives
    the code of the exact quotient."""
    b = (np.arange(0x0001, 0x7F80, dtype=np.uint32) << 16).view(np.float32)   # bf16 > 0
    rng = np.random.default_rng(8)
    maxima = np.concatenate([b[::131], b[rng.integers(0, len(b), 150)],
                             np.float32([1.0, 127.0, 254.0, 1.5, 3.0 * 127.0])])
    pairs = 0
    for m in maxima:
        q64 = np.float64(m) / 127.0
        if not 0.0 < q64 < 65504.0:
            continue
        s = np.float32(np.float16(q64))
        if s == 0.0:
            continue
        xs = b[b <= m]
        xs = np.concatenate([xs, -xs])
        exact = np.clip(np.rint(xs.astype(np.float64) / np.float64(s)), -127, 127)
        r0 = np.float32(1.0) / s
        for r in (np.nextafter(r0, np.float32(0)), r0, np.nextafter(r0, np.float32(np.inf))):
            q = xs * np.float32(r)
            h = np.floor(q) + np.float32(0.5)
            tie = (xs.astype(np.float64) - h.astype(np.float64) * np.float64(s)) == 0.0
            k = np.where(tie, np.rint(h), np.rint(q))
            got = np.clip(k.astype(np.float64), -127, 127)
            assert np.array_equal(exact, got), (float(m), float(r))
        pairs += len(xs)
    assert pairs > 1_000_000
