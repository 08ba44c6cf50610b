"""The INT8 append kernel rounds the correctly rounded fp32 quotient x / s to
the nearest integer (ties to even) where the definition divides exactly.
For bf16 x and a binary16 group scale s = RNE16(max|x| / 127) both give the
same code: x / s is a half-integer exactly or at least 2^-12 from one, and
the fp32 quotient is within 2^-18 of it.  This checks that on the host for
every bf16 value below sampled group maxima (no GPU)."""
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
