"""Pins of the oracle's INT8 group-64 quantiser (symmetric absmax groups of 64
head dims, binary16 scale = RNE(amax / 127), codes = clamp(RNE(x / s), +-127))
against a library binary16 codec, brute force with exact rational arithmetic,
the pages' byte budget and closed-form special cases (no GPU)."""
from fractions import Fraction

import numpy as np

import oracle as O
import synth


def _bits(values):
    """Exact float -> bf16 bit patterns (values must be bf16-representable)."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _bf16(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# every finite non-negative binary16 value, ascending, with its bit pattern
_F16_BITS = np.arange(0x7C00, dtype=np.uint16)
_F16_VALS = _F16_BITS.view(np.float16).astype(np.float64)


def _nearest_f16(x: Fraction) -> int:
    """Brute force: the binary16 pattern nearest to x >= 0, ties to the even
    pattern, saturating at the largest finite value."""
    i = int(np.searchsorted(_F16_VALS, float(x)))
    cands = [j for j in (i - 1, i, i + 1) if 0 <= j < len(_F16_VALS)]
    best = min(cands, key=lambda j: (abs(Fraction(_F16_VALS[j]) - x), _F16_BITS[j] & 1))
    return int(_F16_BITS[best])


def _codes_brute(xs, s: Fraction):
    """argmin over c in [-127, 127] of |x - c s|, ties to the even code."""
    out = []
    for x in xs:
        if s == 0:
            out.append(0)
            continue
        best = min(range(-127, 128), key=lambda c: (abs(Fraction(x) - c * s), c & 1))
        out.append(best)
    return out


def test_f16_value_matches_numpy_for_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for b in range(0, 65536, 1):
        if np.isnan(ref[b]):
            continue
        assert O.f16_value(b) == ref[b]


def test_f64_to_f16_rounds_to_nearest_even_and_saturates():
    # every finite value maps to itself; every midpoint between neighbours goes to the even one
    for j in range(0, len(_F16_VALS) - 1, 7):
        a, b = _F16_VALS[j], _F16_VALS[j + 1]
        assert O.f64_to_f16_sat(a) == _F16_BITS[j]
        mid = (a + b) / 2                      # exact in fp64
        even = _F16_BITS[j] if _F16_BITS[j] % 2 == 0 else _F16_BITS[j + 1]
        assert O.f64_to_f16_sat(mid) == even
        assert O.f64_to_f16_sat(np.nextafter(mid, 0)) == _F16_BITS[j]
        assert O.f64_to_f16_sat(np.nextafter(mid, np.inf)) == _F16_BITS[j + 1]
    assert O.f64_to_f16_sat(65504.0) == 0x7BFF
    assert O.f64_to_f16_sat(1e9) == 0x7BFF          # saturates instead of overflowing
    assert O.f64_to_f16_sat(0.0) == 0
    assert O.f64_to_f16_sat(2.0 ** -25) == 0        # exactly half the smallest subnormal: tie to 0
    assert O.f64_to_f16_sat(3 * 2.0 ** -26) == 1


def test_quantize_matches_exact_brute_force_on_random_groups():
    rng = np.random.default_rng(5)
    x = synth.host_fill(71, 0, 0, 24, 2, 256)            # N(0,1) bf16 rows
    # add groups spanning many binades and some tiny ones (fp16-subnormal scales)
    y = _bf16(x) * np.exp2(rng.integers(-30, 12, size=(24, 2, 1)))
    xb = _bits(y.astype(np.float32))
    codes, scales = O.int8_quantize(xb)
    for t in range(24):
        for h in range(2):
            for g in range(4):
                grp = _bf16(xb[t, h, 64 * g: 64 * g + 64])
                amax = max(abs(Fraction(v)) for v in grp)
                sb = _nearest_f16(amax / 127)
                assert scales[t, h, g] == sb
                s = Fraction(float(np.uint16(sb).view(np.float16)))
                assert list(codes[t, h, 64 * g: 64 * g + 64]) == _codes_brute(grp, s)


def test_exact_ties_round_to_even_codes():
    # amax = 127 gives s = 1 exactly; x = k + 1/2 is then an exact tie
    grp = np.zeros(64)
    grp[0] = 127.0
    grp[1:9] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 126.5, 1.5]
    row = np.tile(grp, 4).reshape(1, 1, 256)
    codes, scales = O.int8_quantize(_bits(row.astype(np.float32)))
    assert np.all(scales == 0x3C00)                     # 1.0
    assert list(codes[0, 0, :9]) == [127, 2, 4, -2, -4, 0, 0, 126, 2]


def test_group_maximum_codes_to_127_and_zero_groups_to_zero():
    x = synth.host_fill(72, 0, 0, 64, 4, 256)
    codes, scales = O.int8_quantize(x)
    xf = _bf16(x).reshape(64, 4, 4, 64)
    c = codes.reshape(64, 4, 4, 64).astype(np.int64)
    i = np.abs(xf).argmax(axis=-1)
    top = np.take_along_axis(c, i[..., None], axis=-1)[..., 0]
    assert np.all(np.abs(top) == 127)
    assert np.all(np.sign(top) == np.sign(np.take_along_axis(xf, i[..., None], axis=-1)[..., 0]))
    z = np.zeros((2, 1, 256), dtype=np.uint16)
    z[1, 0, 64:128] = 0x8000                            # -0.0 in one group
    cz, sz = O.int8_quantize(z)
    assert np.all(cz == 0) and np.all(sz == 0)


def test_reconstruction_error_is_at_most_half_a_step():
    x = synth.host_fill(73, 0, 0, 128, 4, 256, outlier_stream=3, outlier_p=0.01,
                        outlier_mul=20.0)
    codes, scales = O.int8_quantize(x)
    xh = O.int8_dequantize(codes, scales)
    s = np.repeat(np.vectorize(O.f16_value)(scales), 64, axis=-1)
    assert np.all(np.abs(_bf16(x) - xh) <= s / 2 * (1 + 2.0 ** -40))


def test_byte_budget_matches_the_pages():
    # 16.5 KiB per token per device at INT8 group-64, scale planes included,
    # with 16 full-attention layers and 2 of the 4 KV heads per device
    per_head = 256 * 1 + (256 // 64) * 2          # codes + binary16 group scales
    assert 16 * 2 * 2 * per_head == 16.5 * 1024


def test_int8_attention_is_the_dense_softmax_over_dequantised_values():
    rng = np.random.default_rng(9)
    N, Hq, Hkv = 37, 6, 2
    k = synth.host_fill(74, 1, 0, N, Hkv, 256)
    v = synth.host_fill(74, 2, 0, N, Hkv, 256)
    kc, ks = O.int8_quantize(k)
    vc, vs = O.int8_quantize(v)
    kh, vh = O.int8_dequantize(kc, ks), O.int8_dequantize(vc, vs)
    q = rng.standard_normal((Hq, 256))
    got = O.decode_attention(q, kc, vc, int8=(ks, vs))
    for h in range(Hq):
        g = h // (Hq // Hkv)
        z = kh[:, g] @ q[h] / 16.0
        w = np.exp(z - z.max())
        ref = (w[:, None] * vh[:, g]).sum(0) / w.sum()
        assert np.allclose(got[h], ref, rtol=1e-12, atol=1e-13)
