"""Pins of the oracle's NVFP4 quantiser (e2m1 codes, e4m3 scale per 16
elements, fp32 tensor scale) against the format definitions, a library
decoder and brute force with exact rational arithmetic (no GPU)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

E2M1 = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp4_e2m1.json")))


def _bits(values):
    """Exact float -> bf16 bit patterns (values must be bf16-representable)."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def test_e2m1_table():
    mags = E2M1["magnitudes"]
    for c in range(16):
        v = O.e2m1_value(c)
        expect = mags[c & 7] * (-1.0 if c & 8 else 1.0)
        assert v == expect and np.signbit(v) == bool(c & 8)


def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = O.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v) and (c & 0x7F) == 0x7F
        else:
            assert v == ref[c] and np.signbit(v) == np.signbit(ref[c])
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x01) == 2.0 ** -9


# -- brute force with exact rationals -----------------------------------------

_E4M3_POS = [(c, Fraction(O.e4m3_value(c))) for c in range(0x7F)]   # 0x00..0x7E
_E2M1_POS = [(c, Fraction(m)) for c, m in enumerate(E2M1["magnitudes"])]


def _nearest_even(target, table):
    """Argmin of |target - v| over (code, v); ties to the even code.  Values
    above the table's top saturate to it."""
    best = None
    for c, v in table:
        d = abs(target - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    return best[1]


def _brute_block(xbits, S):
    xs = [Fraction(float(v)) for v in O.bf16_to_f64(xbits)]
    b = max(abs(v) for v in xs)
    q = b / (6 * Fraction(float(S)))
    qs = _nearest_even(q, _E4M3_POS)
    eff = Fraction(O.e4m3_value(qs)) * Fraction(float(S))
    codes = []
    for v, bits in zip(xs, xbits):
        mag = 0 if eff == 0 else _nearest_even(abs(v) / eff, _E2M1_POS)
        codes.append(((int(bits) >> 15) << 3) | mag)
    return qs, codes


def _rand_bf16(rng, n, scale=1.0):
    f = (rng.standard_normal(n) * scale).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantize_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, H, D = 6, 2, 64   # 48 blocks per seed
    x = _rand_bf16(rng, T * H * D).reshape(T, H, D)
    # spread magnitudes so blocks land on scale subnormals, normals and saturation
    boost = rng.choice([2.0 ** -12, 2.0 ** -6, 1.0, 8.0, 64.0], size=(T, H, D // 16))
    xf = O.bf16_to_f64(x) * np.repeat(boost, 16, axis=-1)
    x = O.round_bf16(xf)
    S = O.nvfp4_tensor_scale(x) * np.float32(rng.choice([1.0, 0.37, 3.0]))
    codes, scales = O.nvfp4_quantize(x, S)
    for t in range(T):
        for h in range(H):
            for b in range(D // 16):
                qs, cs = _brute_block(x[t, h, 16 * b: 16 * b + 16], S)
                assert scales[t, h, b] == qs
                assert list(codes[t, h, 16 * b: 16 * b + 16]) == cs


def test_e2m1_ties_go_to_even_code():
    """With S = 1 and a block max of 6 the block scale is 1.0 (code 0x38), so
    |x| / eff is |x| itself and every midpoint below is an exact tie."""
    vals = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 0.0, -0.0, 0.251953125, 4.875,
            5.125, -6.0]
    x = _bits(vals).reshape(1, 1, 16)
    codes, scales = O.nvfp4_quantize(x, np.float32(1.0))
    assert scales[0, 0, 0] == 0x38
    mags = [0b111, 0, 2, 2, 4, 4, 6, 6, 0, 6, 0, 0, 1, 6, 7, 7]
    signs = [0, 0, 0, 0, 0, 0, 0, 0, 1, 1, 0, 1, 0, 0, 0, 1]
    assert list(codes[0, 0]) == [(s << 3) | m for s, m in zip(signs, mags)]


def test_block_holding_amax_saturates_scale():
    rng = np.random.default_rng(7)
    x = _rand_bf16(rng, 4 * 256).reshape(4, 1, 256)
    S = O.nvfp4_tensor_scale(x)
    codes, scales = O.nvfp4_quantize(x, S)
    xf = np.abs(O.bf16_to_f64(x))
    t, h, d = np.unravel_index(np.argmax(xf), xf.shape)
    assert scales[t, h, d // 16] == 0x7E
    assert codes[t, h, d] & 7 == 7


def test_tensor_scale_definition():
    x = _bits([0.0, -3.0, 2688.0 * 0.5, 1.0]).reshape(1, 1, 4)
    assert O.nvfp4_tensor_scale(x) == np.float32(0.5)
    assert O.nvfp4_tensor_scale(np.zeros((1, 1, 4), np.uint16)) == np.float32(1.0)


def test_quantize_dequantize_identity_on_representable_values():
    """Blocks built from codes and a scale, each with one |code| = 6 element so
    the block max pins the scale: quantising the dequantised value recovers
    the same codes and scale (S a power of two keeps every value in bf16)."""
    rng = np.random.default_rng(11)
    T, H, D = 8, 4, 256
    S = np.float32(2.0 ** -3)
    scales = rng.integers(0x08, 0x7F, size=(T, H, D // 16)).astype(np.uint8)
    codes = rng.integers(0, 16, size=(T, H, D)).astype(np.uint8)
    codes[..., ::16] = np.where(rng.random((T, H, D // 16)) < 0.5, 7, 15)
    xd = O.nvfp4_dequantize(codes, scales, S)
    x = O.round_bf16(xd)
    assert np.array_equal(O.bf16_to_f64(x), xd)
    c2, s2 = O.nvfp4_quantize(x, S)
    assert np.array_equal(s2, scales)
    # -0 stays -0 only in sign; magnitudes and signs of non-zeros agree
    assert np.array_equal(c2 & 7, codes & 7)
    nz = (codes & 7) != 0
    assert np.array_equal(c2[nz], codes[nz])


def test_pack_low_nibble_first():
    c = np.array([[1, 2, 15, 8]], dtype=np.uint8)
    assert list(O.nvfp4_pack(c)[0]) == [0x21, 0x8F]


def test_nvfp4_bytes_per_token_layer():
    """4 KV heads x (128 code bytes + 16 scale bytes) x (K and V)."""
    heads, D = 4, 256
    assert heads * (D // 2 + D // 16) * 2 == 1152
