"""Pins of the oracle's YaRN table and rotation against what the pages print
and what the mathematics fixes (no GPU)."""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "yarn_constants.json")))


def _table(**kw):
    base = dict(rope_theta=GOLD["rope_theta"], rotary_dim=GOLD["rotary_dim"], factor=GOLD["factor"],
                original_max_position=GOLD["original_max_position"], beta_fast=GOLD["beta_fast"],
                beta_slow=GOLD["beta_slow"])
    base.update(kw)
    return O.yarn_table(**base)


def test_printed_correction_ranges():
    t = _table()
    assert (t.low, t.high) == tuple(GOLD["formula_range"])
    t = _table(correction_max_position=GOLD["deployed_correction_max_position"])
    assert (t.low, t.high) == tuple(GOLD["deployed_range"])


def test_printed_mscale():
    t = _table()
    assert round(t.mscale, GOLD["mscale_printed_decimals"]) == GOLD["mscale_printed"]


@pytest.mark.parametrize("L,factor", [(262144, 4.0), (1048576, 4.0), (1024, 4.0), (4096, 8.0),
                                      (262144, 16.0), (32768, 2.0)])
def test_range_counts_rotations(L, factor):
    """The range bounds are where the number of full turns a pair makes over
    the original context crosses beta_fast / beta_slow: pairs up to `low` turn
    at least beta_fast times, pair low+1 fewer; pair `high` turns at most
    beta_slow times, pair high-1 more.  Counted directly, not via the log."""
    theta_base, d = GOLD["rope_theta"], GOLD["rotary_dim"]
    t = O.yarn_table(rope_theta=theta_base, rotary_dim=d, factor=factor,
                     original_max_position=L, beta_fast=32.0, beta_slow=1.0)
    i = np.arange(d // 2)
    turns = L * theta_base ** (-2.0 * i / d) / (2 * math.pi)
    assert turns[t.low] >= 32.0 > turns[t.low + 1]
    assert turns[t.high] <= 1.0 < turns[t.high - 1]


def test_ramp_endpoints_and_monotone():
    """Pairs below the range keep the trained frequency; pairs from `high` up
    are divided by the factor; in between the ratio falls monotonically."""
    d = GOLD["rotary_dim"]
    t = _table()
    theta = GOLD["rope_theta"] ** (-2.0 * np.arange(d // 2) / d)
    ratio = t.inv_freq / theta
    assert np.allclose(ratio[: t.low + 1], 1.0, rtol=1e-14, atol=0)
    assert np.allclose(ratio[t.high:], 1.0 / GOLD["factor"], rtol=1e-14, atol=0)
    mid = ratio[t.low: t.high + 1]
    assert np.all(np.diff(mid) < 0)
    assert np.all((mid[1:-1] < 1.0) & (mid[1:-1] > 1.0 / GOLD["factor"]))


def test_factor_one_is_plain_rope_table():
    d = GOLD["rotary_dim"]
    t = _table(factor=1.0)
    theta = GOLD["rope_theta"] ** (-2.0 * np.arange(d // 2) / d)
    assert np.allclose(t.inv_freq, theta, rtol=1e-15, atol=0)
    assert t.mscale == 1.0


@pytest.mark.parametrize("base", [1.0000001, 1.001])
def test_base_near_one_interpolates_every_pair(base):
    """A base just above 1 puts the fast end of the correction range far
    past the last pair (beyond the int range for 1 + 1e-7): the ramp is 1
    for every pair, so every frequency is theta_i / s."""
    d = GOLD["rotary_dim"]
    t = _table(rope_theta=base)
    theta = base ** (-2.0 * np.arange(d // 2) / d)
    assert np.allclose(t.inv_freq, theta / GOLD["factor"], rtol=1e-15, atol=0)
    assert t.low >= d and t.high == d - 1


def test_domain_errors():
    with pytest.raises(ValueError):
        _table(factor=0.5)
    with pytest.raises(ValueError):
        _table(rotary_dim=63)


def _rand_bits(rng, shape):
    """Random finite bf16 bit patterns from N(0,1) values."""
    f = rng.standard_normal(shape).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_factor_one_matches_complex_exponential():
    """With s = 1 the rotation is textbook RoPE: pair (x_i, x_{i+d/2}) read as
    the complex number x_i + j x_{i+d/2}, multiplied by exp(j p theta_i)."""
    rng = np.random.default_rng(1)
    T, H, D, d = 7, 3, 256, 64
    x = _rand_bits(rng, (T, H, D))
    pos = np.array([0, 1, 5, 4095, 262143, 777777, 1048575])
    t = _table(factor=1.0)
    y = O.rope(x, pos, t, rotary_dim=d)
    xf = O.bf16_to_f64(x)
    z = xf[..., : d // 2] + 1j * xf[..., d // 2: d]
    theta = GOLD["rope_theta"] ** (-2.0 * np.arange(d // 2) / d)
    zr = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    # The angle p*theta carries an fp64 rounding of ~p*2^-52 rad on either
    # side; the bound scales with the position and |z|.
    tol = 1e-15 * (1.0 + pos[:, None, None]) * (1.0 + np.abs(z))
    assert np.all(np.abs(y[..., : d // 2] - zr.real) <= tol)
    assert np.all(np.abs(y[..., d // 2: d] - zr.imag) <= tol)
    assert np.array_equal(y[..., d:], xf[..., d:])


def test_norm_scaled_by_mscale_on_rotary_dims_only():
    rng = np.random.default_rng(2)
    x = _rand_bits(rng, (5, 4, 256))
    pos = np.array([3, 262144, 524288, 1000003, 1048576])
    t = _table()
    y = O.rope(x, pos, t)
    xf = O.bf16_to_f64(x)
    nx = np.linalg.norm(xf[..., :64], axis=-1)
    ny = np.linalg.norm(y[..., :64], axis=-1)
    assert np.allclose(ny, t.mscale * nx, rtol=1e-12, atol=0)
    assert np.array_equal(y[..., 64:], xf[..., 64:])


def test_position_zero_only_scales():
    rng = np.random.default_rng(3)
    x = _rand_bits(rng, (1, 2, 256))
    t = _table()
    y = O.rope(x, np.array([0]), t)
    xf = O.bf16_to_f64(x)
    assert np.allclose(y[..., :64], t.mscale * xf[..., :64], rtol=1e-15, atol=0)


@pytest.mark.parametrize("m,n,delta", [(1048576, 17, -1000000), (5, 900000, 123456),
                                       (262144, 262143, 786432)])
def test_dot_depends_only_on_position_difference(m, n, delta):
    rng = np.random.default_rng(4)
    q = _rand_bits(rng, (1, 1, 256))
    k = _rand_bits(rng, (1, 1, 256))
    t = _table()
    a = np.dot(O.rope(q, [m], t).ravel(), O.rope(k, [n], t).ravel())
    b = np.dot(O.rope(q, [m + delta], t).ravel(), O.rope(k, [n + delta], t).ravel())
    assert abs(a - b) <= 1e-9 * (abs(a) + 1.0)


def test_bf16_rounding_is_nearest_even():
    """fp64 -> bf16: the result is the nearest bf16 (checked against both
    neighbours), ties to the even pattern; exact bf16 values round-trip."""
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                         [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -133,
                          3 * 2 ** -134, 2 ** -126 - 2 ** -134]])
    bits = O.round_bf16(xs)
    val = O.bf16_to_f64(bits)
    up = O.bf16_to_f64((bits.astype(np.int64) + 1).astype(np.uint16))
    dn_bits = bits.astype(np.int64) - 1
    ok_dn = (bits & 0x7FFF) != 0
    dn = O.bf16_to_f64(np.where(ok_dn, dn_bits, bits).astype(np.uint16))
    err = np.abs(xs - val)
    assert np.all(err <= np.abs(xs - up))
    assert np.all(err[ok_dn] <= np.abs(xs - dn)[ok_dn])
    tie = (err == np.abs(xs - up)) | (ok_dn & (err == np.abs(xs - dn)))
    assert np.all((bits[tie] & 1) == 0)
    assert tie.sum() >= 3
    exact = _rand_bits(rng, (1000,))
    assert np.array_equal(O.round_bf16(O.bf16_to_f64(exact)), exact)


_PARAM_SETS = [dict(original_max_position=262144), dict(original_max_position=1024),
               dict(original_max_position=262144, correction_max_position=1048576),
               dict(original_max_position=4096, factor=1.0)]


@pytest.mark.parametrize("kw", _PARAM_SETS)
@pytest.mark.parametrize("rotary_dim", [64, 2, 256])
def test_rope_bf16_is_one_rounding_of_the_fp64_rotation(kw, rotary_dim):
    """The bf16 rope the GPU results are compared with is, bit for bit, the
    pinned fp64 rotation rounded once to bf16 on the rotary dims, and a copy
    of the input bits on the others (-0 and bf16 subnormals included)."""
    rng = np.random.default_rng(11 + rotary_dim)
    pos = np.concatenate([[0, 1, 262143, 262144, 1048575, 1048576],
                          rng.integers(0, 1 << 21, 58)]).astype(np.int64)
    T, H, D = len(pos), 5, 256
    x = _rand_bits(rng, (T, H, D))
    x[0, 0, :8] = [0x8000, 0x0000, 0x0001, 0x8001, 0x007F, 0x7F7F, 0xFF7F, 0x3F80]
    x[1, 1, rotary_dim - 1] = 0x8000
    x[2, 2, D - 1] = 0x8001
    t = _table(rotary_dim=rotary_dim, **kw)
    y16 = O.rope(x, pos, t, rotary_dim=rotary_dim, bf16_out=True)
    y64 = O.rope(x, pos, t, rotary_dim=rotary_dim)
    assert np.array_equal(y16[..., :rotary_dim], O.round_bf16(y64[..., :rotary_dim]))
    assert np.array_equal(y16[..., rotary_dim:], x[..., rotary_dim:])


def test_rope_bf16_at_position_zero_without_stretch_is_the_identity():
    """Position 0 turns by nothing and factor 1 scales by nothing: every
    element comes back bit for bit."""
    rng = np.random.default_rng(12)
    x = _rand_bits(rng, (16, 24, 256))
    t = _table(factor=1.0)
    assert t.mscale == 1.0
    assert np.array_equal(O.rope(x, np.zeros(16, dtype=np.int64), t, bf16_out=True), x)


def test_rope_bf16_single_pair_matches_numpy_rotation():
    """With factor 1 and rotary_dim 2 the single pair turns by p radians; at
    p = 0 nothing moves and the bf16 result of a turn by p is the correctly
    rounded (x cos p - y sin p, y cos p + x sin p), checked here from numpy's
    cos and sin, independently of the library's rotation loop."""
    rng = np.random.default_rng(13)
    x = _rand_bits(rng, (40, 3, 8))
    pos = rng.integers(0, 1 << 20, 40).astype(np.int64)
    t = _table(factor=1.0, rotary_dim=2)
    assert t.inv_freq[0] == 1.0
    y = O.rope(x, pos, t, rotary_dim=2, bf16_out=True)
    a, b = O.bf16_to_f64(x[..., 0]), O.bf16_to_f64(x[..., 1])
    c, s = np.cos(pos.astype(np.float64))[:, None], np.sin(pos.astype(np.float64))[:, None]
    e0, e1 = a * c - b * s, b * c + a * s
    # numpy's cos/sin may differ from libm's in the last bit: compare against
    # the correctly rounded value with one bf16 step of slack only where the
    # fp64 value lies within 1e-12 (relative) of a rounding boundary
    for got, exact in ((y[..., 0], e0), (y[..., 1], e1)):
        ref = O.round_bf16(exact)
        near = np.abs(O.bf16_to_f64(O.round_bf16(exact * (1 + 1e-12))) -
                      O.bf16_to_f64(O.round_bf16(exact * (1 - 1e-12)))) > 0
        assert np.array_equal(got[~near], ref[~near])
        assert np.all(np.abs(got[near].astype(np.int64) - ref[near].astype(np.int64)) <= 1)
    assert np.array_equal(y[..., 2:], x[..., 2:])
