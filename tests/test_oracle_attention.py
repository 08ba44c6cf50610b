"""Pins of the oracle's decode and prefill attention against closed forms,
invariants and brute force (no GPU)."""
import math

import numpy as np
import pytest

import oracle as O


def _rand_bits(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(0)
    N, Hq, Hkv, D = 37, 24, 4, 256
    q = O.bf16_to_f64(_rand_bits(rng, (Hq, D)))
    k = np.repeat(_rand_bits(rng, (1, Hkv, D)), N, axis=0)
    v = _rand_bits(rng, (N, Hkv, D))
    out = O.decode_attention(q, k, v)
    mean = O.bf16_to_f64(v).mean(axis=0)
    for h in range(Hq):
        assert np.allclose(out[h], mean[h // 6], rtol=0, atol=1e-14)


def test_single_key_gives_its_value():
    rng = np.random.default_rng(1)
    q = O.bf16_to_f64(_rand_bits(rng, (24, 256)))
    k = _rand_bits(rng, (1, 4, 256))
    v = _rand_bits(rng, (1, 4, 256))
    out, lse = O.decode_attention(q, k, v, with_lse=True)
    vf = O.bf16_to_f64(v)[0]
    for h in range(24):
        assert np.array_equal(out[h], vf[h // 6])
    z = (q * np.repeat(O.bf16_to_f64(k)[0], 6, axis=0)).sum(-1) / 16.0
    assert np.allclose(lse, z, rtol=0, atol=1e-12)


def test_two_keys_closed_form_and_scale():
    """K1 = 0 gives logit 0; K2 = 2q gives logit 2|q|^2 / sqrt(D).  The output
    is (V1 + e^a V2) / (1 + e^a): pins the 1/sqrt(D) scale and the softmax."""
    rng = np.random.default_rng(2)
    D = 256
    qb = _rand_bits(rng, (1, D), scale=0.25)
    q = O.bf16_to_f64(qb)
    k = np.zeros((2, 1, D), np.uint16)
    k[1, 0] = O.round_bf16(2.0 * q[0])          # exact: doubling a bf16
    v = _rand_bits(rng, (2, 1, D))
    out = O.decode_attention(q, k, v)
    a = 2.0 * float(np.dot(q[0], q[0])) / math.sqrt(D)
    vf = O.bf16_to_f64(v)
    expect = (vf[0, 0] + math.exp(a) * vf[1, 0]) / (1.0 + math.exp(a))
    assert 1.0 < a < 30.0
    assert np.allclose(out[0], expect, rtol=0, atol=1e-13)


def test_gqa_grouping_is_consecutive():
    """Changing the values of KV head g changes exactly query heads 6g..6g+5."""
    rng = np.random.default_rng(3)
    N, Hq, Hkv, D = 50, 24, 4, 256
    q = O.bf16_to_f64(_rand_bits(rng, (Hq, D)))
    k = _rand_bits(rng, (N, Hkv, D))
    v = _rand_bits(rng, (N, Hkv, D))
    base = O.decode_attention(q, k, v)
    for g in range(Hkv):
        v2 = v.copy()
        v2[:, g] = _rand_bits(rng, (N, D))
        out = O.decode_attention(q, k, v2)
        changed = [h for h in range(Hq) if not np.array_equal(out[h], base[h])]
        assert changed == list(range(6 * g, 6 * g + 6))


@pytest.mark.parametrize("split", [1, 17, 64, 99])
def test_split_and_lse_merge_is_exact(split):
    rng = np.random.default_rng(4)
    N, Hq, Hkv, D = 100, 8, 2, 256
    q = O.bf16_to_f64(_rand_bits(rng, (Hq, D), scale=2.0))
    k = _rand_bits(rng, (N, Hkv, D))
    v = _rand_bits(rng, (N, Hkv, D))
    full, lse = O.decode_attention(q, k, v, with_lse=True)
    o1, l1 = O.decode_attention(q, k[:split], v[:split], with_lse=True)
    o2, l2 = O.decode_attention(q, k[split:], v[split:], with_lse=True)
    M = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - M), np.exp(l2 - M)
    merged = (w1[:, None] * o1 + w2[:, None] * o2) / (w1 + w2)[:, None]
    assert np.allclose(merged, full, rtol=0, atol=1e-12)
    assert np.allclose(M + np.log(w1 + w2), lse, rtol=0, atol=1e-12)


def test_empty_cache_gives_zeros():
    q = np.ones((24, 256))
    k = np.zeros((0, 4, 256), np.uint16)
    out, lse = O.decode_attention(q, k, k, with_lse=True)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_needle_dominates_within_mass_bound():
    """A key equal to twice the (roped) query concentrates the head's softmax
    mass on it; |o - V*| is bounded by (1 - w*) max |V_n - V*|."""
    rng = np.random.default_rng(5)
    N, D = 20000, 256
    t = O.yarn_table()
    qb = _rand_bits(rng, (1, 24, D))
    q = O.rope(qb, [N], t)[0]
    q_bits = O.round_bf16(q)
    qf = O.bf16_to_f64(q_bits)
    k = _rand_bits(rng, (N, 4, D))
    v = _rand_bits(rng, (N, 4, D))
    p = 12345
    for g in range(4):
        k[p, g] = O.round_bf16(2.0 * qf[6 * g])
    out, lse = O.decode_attention(qf, k, v, with_lse=True)
    vf = O.bf16_to_f64(v)
    for g in range(4):
        h = 6 * g
        z_star = float(np.dot(qf[h], O.bf16_to_f64(k[p, g]))) / 16.0
        w_star = math.exp(z_star - lse[h])
        assert w_star > 0.99
        bound = (1.0 - w_star) * np.abs(vf[:, g] - vf[p, g]).max()
        assert np.abs(out[h] - vf[p, g]).max() <= bound + 1e-12


def test_dense_brute_force_tiny():
    """Dense softmax with explicit GQA expansion, for small shapes."""
    rng = np.random.default_rng(6)
    N, Hq, Hkv, D = 19, 12, 3, 32
    q = O.bf16_to_f64(_rand_bits(rng, (Hq, D)))
    k = _rand_bits(rng, (N, Hkv, D))
    v = _rand_bits(rng, (N, Hkv, D))
    out = O.decode_attention(q, k, v, scale=0.3)
    kf, vf = O.bf16_to_f64(k), O.bf16_to_f64(v)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        z = 0.3 * kf[:, g] @ q[h]
        w = np.exp(z - z.max())
        w /= w.sum()
        assert np.allclose(out[h], w @ vf[:, g], rtol=0, atol=1e-13)


def test_prefill_is_causal_including_self():
    rng = np.random.default_rng(7)
    N, Hq, Hkv, D = 40, 6, 1, 64
    q = O.bf16_to_f64(_rand_bits(rng, (5, Hq, D)))
    pos = np.array([0, 7, 8, 30, 39])
    k = _rand_bits(rng, (N, Hkv, D))
    v = _rand_bits(rng, (N, Hkv, D))
    out = O.prefill_attention(q, pos, k, v)
    # row at position 0 sees only key 0
    assert np.array_equal(out[0, 0], O.bf16_to_f64(v[0, 0]))
    # keys after a row's position do not matter; its own key does
    k2, v2 = k.copy(), v.copy()
    k2[9:], v2[9:] = _rand_bits(rng, (N - 9, Hkv, D)), _rand_bits(rng, (N - 9, Hkv, D))
    out2 = O.prefill_attention(q, pos, k2, v2)
    assert np.array_equal(out2[:3], out[:3]) and not np.array_equal(out2[3:], out[3:])
    v3 = v.copy()
    v3[8] = _rand_bits(rng, (Hkv, D))
    out3 = O.prefill_attention(q, pos, k, v3)
    assert np.array_equal(out3[:2], out[:2]) and not np.array_equal(out3[2], out[2])
    # dense causal mask for the tiny case
    kf, vf = O.bf16_to_f64(k), O.bf16_to_f64(v)
    for r, p in enumerate(pos):
        for h in range(Hq):
            z = kf[: p + 1, 0] @ q[r, h] / 8.0
            w = np.exp(z - z.max())
            assert np.allclose(out[r, h], (w / w.sum()) @ vf[: p + 1, 0], rtol=0, atol=1e-13)


def test_nvfp4_attention_equals_bf16_attention_on_dequantised_values():
    """When the dequantised cache is exactly bf16-representable, the NVFP4
    attention must equal the bf16 attention on those values, to the bit."""
    rng = np.random.default_rng(8)
    N, Hq, Hkv, D = 64, 24, 4, 256
    S = np.float32(2.0 ** -4)
    kc = rng.integers(0, 16, size=(N, Hkv, D)).astype(np.uint8)
    vc = rng.integers(0, 16, size=(N, Hkv, D)).astype(np.uint8)
    ks = rng.integers(0x20, 0x50, size=(N, Hkv, D // 16)).astype(np.uint8)
    vs = rng.integers(0x20, 0x50, size=(N, Hkv, D // 16)).astype(np.uint8)
    kd = O.round_bf16(O.nvfp4_dequantize(kc, ks, S))
    vd = O.round_bf16(O.nvfp4_dequantize(vc, vs, S))
    q = O.bf16_to_f64(_rand_bits(rng, (Hq, D)))
    a = O.decode_attention(q, kc, vc, nvfp4=(ks, vs, S, S))
    b = O.decode_attention(q, kd, vd)
    assert np.array_equal(a, b)


def test_bf16_kv_bytes_per_token_is_64_kib():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_sizes.json")))
    assert O.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], 2) == \
        g["bf16_bytes_per_token"]
