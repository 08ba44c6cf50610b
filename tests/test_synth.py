"""The seeded input generator: published-definition test vector, table
properties and recipe invariants (no GPU)."""
import numpy as np

import oracle as O
import synth


def test_splitmix64_reference_outputs():
    """Seed 0 / stream 0 has stream key 0, so the draws are the plain
    SplitMix64 sequence from state 0 (the published reference outputs)."""
    d = synth.draws(0, 0, 0, 3)
    assert [int(x) for x in d] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_access_is_positional():
    a = synth.draws(1003, 65, 0, 1000)
    b = synth.draws(1003, 65, 400, 100)
    assert np.array_equal(a[400:500], b)
    assert not np.array_equal(synth.draws(1003, 66, 0, 1000), a)


def test_normal_table():
    t = O.bf16_to_f64(synth.normal_table())
    assert np.all(np.diff(t) >= 0)
    assert np.array_equal(t, -t[::-1])
    assert abs(t.mean()) < 1e-12 and abs(t.std() - 1.0) < 2e-3


def test_fill_is_sliceable_and_applies_recipe():
    full = synth.host_fill(1002, synth.stream_id(0, synth.K), 0, 40, 4, 256)
    part = synth.host_fill(1002, synth.stream_id(0, synth.K), 17, 5, 4, 256)
    assert np.array_equal(full[17:22], part)
    mul = synth.outlier_channels(1002, 0, synth.K, 4, 256, 4, 8.0)
    scaled = synth.host_fill(1002, synth.stream_id(0, synth.K), 0, 40, 4, 256, chan_mul=mul)
    assert np.array_equal(O.bf16_to_f64(scaled), O.bf16_to_f64(full) * mul[None])
    assert (mul == 8.0).sum() == 16


def test_element_outliers_rate_and_value():
    n = 4096
    base = synth.host_fill(1004, 1, 0, n, 4, 256)
    out = synth.host_fill(1004, 1, 0, n, 4, 256, outlier_stream=3, outlier_p=0.01,
                          outlier_mul=20.0)
    diff = base != out
    rate = diff.mean()
    assert 0.009 < rate < 0.011
    b = O.bf16_to_f64(base[diff])
    assert np.array_equal(O.bf16_to_f64(out[diff]), O.bf16_to_f64(O.round_bf16(b * 20.0)))


def test_block_permutation_is_a_permutation():
    p = synth.block_permutation(1002, 16384)
    assert np.array_equal(np.sort(p), np.arange(16384))
