"""Pins of the oracle's paged gather (the HND page layout: a page holds, per
KV head, block_size consecutive token rows; logical token n of a sequence is
in block table[n // block_size], slot n % block_size), which reads back every
paged bit-exact GPU check.  No GPU."""
import numpy as np
import pytest

import oracle as O


def _brute_gather(pool, num_blocks, H, bs, rb, table, ntok):
    """Token by token, head by head, byte by byte from the definition."""
    flat = pool.reshape(-1)
    out = np.zeros((ntok, H, rb), dtype=np.uint8)
    for n in range(ntok):
        blk = int(table[n // bs])
        if not 0 <= blk < num_blocks:
            raise IndexError(n)
        slot = n % bs
        for h in range(H):
            start = ((blk * H + h) * bs + slot) * rb
            for i in range(rb):
                out[n, h, i] = flat[start + i]
    return out


@pytest.mark.parametrize("rb", [2, 128, 144, 512])
@pytest.mark.parametrize("H,bs", [(4, 16), (1, 16), (3, 4)])
def test_gather_matches_brute_force_on_a_shuffled_pool(rb, H, bs):
    rng = np.random.default_rng(rb * 31 + H * 7 + bs)
    num_blocks = 6
    pool = rng.integers(0, 256, size=num_blocks * H * bs * rb, dtype=np.uint8)
    pages = 5                                      # one pool block stays unused
    table = rng.permutation(num_blocks)[:pages].astype(np.int32)
    ntok = pages * bs - 3                          # a ragged last page
    got = O.gather_paged(pool, num_blocks, H, bs, rb, table, ntok)
    assert np.array_equal(got, _brute_gather(pool, num_blocks, H, bs, rb, table, ntok))


@pytest.mark.parametrize("rb", [2, 144])
def test_gather_inverts_a_scatter_through_the_page_axes(rb):
    """Rows written into the pool through its [block][head][slot][row] axes
    (numpy fancy indexing) come back in logical order; untouched pool bytes
    never appear."""
    rng = np.random.default_rng(rb)
    num_blocks, H, bs = 9, 4, 16
    ntok = 7 * bs + 5
    table = rng.permutation(num_blocks)[:8].astype(np.int32)
    rows = rng.integers(0, 255, size=(ntok, H, rb), dtype=np.uint8)
    pool = np.full((num_blocks, H, bs, rb), 255, dtype=np.uint8)
    n = np.arange(ntok)
    pool[table[n // bs][:, None], np.arange(H)[None, :], (n % bs)[:, None]] = rows
    got = O.gather_paged(pool.reshape(-1), num_blocks, H, bs, rb, table, ntok)
    assert np.array_equal(got, rows)


def test_identity_table_is_the_transposed_pool():
    """With table[i] = i the gather is the pool with its head and slot axes
    swapped."""
    rng = np.random.default_rng(3)
    num_blocks, H, bs, rb = 4, 4, 16, 32
    pool = rng.integers(0, 256, size=(num_blocks, H, bs, rb), dtype=np.uint8)
    got = O.gather_paged(pool.reshape(-1), num_blocks, H, bs, rb,
                         np.arange(num_blocks, dtype=np.int32), num_blocks * bs)
    assert np.array_equal(got, pool.transpose(0, 2, 1, 3).reshape(num_blocks * bs, H, rb))


@pytest.mark.parametrize("bad", [6, -1, 1 << 30])
def test_table_entry_outside_the_pool_raises(bad):
    pool = np.zeros(6 * 4 * 16 * 2, dtype=np.uint8)
    table = np.array([0, bad, 2], dtype=np.int32)
    O.gather_paged(pool, 6, 4, 16, 2, table, 16)          # the bad page is not reached
    with pytest.raises(IndexError):
        O.gather_paged(pool, 6, 4, 16, 2, table, 17)
