"""Pins of the decode-cache oracle (oracle/cache.py) against what the pages and
the arithmetic fix: the Eq (11) chunk update equals the batch block mean of
[P2] Eq 6, equals a key-by-key Eq (11) stream, and touches only the blocks the
new tokens fall into; exact small-integer cases check the count bookkeeping
(a wrong r_old, a dropped old term or a divide by b instead of the count
fails them)."""
import numpy as np

from oracle import cache, routing


def test_append_update_exact_integers():
    # block of b = 4: two old keys (1, 3) -> mean 2; add (5, 7): mean of all four = 4
    c = cache.append_update(np.array([2.0]), 2, np.array([[5.0], [7.0]]))
    assert c[0] == 4.0
    # empty block (r_old = 0): the stale summary is ignored
    c = cache.append_update(np.array([123.0]), 0, np.array([[1.0], [2.0], [6.0]]))
    assert c[0] == 3.0
    # no new keys: unchanged
    c = cache.append_update(np.array([0.5, -1.0]), 3, np.zeros((0, 2)))
    assert np.array_equal(c, [0.5, -1.0])
    # a partial block divides by its count, not by b ([P2] Eq 11 r_j)
    c = cache.append_update(np.array([10.0]), 1, np.array([[20.0]]))
    assert c[0] == 15.0


def test_touched_blocks():
    assert list(cache.touched_blocks(0, 0, 64)) == []
    assert list(cache.touched_blocks(100, 1, 64)) == [1]
    assert list(cache.touched_blocks(127, 2, 64)) == [1, 2]
    assert list(cache.touched_blocks(128, 64, 64)) == [2]
    assert list(cache.touched_blocks(130, 200, 64)) == [2, 3, 4, 5]


def test_chunked_appends_equal_batch_mean_and_key_stream():
    rng = np.random.default_rng(11)
    b, d, cap = 8, 6, 64
    k_all = rng.standard_normal((cap, d))
    v_all = rng.standard_normal((cap, d))
    k = np.zeros((cap, d)); v = np.zeros((cap, d))
    c = np.zeros((cap // b, d))
    length = 0
    for n in [1, 1, 5, 8, 3, 13, 0, 7, 17]:           # crosses, starts and ends on block edges
        k, v, c = cache.append_kv(k, v, c, length, k_all[length:length + n], v_all[length:length + n], b)
        length += n
        assert np.array_equal(k[:length], k_all[:length]) and np.array_equal(v[:length], v_all[:length])
        assert not k[length:].any() and not v[length:].any()
        want = routing.block_summaries(k_all, length, b)
        got = c[:cache.blocks_after(length, b)]
        assert np.max(np.abs(got - want)) < 1e-13
    # the last, partial block against a key-by-key Eq 11 stream
    j = (length - 1) // b
    stream = routing.incremental_summary(k_all[j * b:length])
    assert np.max(np.abs(stream[-1] - c[j])) < 1e-13


def test_untouched_blocks_and_padding_unchanged():
    rng = np.random.default_rng(12)
    b, d, cap = 4, 3, 24
    k = rng.standard_normal((cap, d)); v = rng.standard_normal((cap, d))
    c = routing.block_summaries(k, 10, b)
    c_full = np.vstack([c, np.full((cap // b - c.shape[0], d), 7.0)])   # stale slots past the length
    k2, v2, c2 = cache.append_kv(k, v, c_full, 10, np.ones((3, d)), np.ones((3, d)), b)
    assert np.array_equal(c2[:2], c_full[:2])                 # blocks 0, 1 untouched
    assert np.array_equal(c2[4:], c_full[4:])                 # blocks past the new length untouched
    # block 2 had keys 8, 9 and gets 10, 11 (ones); block 3 starts fresh with key 12
    assert np.allclose(c2[2], (k[8] + k[9] + 2.0) / 4, atol=1e-14)
    assert np.array_equal(c2[3], np.ones(d))
    assert np.array_equal(k2[10:13], np.ones((3, d))) and np.array_equal(k2[13:], k[13:])


def test_max_append_equals_batch_max_of_the_grown_block():
    """Max-pooled summaries kept with the cache: appending chunks to a block
    gives the per-dimension maximum of all its valid keys, as a batch max over
    the grown cache does; a block with no valid key starts from the new keys."""
    rng = np.random.default_rng(21)
    b, d, cap = 8, 5, 40
    k = rng.standard_normal((cap, d))
    v = rng.standard_normal((cap, d))
    length = 11
    summ = np.full((cap // b, d), -7.0)             # stale values in untouched slots
    summ[:2] = routing.block_summaries(k, length, b, "max")
    for n_new in (1, 3, 7, 9):
        kn = rng.standard_normal((n_new, d))
        vn = rng.standard_normal((n_new, d))
        k, v, summ = cache.append_kv(k, v, summ, length, kn, vn, b, kpool="max")
        length += n_new
        nb = cache.blocks_after(length, b)
        assert np.array_equal(summ[:nb], cache.summaries_after(k, length, b, "max"))
