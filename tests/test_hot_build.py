"""Host build of the Engram-Nine hot-tier index (engram_hot_build).

The hot tier of "DeepSeek Engram series guide", experiment 3 "Engram-Nine"
(Figure 1: two-tier retrieval), indexes the hot n-grams of one order with a
minimal perfect hash plus a fingerprint.  These tests hold the library's
host build to the definition include/engram.h gives for it, written out
again here from that text:
  * every n-gram gets its own slot, the slots are exactly 0..n_hot-1, and
    each slot holds its n-gram (newest id first) and row r of key r;
  * the documented hash (SplitMix64 finaliser, bucket by multiply-shift,
    pilot displacement) sends every key to the slot that holds it;
  * the build is deterministic and rejects repeated n-grams and bad sizes.
They call host code only; the device lookup is checked against the oracle
in the GPU tests."""
import os

import numpy as np
import pytest

from hashed_gram_embedding_amd import engram as eg

pytestmark = pytest.mark.skipif(not os.path.exists(eg.LIB_PATH), reason="libengram.so not built")

M64 = (1 << 64) - 1


def mix(v):
    v &= M64
    v ^= v >> 30
    v = (v * 0xBF58476D1CE4E5B9) & M64
    v ^= v >> 27
    v = (v * 0x94D049BB133111EB) & M64
    return v ^ (v >> 31)


def rng_range(a, r):
    return (a * r) >> 64


def documented_slot(key_oldest_first, seed, pilots, n_hot):
    n = len(key_oldest_first)
    h = mix(seed ^ n)
    for x in reversed(key_oldest_first):      # x'_t first
        h = mix(h ^ int(x))
    m = max(1, (n_hot + 3) // 4) if n_hot > 4 else 1
    p = int(pilots[rng_range(h, m)])
    return rng_range(mix(h ^ mix(p + 1)), n_hot)


def random_keys(rng, n_hot, n, vocab):
    seen = set()
    out = []
    while len(out) < n_hot:
        k = tuple(int(v) for v in rng.integers(0, vocab, size=n))
        if k not in seen:
            seen.add(k)
            out.append(k)
    return np.array(out, dtype=np.int32).reshape(n_hot, n)


@pytest.mark.parametrize("n", [2, 3, 4])
@pytest.mark.parametrize("n_hot", [1, 2, 3, 4, 5, 17, 1000, 20000])
def test_build_is_a_bijection_matching_the_documented_hash(n, n_hot):
    rng = np.random.default_rng(1000 * n + n_hot)
    keys = random_keys(rng, n_hot, n, vocab=max(8, int(2 * n_hot ** (1 / n)) + 3))
    pilots, slots, seed = eg.hot_build(keys, seed=7)
    assert pilots.shape[0] == eg.lib().engram_hot_buckets(n_hot)
    assert 7 <= seed < 7 + 16
    rows = slots[:, 4]
    assert np.array_equal(np.sort(rows), np.arange(n_hot))
    # slot s holds key rows[s], newest id first, zero padded
    held = slots[:, :4]
    assert np.array_equal(held[:, :n], keys[rows][:, ::-1])
    assert np.all(held[:, n:] == 0) and np.all(slots[:, 5:] == 0)
    where = np.empty(n_hot, dtype=np.int64)
    where[rows] = np.arange(n_hot)
    check = range(n_hot) if n_hot <= 2000 else rng.choice(n_hot, 2000, replace=False)
    for r in check:
        assert documented_slot(list(keys[r]), seed, pilots, n_hot) == where[r]


def test_bucket_count():
    L = eg.lib()
    assert [L.engram_hot_buckets(v) for v in (-3, 0, 1, 4, 5, 8, 9, 400000)] == [0, 0, 1, 1, 2, 2, 3, 100000]


def test_build_is_deterministic_and_seed_dependent():
    keys = random_keys(np.random.default_rng(3), 5000, 3, 60)
    a = eg.hot_build(keys, seed=11)
    b = eg.hot_build(keys, seed=11)
    assert all(np.array_equal(x, y) for x, y in zip(a[:2], b[:2])) and a[2] == b[2]
    c = eg.hot_build(keys, seed=12345)
    assert not np.array_equal(a[1], c[1])


def test_build_rejects_repeated_ngrams_and_bad_arguments():
    keys = np.array([[1, 2], [3, 4], [1, 2]], dtype=np.int32)
    with pytest.raises(eg.EngramError) as ex:
        eg.hot_build(keys)
    assert ex.value.status == eg.EINVAL and "equal" in str(ex.value)
    # the same ids in another order are a different n-gram
    eg.hot_build(np.array([[1, 2], [2, 1]], dtype=np.int32))
    for bad in (np.zeros((3, 1), np.int32), np.zeros((3, 5), np.int32), np.array([[1, -2]], np.int32)):
        with pytest.raises(eg.EngramError) as ex:
            eg.hot_build(bad)
        assert ex.value.status == eg.EINVAL
    L = eg.lib()
    import ctypes
    used = ctypes.c_uint64(0)
    assert L.engram_hot_build(None, 3, 2, 0, None, None, ctypes.byref(used)) == eg.EINVAL
    k = np.array([[1, 2]], dtype=np.int32)
    assert L.engram_hot_build(k.ctypes.data, 0, 2, 0, None, None, ctypes.byref(used)) == eg.EINVAL


def test_full_size_build_of_four_hundred_thousand_ngrams():
    """The largest hot set of the study's configurations (400K n-grams)."""
    rng = np.random.default_rng(5)
    keys = np.unique(rng.integers(0, 98560, size=(420000, 2), dtype=np.int64), axis=0)[:400000]
    keys = keys[rng.permutation(keys.shape[0])].astype(np.int32)
    pilots, slots, seed = eg.hot_build(keys)
    assert np.array_equal(np.sort(slots[:, 4]), np.arange(400000))
    assert np.array_equal(slots[:, :2], keys[slots[:, 4]][:, ::-1])
